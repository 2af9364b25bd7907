// Measurement probes: a pure streaming read (the attainable read bandwidth of the
// GPU) and a plain copy (known traffic, to calibrate the memory counters).
//
// The read probe is the fastest shape a sweep over grid sizes, block sizes, loads in
// flight and cache policy found on MI355X: one 512-thread workgroup per CU, a grid-stride
// loop with 4 dwordx4 loads in flight per lane, nontemporal loads.
#include "nm_internal.h"
#include "nm_probe.h"
#include "nm_spmv_impl.h"
#include "nm_sparse.h"

namespace nm {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void nm_probe_read_kernel(const uint4* __restrict__ src,
                                                                      int64_t n16,
                                                                      uint32_t* __restrict__ sink,
                                                                      uint32_t magic) {
  const int64_t stride = int64_t(gridDim.x) * kProbeThreads;
  int64_t i = int64_t(blockIdx.x) * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 a[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) a[k] = spmv_detail::load16<true>(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= a[k].x ^ a[k].y ^ a[k].z ^ a[k].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = spmv_detail::load16<true>(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == magic) sink[0] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void nm_probe_copy_kernel(uint4* __restrict__ dst,
                                                                      const uint4* __restrict__ src,
                                                                      int64_t n16) {
  const int64_t stride = int64_t(gridDim.x) * kProbeThreads;
  int64_t i = int64_t(blockIdx.x) * kProbeThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 a[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) a[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) dst[i + k * stride] = a[k];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

unsigned probe_blocks(const DeviceInfo& dev, int64_t n16) {
  int64_t blocks = int64_t(dev.cu_count > 0 ? dev.cu_count : 256);
  const int64_t need = (n16 + kProbeThreads - 1) / kProbeThreads;
  if (blocks > need) blocks = need;
  return unsigned(blocks < 1 ? 1 : blocks);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace nm

extern "C" {

int nm_probe_read(const void* src, size_t bytes, uint32_t* sink, uint32_t magic, void* stream) {
  if (!src || !sink) return NM_ERR_NULL;
  if (bytes == 0 || (bytes % 16) != 0 || bytes > (size_t(1) << 50)) return NM_ERR_SHAPE;
  if (!nm::aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e == hipSuccess) {
    const uint4* s4 = static_cast<const uint4*>(src);
    int64_t n16 = int64_t(bytes / 16);
    void* args[] = {&s4, &n16, &sink, &magic};
    e = nm::launch(reinterpret_cast<const void*>(&nm::nm_probe_read_kernel),
                   dim3(nm::probe_blocks(dev, n16)), dim3(nm::kProbeThreads), args, 0,
                   static_cast<hipStream_t>(stream), dev);
  }
  if (e != hipSuccess) {
    nm::set_last_hip_error(e);
    return NM_ERR_HIP;
  }
  return NM_OK;
}

int nm_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!src || !dst) return NM_ERR_NULL;
  if (bytes == 0 || (bytes % 16) != 0 || bytes > (size_t(1) << 50)) return NM_ERR_SHAPE;
  if (!nm::aligned16(src) || !nm::aligned16(dst)) return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e == hipSuccess) {
    uint4* d4 = static_cast<uint4*>(dst);
    const uint4* s4 = static_cast<const uint4*>(src);
    int64_t n16 = int64_t(bytes / 16);
    void* args[] = {&d4, &s4, &n16};
    e = nm::launch(reinterpret_cast<const void*>(&nm::nm_probe_copy_kernel),
                   dim3(nm::probe_blocks(dev, n16)), dim3(nm::kProbeThreads), args, 0,
                   static_cast<hipStream_t>(stream), dev);
  }
  if (e != hipSuccess) {
    nm::set_last_hip_error(e);
    return NM_ERR_HIP;
  }
  return NM_OK;
}

}  // extern "C"
