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

// The same pure read with its launch shape given by the caller: `blocks` workgroups of
// `threads` lanes, UNROLL dwordx4 loads in flight per lane. BLOCKED = false: one grid-stride
// sweep over the whole buffer (at any moment the grid reads one contiguous window);
// BLOCKED = true: workgroup b reads its own contiguous slice of ceil(n16 / blocks) uint4s,
// the way a product whose workgroups own consecutive rows streams its weights.
template <int UNROLL, bool BLOCKED>
__global__ __launch_bounds__(1024) void nm_probe_read_shaped_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                    uint32_t* __restrict__ sink, uint32_t magic) {
  const int64_t nt = blockDim.x;
  int64_t lo = 0, hi = n16, i, stride;
  if constexpr (BLOCKED) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    lo = int64_t(blockIdx.x) * per;
    hi = lo + per < n16 ? lo + per : n16;
    i = lo + threadIdx.x;
    stride = nt;
  } else {
    i = int64_t(blockIdx.x) * nt + threadIdx.x;
    stride = int64_t(gridDim.x) * nt;
  }
  uint32_t acc = 0;
  for (; i + (UNROLL - 1) * stride < hi; i += UNROLL * stride) {
    uint4 a[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) a[k] = spmv_detail::load16<true>(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) acc ^= a[k].x ^ a[k].y ^ a[k].z ^ a[k].w;
  }
  for (; i < hi; i += stride) {
    const uint4 a = spmv_detail::load16<true>(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  (void)lo;
  if (acc == magic) sink[0] = acc;
}

template <bool BLOCKED>
const void* shaped_kernel(int unroll) {
  switch (unroll) {
    case 1: return reinterpret_cast<const void*>(&nm_probe_read_shaped_kernel<1, BLOCKED>);
    case 2: return reinterpret_cast<const void*>(&nm_probe_read_shaped_kernel<2, BLOCKED>);
    case 4: return reinterpret_cast<const void*>(&nm_probe_read_shaped_kernel<4, BLOCKED>);
    default: return reinterpret_cast<const void*>(&nm_probe_read_shaped_kernel<8, BLOCKED>);
  }
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

int nm_probe_read_shaped(const void* src, size_t bytes, uint32_t* sink, uint32_t magic, int blocks, int threads,
                         int unroll, int blocked, void* stream) {
  if (!src || !sink) return NM_ERR_NULL;
  if (bytes == 0 || (bytes % 16) != 0 || bytes > (size_t(1) << 50)) return NM_ERR_SHAPE;
  if (blocks < 1 || blocks > (1 << 20) || threads < 64 || threads > 1024 || threads % 64 != 0) return NM_ERR_SHAPE;
  if (!(unroll == 1 || unroll == 2 || unroll == 4 || unroll == 8) || !(blocked == 0 || blocked == 1))
    return NM_ERR_SHAPE;
  if (!nm::aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e == hipSuccess) {
    const uint4* s4 = static_cast<const uint4*>(src);
    int64_t n16 = int64_t(bytes / 16);
    void* args[] = {&s4, &n16, &sink, &magic};
    const void* fn = blocked ? nm::shaped_kernel<true>(unroll) : nm::shaped_kernel<false>(unroll);
    e = nm::launch(fn, dim3(unsigned(blocks)), dim3(unsigned(threads)), args, 0, static_cast<hipStream_t>(stream),
                   dev);
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
