// nm_spmm_noalloc: nm_spmm_ws for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation). The column
// split's workspace (the tiles' counters and partial tiles) is a static device array of the
// library instead of caller memory; every GPU the library runs on holds its own copy of the
// array until the process ends.
#include <mutex>

#include "nm_internal.h"
#include "nm_sparse.h"

namespace nm {
namespace {

constexpr size_t kScratchBytes = NM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

// In host code `scratch` names a host-side stand-in, not the device array: kernels and
// fills take the address hipGetSymbolAddress gives per device (g_scratch) instead.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxScratchDevices];   // device address of `scratch` per device, guarded by the mutex

__global__ void zero_scratch_kernel(uint4* p, uint32_t n) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The array's address on device `dev` (the current device). On the first call there it is
// looked up, and the whole array is cleared by a fill kernel queued on `stream` ahead of the
// call's own kernels (the split kernels need their counters at zero, and leave them zero).
hipError_t scratch_on(int dev, hipStream_t stream, void** out) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    const uint32_t n = uint32_t(kScratchBytes / 16);
    hipLaunchKernelGGL(zero_scratch_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint4*>(p), n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace nm

int nm_spmm_noalloc(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                    int64_t rows, int64_t cols, int64_t batch, int N, int M, void* stream) {
  const int st = nm::spmm_check(values, masks, X, Y, rows, cols, batch, N, M);
  if (st != NM_OK) return st;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) {
    nm::set_last_hip_error(e);
    return NM_ERR_HIP;
  }
  if (nm::spmm_workspace_bytes(rows, cols, batch, N, M, dev) > nm::kScratchBytes) return NM_ERR_SCRATCH;
  void* ws = nullptr;
  e = nm::scratch_on(dev.device, static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess) {
    nm::set_last_hip_error(e);
    return NM_ERR_HIP;
  }
  return nm::spmm_dispatch(values, masks, X, Y, rows, cols, batch, N, M, stream, ws, nm::kScratchBytes);
}
