// C ABI of libnmsparse.so: argument validation (no HIP call before it passes),
// status strings, the per-device attribute cache and the dispatch to the kernels.
#include <cstring>
#include <mutex>
#include <set>
#include <utility>

#include "nm_internal.h"
#include "nm_sparse.h"

namespace nm {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
DeviceInfo g_dev[kMaxDevices];
thread_local int t_last_hip_error = 0;
std::set<std::pair<const void*, int>> g_lds_raised;  // guarded by g_dev_mutex

// 50% (16 kept values per mask word) and 25% (8 per word) patterns.
bool valid_pattern(int N, int M) {
  return (N == 2 && M == 4) || (N == 4 && M == 8) || (N == 8 && M == 16) || (N == 16 && M == 32) ||
         (N == 1 && M == 4) || (N == 2 && M == 8) || (N == 4 && M == 16) || (N == 8 && M == 32);
}

// rows >= 1, cols >= 32, cols % 32 == 0, and every size the kernels form fits: int row
// indices up to rows + 64 (a workgroup's rows past the last one), int column indices, and
// rows*cols*2 bytes.
bool valid_shape(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 32 || (cols % 32) != 0) return false;
  if (rows > (int64_t(1) << 31) - 64 || cols > (int64_t(1) << 30)) return false;
  if (rows > (int64_t(1) << 62) / 2 / cols) return false;  // rows*cols*2 bytes must fit
  return true;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_fail(hipError_t e) {
  set_last_hip_error(e);
  return NM_ERR_HIP;
}

}  // namespace

void set_last_hip_error(hipError_t e) { t_last_hip_error = int(e); }

hipError_t current_device_info(DeviceInfo* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if (g_dev[dev].device != dev) {
    DeviceInfo info;
    info.device = dev;
    e = hipDeviceGetAttribute(&info.cu_count, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&info.max_lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    g_dev[dev] = info;
  }
  *out = g_dev[dev];
  return hipSuccess;
}

hipError_t launch(const void* kernel, dim3 grid, dim3 block, void** args, size_t lds,
                  hipStream_t stream, const DeviceInfo& dev) {
  if (lds > 64 * 1024) {
    if (lds > size_t(dev.max_lds_per_block)) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    const std::pair<const void*, int> key(kernel, dev.device);
    if (g_lds_raised.find(key) == g_lds_raised.end()) {
      hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         dev.max_lds_per_block);
      if (e != hipSuccess) return e;
      g_lds_raised.insert(key);
    }
  }
  return hipLaunchKernel(kernel, grid, block, args, lds, stream);
}

// The prefill kernels take the 50% patterns they cover from kMatrixCoreMinBatch vectors,
// except where 16-vector launches of the skinny kernels measured faster: the prefill kernels
// cost a fixed time per 64-column step on a grid of few workgroups, nearly the same from
// 32 to 128 vectors, while the skinny launches add up per 16. Measured on MI355X (2:4, µs at
// 32 / 48 / 64 vectors, skinny against prefill): 4096 x 4096 16.7 / 23.9 / 30.9 against
// 26.3; 4096 x 14336 44.6 / 65.0 / 84.8 against 82; 8192 x 8192 40.4 / 59.7 against 51;
// 14336 x 4096 32.7 against 27.9 already at 32. So: up to 48 vectors on layers of at most
// 4096 rows, up to 32 on layers of at most 8192, where the skinny kernels take the layer.
int64_t prefill_min_batch(int N) { return N == 16 ? kExpandPrefillMinBatch : kMatrixCoreMinBatch; }

bool prefill_route(int64_t rows, int64_t cols, int64_t batch, int N, int M, const DeviceInfo& dev) {
  if (!prefill_pattern(N, M) || batch < prefill_min_batch(N)) return false;
  const bool short_batch = (batch <= kSkinnyBeforePrefillMaxBatch && rows <= kSkinnyBeforePrefillMaxRows) ||
                           (batch <= kMatrixCoreMinBatch && rows <= 2 * kSkinnyBeforePrefillMaxRows);
  return !(short_batch && use_skinny(rows, cols, kSkinnyBatch, N, M, dev));
}

// From a sweep on MI355X at 17..256 vectors (µs, column split against the unsplit prefill
// kernel and against 16-vector skinny launches): 4096 x 4096 2:4 at 32 vectors 10.8 against
// 25.9 and 16.7; 1024 x 8192 at 64 12.3 against 48.7 and 46.3; 4096 x 14336 4:8 at 64 30.7
// against 97.2 and 106; 14336 x 4096 at 64 26.8 against 27.9. At 16 vectors and below one
// skinny launch is as fast or faster (4096 x 4096 2:4: 9.2 against 11.9).
bool colsplit_route(int64_t rows, int64_t cols, int64_t batch, int N, int M, const DeviceInfo& dev) {
  const bool size = batch > kSkinnyBatch || (N == 16 && batch >= kExpandColSplitMinBatch &&
                                             rows <= kExpandColSplitMaxRows);
  return size && prefill_pattern(N, M) && prefill_workspace_bytes(rows, cols, batch, N, dev) > 0;
}

// nm_spmm's argument checks, before any HIP call.
int spmm_check(const uint16_t* values, const uint32_t* masks, const uint16_t* X, const uint16_t* Y, int64_t rows,
               int64_t cols, int64_t batch, int N, int M) {
  if (!values || !masks || !X || !Y) return NM_ERR_NULL;
  if (!valid_shape(rows, cols) || batch < 1 || batch > kPrefillMaxTokens) return NM_ERR_SHAPE;
  if (!valid_pattern(N, M) || (batch > 1 && M != 2 * N)) return NM_ERR_PATTERN;
  if (!aligned(values, 16) || !aligned(masks, 4) || !aligned(X, 16) || !aligned(Y, 2)) return NM_ERR_ALIGN;
  // beyond 2^21 columns no skinny launch fits, so such batches go to the prefill kernels,
  // whose limit this is
  if (prefill_pattern(N, M) && batch >= prefill_min_batch(N) && cols > kPrefillMaxCols) return NM_ERR_SHAPE;
  return NM_OK;
}

// nm_spmm's dispatch, with an optional workspace for the skinny kernels' column splits.
int spmm_dispatch(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y, int64_t rows,
                  int64_t cols, int64_t batch, int N, int M, void* stream, void* workspace, size_t workspace_bytes) {
  const int st = spmm_check(values, masks, X, Y, rows, cols, batch, N, M);
  if (st != NM_OK) return st;
  if (!aligned(workspace, 16)) return NM_ERR_ALIGN;
  DeviceInfo dev;
  hipError_t e = current_device_info(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (workspace != nullptr && colsplit_route(rows, cols, batch, N, M, dev) &&
      workspace_bytes >= prefill_workspace_bytes(rows, cols, batch, N, dev)) {
    // column-split prefill product (launch_prefill_spmm takes the split with this workspace)
    e = launch_prefill_spmm(values, masks, X, Y, rows, cols, batch, N, M, static_cast<hipStream_t>(stream), dev,
                            workspace, workspace_bytes);
    return e == hipSuccess ? NM_OK : hip_fail(e);
  }
  if (prefill_route(rows, cols, batch, N, M, dev)) {  // matrix-core prefill product
    if (!prefill_fits(rows, cols, batch)) return NM_ERR_SHAPE;
    e = launch_prefill_spmm(values, masks, X, Y, rows, cols, batch, N, M, static_cast<hipStream_t>(stream), dev,
                            workspace, workspace_bytes);
    return e == hipSuccess ? NM_OK : hip_fail(e);
  }
  if (M != 2 * N && cols > max_cols_for(dev)) return NM_ERR_TOO_WIDE;  // 25%: single-vector kernel only
  if (N == 16 && M == 32 && batch >= kSkinnyMinBatch) {
    // 16:32 from 5 vectors up to the prefill route's batch: each launch of up to 16 vectors
    // on the expansion kernel where that measured faster, else on the small-batch kernel 8
    // vectors at a time
    for (int64_t b0 = 0; b0 < batch; b0 += kSkinnyBatch) {
      const int64_t nb = batch - b0 < kSkinnyBatch ? batch - b0 : kSkinnyBatch;
      if (skinny_expand_chunk(rows, cols, nb, dev)) {
        e = launch_skinny_spmm(values, masks, X + b0 * cols, Y + b0 * rows, rows, cols, int(nb), N, M,
                               static_cast<hipStream_t>(stream), dev);
        if (e != hipSuccess) return hip_fail(e);
        continue;
      }
      for (int64_t c0 = b0; c0 < b0 + nb; c0 += kSmallBatch) {
        const int nc = int(b0 + nb - c0 < kSmallBatch ? b0 + nb - c0 : kSmallBatch);
        e = launch_spmm(values, masks, X + c0 * cols, Y + c0 * rows, rows, cols, nc, N, M,
                        static_cast<hipStream_t>(stream), dev);
        if (e != hipSuccess) return hip_fail(e);
      }
    }
    return NM_OK;
  }
  if (use_skinny(rows, cols, batch < kSkinnyBatch ? batch : kSkinnyBatch, N, M, dev)) {
    // 50% patterns at 5..31 vectors where measured faster: the matrix instructions, 16
    // vectors per launch (launches in stream order, so one workspace serves them all); a
    // last launch too small for them (17..20 vectors leave 1..4) runs on the small-batch kernel
    for (int64_t b0 = 0; b0 < batch; b0 += kSkinnyBatch) {
      const int nb = int(batch - b0 < kSkinnyBatch ? batch - b0 : kSkinnyBatch);
      if (use_skinny(rows, cols, nb, N, M, dev)) {
        e = launch_skinny_spmm(values, masks, X + b0 * cols, Y + b0 * rows, rows, cols, nb, N, M,
                               static_cast<hipStream_t>(stream), dev, workspace, workspace_bytes);
      } else {
        e = launch_spmm(values, masks, X + b0 * cols, Y + b0 * rows, rows, cols, nb < kSmallBatch ? nb : int(kSmallBatch),
                        N, M, static_cast<hipStream_t>(stream), dev);
        if (e == hipSuccess && nb > kSmallBatch)
          e = launch_spmm(values, masks, X + (b0 + kSmallBatch) * cols, Y + (b0 + kSmallBatch) * rows, rows, cols,
                          int(nb - kSmallBatch), N, M, static_cast<hipStream_t>(stream), dev);
      }
      if (e != hipSuccess) return hip_fail(e);
    }
    return NM_OK;
  }
  // otherwise (fewer vectors, smaller layers, most 16:32 shapes): the small-batch kernel on consecutive
  // groups of kSmallBatch rows of X (X and Y rows are contiguous)
  for (int64_t b0 = 0; b0 < batch; b0 += kSmallBatch) {
    const int nb = int(batch - b0 < kSmallBatch ? batch - b0 : kSmallBatch);
    e = launch_spmm(values, masks, X + b0 * cols, Y + b0 * rows, rows, cols, nb, N, M,
                    static_cast<hipStream_t>(stream), dev);
    if (e != hipSuccess) return hip_fail(e);
  }
  return NM_OK;
}

// Workspace bytes spmm_dispatch can use for the product (0 when it would not use one).
size_t spmm_workspace_bytes(int64_t rows, int64_t cols, int64_t batch, int N, int M, const DeviceInfo& dev) {
  if (!valid_shape(rows, cols) || !valid_pattern(N, M) || batch < 1 || batch > kPrefillMaxTokens) return 0;
  if (colsplit_route(rows, cols, batch, N, M, dev)) return prefill_workspace_bytes(rows, cols, batch, N, dev);
  if (prefill_route(rows, cols, batch, N, M, dev)) return 0;
  if (!use_skinny(rows, cols, batch < kSkinnyBatch ? batch : kSkinnyBatch, N, M, dev)) return 0;
  return skinny_workspace_bytes(rows, cols, int(batch < kSkinnyBatch ? batch : kSkinnyBatch), N, dev);
}
}  // namespace nm

extern "C" {

size_t nm_values_count(int64_t rows, int64_t cols, int N, int M) {
  if (!nm::valid_shape(rows, cols) || !nm::valid_pattern(N, M)) return 0;
  return size_t(rows) * size_t(cols) / size_t(M) * size_t(N);
}

size_t nm_masks_count(int64_t rows, int64_t cols) {
  if (!nm::valid_shape(rows, cols)) return 0;
  return size_t(rows) * size_t(cols / 32);
}

int64_t nm_max_cols(void) {
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) {
    nm::set_last_hip_error(e);
    return 0;
  }
  return nm::max_cols_for(dev);
}

int nm_pack(const uint16_t* W, uint16_t* values, uint32_t* masks, int64_t rows, int64_t cols,
            int N, int M, void* stream) {
  if (!W || !values || !masks) return NM_ERR_NULL;
  if (!nm::valid_shape(rows, cols)) return NM_ERR_SHAPE;
  if (!nm::valid_pattern(N, M)) return NM_ERR_PATTERN;
  if (!nm::aligned(W, 16) || !nm::aligned(values, 16) || !nm::aligned(masks, 4)) return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  e = nm::launch_pack(W, values, masks, rows, cols, N, M, static_cast<hipStream_t>(stream), dev);
  return e == hipSuccess ? NM_OK : nm::hip_fail(e);
}

int nm_unpack(const uint16_t* values, const uint32_t* masks, uint16_t* W, int64_t rows, int64_t cols, int N, int M,
              void* stream) {
  if (!values || !masks || !W) return NM_ERR_NULL;
  if (!nm::valid_shape(rows, cols)) return NM_ERR_SHAPE;
  if (!nm::valid_pattern(N, M)) return NM_ERR_PATTERN;
  if (!nm::aligned(W, 16) || !nm::aligned(values, 16) || !nm::aligned(masks, 4)) return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  e = nm::launch_unpack(values, masks, W, rows, cols, N, M, static_cast<hipStream_t>(stream), dev);
  return e == hipSuccess ? NM_OK : nm::hip_fail(e);
}

int nm_spmv(const uint16_t* values, const uint32_t* masks, const uint16_t* x, uint16_t* y,
            int64_t rows, int64_t cols, int N, int M, void* stream) {
  if (!values || !masks || !x || !y) return NM_ERR_NULL;
  if (!nm::valid_shape(rows, cols)) return NM_ERR_SHAPE;
  if (!nm::valid_pattern(N, M)) return NM_ERR_PATTERN;
  if (!nm::aligned(values, 16) || !nm::aligned(masks, 4) || !nm::aligned(x, 16) || !nm::aligned(y, 2))
    return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  if (cols > nm::max_cols_for(dev)) return NM_ERR_TOO_WIDE;
  e = nm::launch_spmv(values, masks, x, y, rows, cols, N, M, static_cast<hipStream_t>(stream), dev);
  return e == hipSuccess ? NM_OK : nm::hip_fail(e);
}

int nm_spmv_group(int count, const uint16_t* const* values, const uint32_t* const* masks, const uint16_t* x,
                  uint16_t* const* y, const int64_t* rows, int64_t cols, int N, int M, void* stream) {
  if (!values || !masks || !x || !y || !rows) return NM_ERR_NULL;
  if (count < 1 || count > nm::kMaxSpmvGroup) return NM_ERR_SHAPE;
  for (int k = 0; k < count; ++k)
    if (!values[k] || !masks[k] || !y[k]) return NM_ERR_NULL;
  for (int k = 0; k < count; ++k)
    if (!nm::valid_shape(rows[k], cols)) return NM_ERR_SHAPE;
  if (!nm::valid_pattern(N, M)) return NM_ERR_PATTERN;
  if (!nm::aligned(x, 16)) return NM_ERR_ALIGN;
  for (int k = 0; k < count; ++k)
    if (!nm::aligned(values[k], 16) || !nm::aligned(masks[k], 4) || !nm::aligned(y[k], 2)) return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  if (cols > nm::max_cols_for(dev)) return NM_ERR_TOO_WIDE;
  e = nm::launch_spmv_group(count, values, masks, x, y, rows, cols, N, M, static_cast<hipStream_t>(stream), dev);
  return e == hipSuccess ? NM_OK : nm::hip_fail(e);
}

int nm_gemv_dense(const uint16_t* W, const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols,
                  void* stream) {
  if (!W || !x || !y) return NM_ERR_NULL;
  if (!nm::valid_shape(rows, cols)) return NM_ERR_SHAPE;
  if (!nm::aligned(W, 16) || !nm::aligned(x, 16) || !nm::aligned(y, 2)) return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  if (cols > nm::max_cols_for(dev)) return NM_ERR_TOO_WIDE;
  e = nm::launch_gemv(W, x, y, rows, cols, static_cast<hipStream_t>(stream), dev);
  return e == hipSuccess ? NM_OK : nm::hip_fail(e);
}

int nm_spmm_prefill(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y, int64_t rows,
                    int64_t cols, int64_t tokens, int N, int M, void* stream) {
  if (!values || !masks || !X || !Y) return NM_ERR_NULL;
  if (!nm::valid_shape(rows, cols) || tokens < 1 || !nm::prefill_fits(rows, cols, tokens)) return NM_ERR_SHAPE;
  if (!nm::prefill_pattern(N, M)) return NM_ERR_PATTERN;
  if (!nm::aligned(values, 16) || !nm::aligned(masks, 4) || !nm::aligned(X, 16) || !nm::aligned(Y, 2))
    return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  e = nm::launch_prefill_spmm(values, masks, X, Y, rows, cols, tokens, N, M, static_cast<hipStream_t>(stream), dev);
  return e == hipSuccess ? NM_OK : nm::hip_fail(e);
}

int nm_gemm_dense_prefill(const uint16_t* W, const uint16_t* X, uint16_t* Y, int64_t rows, int64_t cols,
                          int64_t tokens, void* stream) {
  if (!W || !X || !Y) return NM_ERR_NULL;
  if (!nm::valid_shape(rows, cols) || tokens < 1 || !nm::prefill_fits(rows, cols, tokens)) return NM_ERR_SHAPE;
  if (!nm::aligned(W, 16) || !nm::aligned(X, 16) || !nm::aligned(Y, 2)) return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  e = nm::launch_prefill_gemm(W, X, Y, rows, cols, tokens, static_cast<hipStream_t>(stream), dev);
  return e == hipSuccess ? NM_OK : nm::hip_fail(e);
}


int nm_spmm(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
            int64_t rows, int64_t cols, int64_t batch, int N, int M, void* stream) {
  return nm::spmm_dispatch(values, masks, X, Y, rows, cols, batch, N, M, stream, nullptr, 0);
}

int nm_spmm_ws(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y, int64_t rows,
               int64_t cols, int64_t batch, int N, int M, void* workspace, size_t workspace_bytes, void* stream) {
  return nm::spmm_dispatch(values, masks, X, Y, rows, cols, batch, N, M, stream, workspace, workspace_bytes);
}

size_t nm_spmm_workspace_bytes(int64_t rows, int64_t cols, int64_t batch, int N, int M) {
  if (!nm::valid_shape(rows, cols) || !nm::valid_pattern(N, M) || batch < 1) return 0;
  nm::DeviceInfo dev;
  if (nm::current_device_info(&dev) != hipSuccess) return 0;
  return nm::spmm_workspace_bytes(rows, cols, batch, N, M, dev);
}

int nm_spmm_skinny(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                   int64_t rows, int64_t cols, int64_t batch, int N, int M, void* stream) {
  if (!values || !masks || !X || !Y) return NM_ERR_NULL;
  if (!nm::valid_shape(rows, cols) || batch < 1 || batch > nm::kPrefillMaxTokens || cols > nm::kPrefillMaxCols)
    return NM_ERR_SHAPE;
  if (!nm::skinny_pattern(N, M)) return NM_ERR_PATTERN;
  if (!nm::aligned(values, 16) || !nm::aligned(masks, 4) || !nm::aligned(X, 16) || !nm::aligned(Y, 2))
    return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  const int64_t first = batch < nm::kSkinnyBatch ? batch : nm::kSkinnyBatch;
  if (!nm::skinny_fits(rows, cols, first, N, M, dev)) return NM_ERR_SHAPE;
  for (int64_t b0 = 0; b0 < batch; b0 += nm::kSkinnyBatch) {
    const int nb = int(batch - b0 < nm::kSkinnyBatch ? batch - b0 : nm::kSkinnyBatch);
    e = nm::launch_skinny_spmm(values, masks, X + b0 * cols, Y + b0 * rows, rows, cols, nb, N, M,
                               static_cast<hipStream_t>(stream), dev);
    if (e != hipSuccess) return nm::hip_fail(e);
  }
  return NM_OK;
}

int nm_gemm_dense(const uint16_t* W, const uint16_t* X, uint16_t* Y, int64_t rows, int64_t cols,
                  int64_t batch, void* stream) {
  if (!W || !X || !Y) return NM_ERR_NULL;
  if (!nm::valid_shape(rows, cols) || batch < 1 || batch > nm::kPrefillMaxTokens) return NM_ERR_SHAPE;
  if (batch >= nm::kMatrixCoreMinBatch) return nm_gemm_dense_prefill(W, X, Y, rows, cols, batch, stream);
  if (!nm::aligned(W, 16) || !nm::aligned(X, 16) || !nm::aligned(Y, 2)) return NM_ERR_ALIGN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  for (int64_t b0 = 0; b0 < batch; b0 += nm::kSmallBatch) {
    const int nb = int(batch - b0 < nm::kSmallBatch ? batch - b0 : nm::kSmallBatch);
    e = nm::launch_gemm(W, X + b0 * cols, Y + b0 * rows, rows, cols, nb, static_cast<hipStream_t>(stream), dev);
    if (e != hipSuccess) return nm::hip_fail(e);
  }
  return NM_OK;
}

const char* nm_spmm_variant(int64_t rows, int64_t cols, int64_t batch, int N, int M) {
  if (!nm::valid_shape(rows, cols) || !nm::valid_pattern(N, M) || batch < 1 || batch > nm::kPrefillMaxTokens) return "";
  if (batch > 1 && M != 2 * N) return "";
  nm::DeviceInfo dev;
  if (nm::current_device_info(&dev) != hipSuccess) return "";
  if (batch == 1 && cols <= nm::max_cols_for(dev)) return nm::spmv_variant(rows, cols, N, M, dev);
  if (nm::prefill_route(rows, cols, batch, N, M, dev))
    return nm::prefill_fits(rows, cols, batch) ? nm::prefill_variant(rows, batch, true, dev, N) : "";
  if (N == 16 && batch >= nm::kSkinnyMinBatch &&
      nm::skinny_expand_chunk(rows, cols, batch < nm::kSkinnyBatch ? batch : nm::kSkinnyBatch, dev))
    return nm::skinny_variant(N);
  if (nm::use_skinny(rows, cols, batch < nm::kSkinnyBatch ? batch : nm::kSkinnyBatch, N, M, dev))
    return nm::skinny_variant(N);
  return nm::spmm_variant(rows, cols, N, batch < nm::kSmallBatch ? batch : nm::kSmallBatch, dev);
}

const char* nm_spmm_ws_variant(int64_t rows, int64_t cols, int64_t batch, int N, int M) {
  const char* v = nm_spmm_variant(rows, cols, batch, N, M);
  if (*v == '\0') return v;
  nm::DeviceInfo dev;
  if (nm::current_device_info(&dev) != hipSuccess) return "";
  if (nm::colsplit_route(rows, cols, batch, N, M, dev)) return nm::prefill_colsplit_variant(rows, cols, batch, dev, N);
  const int nb = int(batch < nm::kSkinnyBatch ? batch : nm::kSkinnyBatch);
  if (N != 16 && std::strcmp(v, nm::skinny_variant(N)) == 0 && nm::skinny_workspace_bytes(rows, cols, nb, N, dev) > 0)
    return N == 2 ? "skinny_colsplit_kernel<false>" : "skinny_colsplit_kernel<true>";
  return v;
}

const char* nm_prefill_variant(int64_t rows, int64_t cols, int64_t tokens, int sparse) {
  if (!nm::valid_shape(rows, cols) || tokens < 1 || !nm::prefill_fits(rows, cols, tokens)) return "";
  nm::DeviceInfo dev;
  if (nm::current_device_info(&dev) != hipSuccess) return "";
  return nm::prefill_variant(rows, tokens, sparse != 0, dev, sparse == 3 ? 16 : sparse == 2 ? 4 : 2);
}

const char* nm_spmv_variant(int64_t rows, int64_t cols, int N, int M) {
  if (!nm::valid_shape(rows, cols) || !nm::valid_pattern(N, M)) return "";
  nm::DeviceInfo dev;
  if (nm::current_device_info(&dev) != hipSuccess) return "";
  return nm::spmv_variant(rows, cols, N, M, dev);
}

int nm_spmv_launch_shape(int64_t rows, int64_t cols, int N, int M, int64_t* shape) {
  if (!shape) return NM_ERR_NULL;
  if (!nm::valid_shape(rows, cols)) return NM_ERR_SHAPE;
  if (!nm::valid_pattern(N, M)) return NM_ERR_PATTERN;
  nm::DeviceInfo dev;
  hipError_t e = nm::current_device_info(&dev);
  if (e != hipSuccess) return nm::hip_fail(e);
  if (cols > nm::max_cols_for(dev)) return NM_ERR_TOO_WIDE;
  const nm::WorkgroupShape s = M == 4 * N ? nm::spmv_quarter_shape(rows, cols, dev) : nm::spmv_shape(rows, cols, N, dev);
  shape[0] = s.rpb;
  shape[1] = s.row_groups;
  shape[2] = s.cs;
  shape[3] = s.grid;
  return NM_OK;
}

const char* nm_status_string(int status) {
  switch (status) {
    case NM_OK: return "ok";
    case NM_ERR_NULL: return "a required pointer is NULL";
    case NM_ERR_SHAPE: return "invalid shape: need rows >= 1, cols >= 32, cols % 32 == 0, batch/tokens >= 1 (and sizes that fit)";
    case NM_ERR_PATTERN: return "unsupported N:M pattern: need 2:4, 4:8, 8:16, 16:32 or (one vector only) 1:4, 2:8, 4:16, 8:32";
    case NM_ERR_ALIGN: return "misaligned pointer: W, values and x need 16 bytes, masks 4, y 2";
    case NM_ERR_TOO_WIDE: return "cols too large: x does not fit in the LDS of one workgroup";
    case NM_ERR_HIP: return "a HIP runtime call failed";
    case NM_ERR_SCRATCH: return "the column split of this shape needs more than the library's static scratch";
    default: return "unknown status";
  }
}

int nm_last_hip_error(void) { return nm::t_last_hip_error; }

}  // extern "C"
