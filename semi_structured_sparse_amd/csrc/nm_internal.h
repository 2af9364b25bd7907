// Internal declarations shared by the translation units of libnmsparse.so.
// Not part of the public ABI (include/nm_sparse.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nm {

// Attributes of one HIP device, read once per device and cached.
struct DeviceInfo {
  int device = -1;
  int cu_count = 0;
  int max_lds_per_block = 0;  // bytes one workgroup may allocate
};

// Attributes of the current device; returns hipSuccess or the failing call's error.
hipError_t current_device_info(DeviceInfo* out);

// Records the raw HIP error for nm_last_hip_error() on this thread.
void set_last_hip_error(hipError_t e);

// Launches a kernel through hipLaunchKernel (which reports launch errors directly,
// without touching the thread's sticky last-error state). A kernel that needs more than
// the 64 KiB default of dynamic LDS gets its limit raised to the device maximum once
// per (kernel, device).
hipError_t launch(const void* kernel, dim3 grid, dim3 block, void** args, size_t lds,
                  hipStream_t stream, const DeviceInfo& dev);

// Kernel launchers (arguments already validated by the API layer).
hipError_t launch_pack(const uint16_t* W, uint16_t* values, uint32_t* masks, int64_t rows,
                       int64_t cols, int N, int M, hipStream_t stream, const DeviceInfo& dev);
hipError_t launch_unpack(const uint16_t* values, const uint32_t* masks, uint16_t* W, int64_t rows, int64_t cols,
                         int N, int M, hipStream_t stream, const DeviceInfo& dev);
hipError_t launch_spmv(const uint16_t* values, const uint32_t* masks, const uint16_t* x,
                       uint16_t* y, int64_t rows, int64_t cols, int N, int M, hipStream_t stream,
                       const DeviceInfo& dev);
hipError_t launch_gemv(const uint16_t* W, const uint16_t* x, uint16_t* y, int64_t rows,
                       int64_t cols, hipStream_t stream, const DeviceInfo& dev);

// Workgroup shape of one SpMV / GEMV launch: `rpb` rows per workgroup, split into
// `row_groups` groups of 8 rows, each with `cs` waves that split the columns; `grid`
// workgroups.
struct WorkgroupShape {
  int rpb = 8;
  int row_groups = 1;
  int cs = 8;
  int64_t grid = 0;
  int ci = 1;  // column ranges per wave (the narrow-layer kernel when > 1)
};

// Small-batch products (1 <= batch <= kSmallBatch): X [batch][cols], Y [batch][rows].
constexpr int64_t kSmallBatch = 8;
// From this many vectors on, nm_spmm (2:4) and nm_gemm_dense use the matrix-core kernels;
// below it, the small-batch kernel 8 vectors at a time (measured faster there on MI355X:
// the matrix-core kernels pay a fixed latency per 64-column step and have few workgroups
// when the token count is small).
constexpr int64_t kMatrixCoreMinBatch = 32;
hipError_t launch_spmm(const uint16_t* values, const uint32_t* masks, const uint16_t* X,
                       uint16_t* Y, int64_t rows, int64_t cols, int batch, int N, int M,
                       hipStream_t stream, const DeviceInfo& dev);
hipError_t launch_gemm(const uint16_t* W, const uint16_t* X, uint16_t* Y, int64_t rows,
                       int64_t cols, int batch, hipStream_t stream, const DeviceInfo& dev);

// Name of the small-batch kernel instantiation launch_spmm runs for a rows x cols layer,
// pattern N:2N and a batch of 1..8 vectors (static string; "" otherwise).
const char* spmm_variant(int64_t rows, int64_t cols, int N, int64_t batch, const DeviceInfo& dev);

// Name of the kernel configuration launch_spmv picks (static string) and its shape.
const char* spmv_variant(int64_t rows, int64_t cols, int N, int M, const DeviceInfo& dev);
WorkgroupShape spmv_shape(int64_t rows, int64_t cols, int N, const DeviceInfo& dev);
constexpr int kMaxSpmvGroup = 8;  // products per nm_spmv_group call
hipError_t launch_spmv_group(int count, const uint16_t* const* values, const uint32_t* const* masks,
                             const uint16_t* x, uint16_t* const* y, const int64_t* rows, int64_t cols, int N,
                             int M, hipStream_t stream, const DeviceInfo& dev);
WorkgroupShape spmv_quarter_shape(int64_t rows, int64_t cols, const DeviceInfo& dev);
WorkgroupShape dense_shape(int64_t rows, int64_t cols, const DeviceInfo& dev);

// Widest x the SpMV / GEMV kernels can stage for the given device.
int64_t max_cols_for(const DeviceInfo& dev);

// Prefill-sized products on the matrix cores: X [tokens][cols], Y [tokens][rows]. The
// sparse one takes the 50% patterns: 2:4 on the sparse instruction, 4:8 and 8:16 as two 2:4
// operands, 16:32 expanded to dense fragments. Limits: cols <= kPrefillMaxCols (byte offsets
// inside a workgroup's slices are 32-bit), tokens <= kPrefillMaxTokens.
constexpr int64_t kPrefillMaxCols = int64_t(1) << 21;
constexpr int64_t kPrefillMaxTokens = int64_t(1) << 24;
bool prefill_fits(int64_t rows, int64_t cols, int64_t tokens);
// 50% patterns with a matrix-core prefill product: all four.
bool prefill_pattern(int n, int m);
// With a workspace of at least prefill_workspace_bytes (0: the shape takes no column split)
// a grid too small for the CUs (mid-size batches), or a prompt of more than 128 tokens whose
// columns are better split over taller tiles, splits each output tile's columns over several
// workgroups; without one (or a smaller one) it runs the 64-row split if that fits, else
// unsplit. The counters must be zero before the launch, which leaves them zero (the same
// counter region as the skinny kernels' column splits, so one workspace serves both in
// stream order). n: the pattern's N (the split kernels and their costs depend on it).
size_t prefill_workspace_bytes(int64_t rows, int64_t cols, int64_t tokens, int n, const DeviceInfo& dev);
hipError_t launch_prefill_spmm(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                               int64_t rows, int64_t cols, int64_t tokens, int n, int m, hipStream_t stream,
                               const DeviceInfo& dev, void* workspace = nullptr, size_t workspace_bytes = 0);
// Bytes at the start of a workspace that hold the column splits' per-tile counters (fixed
// per device, so that every shape finds its counters where earlier launches left zeros).
size_t counter_bytes(const DeviceInfo& dev);
hipError_t launch_prefill_gemm(const uint16_t* W, const uint16_t* X, uint16_t* Y, int64_t rows, int64_t cols,
                               int64_t tokens, hipStream_t stream, const DeviceInfo& dev);
// Small-batch 50% product on the matrix instructions, 1..16 tokens (X [tokens][cols],
// Y [tokens][rows]): 2:4 directly, 4:8 and 8:16 split into two 2:4 operands on the sparse
// instruction, 16:32 expanded to dense fragments on the dense one. skinny_pattern tells
// whether a pattern has this product; skinny_fits whether a pattern and shape are within its
// limits.
bool skinny_pattern(int n, int m);
bool skinny_fits(int64_t rows, int64_t cols, int64_t tokens, int n, int m, const DeviceInfo& dev);
// With a workspace of at least skinny_workspace_bytes for a launch of `tokens` vectors (0:
// that launch takes no column split), layers of at most half as many 16-row tiles as CUs
// split their columns over several workgroups per tile where that measured faster; without
// one (or a smaller one) they run unsplit. The bytes do not grow with tokens: the size for
// the largest launch serves the smaller ones. The workspace's counters must be zero before
// the first launch; every launch leaves them zero.
size_t skinny_workspace_bytes(int64_t rows, int64_t cols, int tokens, int n, const DeviceInfo& dev);
hipError_t launch_skinny_spmm(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                              int64_t rows, int64_t cols, int tokens, int n, int m, hipStream_t stream,
                              const DeviceInfo& dev, void* workspace = nullptr, size_t workspace_bytes = 0);
// nm_spmm runs the skinny kernel, kSkinnyBatch vectors per launch, from kSkinnyMinBatch
// vectors up to kMatrixCoreMinBatch, where the prefill kernels take over: on layers of at
// least kSkinnyMinRows rows for 2:4, 4:8 and 8:16; on smaller layers (down to
// kSkinnySmallMinRows rows) for 2:4, and for the split 4:8 / 8:16 from 9 vectors (at most
// 5120 columns) or 12. Measured on MI355X over 256..1536 rows x 4096..8192 columns at 5..16
// vectors: there the skinny kernel's fixed cost (about 6 us) is below the small-batch
// kernel's time for 2:4 at every batch (1024 x 4096 at 8 vectors: 6.7 against 8.0 us), and
// for the split patterns once the small-batch kernel needs a second pass of 8 vectors.
// 16:32, whose expansion costs LDS traffic every step, only from kSkinnyExpandMinBatch
// vectors on layers of at least kSkinnyExpandMinRows rows and at most kSkinnyExpandMaxCols
// columns (X of 16 vectors in one LDS phase): measured there at 1.2-1.5x the small-batch
// kernel (4096 x 4096 at 16 vectors: 15.6 against 21.5 us), and behind it elsewhere (at 5..8
// vectors, on 1024-row layers, on 5120 columns and more).
constexpr int64_t kSkinnyMinBatch = 5;
constexpr int64_t kSkinnyMinRows = 2048;
constexpr int64_t kSkinnySmallMinRows = 256;
constexpr int64_t kSkinnyBatch = 16;
constexpr int64_t kSkinnyExpandMinBatch = 12;
constexpr int64_t kSkinnyExpandMinRows = 4096;
constexpr int64_t kSkinnyExpandMaxCols = 4096;
constexpr int64_t kSkinnyExpandFullChunk = 14;     // vectors of a nearly full 16-vector launch
// Batches of 32 .. kSkinnyBeforePrefillMaxBatch vectors stay on skinny launches on layers of
// at most kSkinnyBeforePrefillMaxRows rows (32 vectors up to twice that), see prefill_route.
constexpr int64_t kSkinnyBeforePrefillMaxBatch = 48;
// 16:32 takes the prefill kernels (expanded fragments) from this batch on: below it, its
// 16-vector launches are as fast (4096 x 4096 at 32 vectors: 28.8 us against about 51 for one
// launch of 64 x 64 tiles walking every column; at 64 vectors 55.7 against 51).
constexpr int64_t kExpandPrefillMinBatch = 64;
// With a workspace, 16:32 batches of kExpandColSplitMinBatch..kSkinnyBatch vectors on layers
// of at most kExpandColSplitMaxRows rows take the column-split expansion kernel instead of
// the small-batch or 16-vector expansion launch (1024 x 4096 at 16 vectors: 11.2 against
// 15.2 us; 2048 x 4096: 11.7 against 14.7; 4096 x 4096: 16.4 against 15.7, so not there).
constexpr int64_t kExpandColSplitMinBatch = 12;
constexpr int64_t kExpandColSplitMaxRows = 2048;
constexpr int64_t kSkinnyBeforePrefillMaxRows = 4096;
constexpr int64_t kSkinnyExpandFullMinRows = 2048;
bool use_skinny(int64_t rows, int64_t cols, int64_t batch, int n, int m, const DeviceInfo& dev);
// 16:32 is routed per launch of up to kSkinnyBatch vectors: a launch of `tokens` vectors
// takes the expansion kernel where that measured faster than the small-batch kernel (whose
// time grows with every 8 vectors while the expansion kernel's hardly does).
bool skinny_expand_chunk(int64_t rows, int64_t cols, int64_t tokens, const DeviceInfo& dev);
const char* skinny_variant(int n);

// nm_spmm's argument checks (host only, no HIP call): NM_OK or the status to return.
int spmm_check(const uint16_t* values, const uint32_t* masks, const uint16_t* X, const uint16_t* Y, int64_t rows,
               int64_t cols, int64_t batch, int N, int M);
// nm_spmm's dispatch; with a workspace of at least spmm_workspace_bytes (counters zero) the
// skinny kernels split the columns of short layers, and batches of more than kSkinnyBatch
// vectors take the column-split prefill kernel where colsplit_route says so.
int spmm_dispatch(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y, int64_t rows,
                  int64_t cols, int64_t batch, int N, int M, void* stream, void* workspace, size_t workspace_bytes);
size_t spmm_workspace_bytes(int64_t rows, int64_t cols, int64_t batch, int N, int M, const DeviceInfo& dev);

// Whether nm_spmm runs a batch on the prefill kernels (else on skinny or small-batch launches).
bool prefill_route(int64_t rows, int64_t cols, int64_t batch, int N, int M, const DeviceInfo& dev);
// The smallest batch nm_spmm runs on the prefill kernels for pattern N (32; 16:32: 64).
int64_t prefill_min_batch(int N);
// Whether nm_spmm_ws, given a workspace of prefill_workspace_bytes, runs a batch on the
// column-split prefill kernel: 50% batches of more than kSkinnyBatch vectors whose
// small-tile grid leaves CUs idle or that split better over taller tiles, and the 16:32
// batches above on small layers.
bool colsplit_route(int64_t rows, int64_t cols, int64_t batch, int N, int M, const DeviceInfo& dev);

// Name of the kernel configuration the prefill launchers pick (static string).
// (sparse: n = the pattern's N, 2, 4, 8 or 16)
const char* prefill_variant(int64_t rows, int64_t tokens, bool sparse, const DeviceInfo& dev, int n = 2);
// The column-split kernel launch_prefill_spmm runs with a workspace ("" if none).
const char* prefill_colsplit_variant(int64_t rows, int64_t cols, int64_t tokens, const DeviceInfo& dev, int n);

}  // namespace nm
