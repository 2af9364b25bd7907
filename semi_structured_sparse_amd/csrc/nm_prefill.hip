// Launchers of the prefill-sized products (many tokens per weight) on the matrix cores:
// the 50% sparse products (2:4 directly, 4:8 and 8:16 split into two 2:4 operands) and the
// dense product. The kernels are in nm_prefill_impl.h.
#include "nm_internal.h"
#include "nm_prefill_impl.h"

namespace nm {

using namespace prefill_detail;

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile shapes (TR x TT output tiles of 16 x 16 per wave, KS columns per step, loads D steps
// ahead), from sweeps on MI355X over 4096..14336 rows and columns at 2048 tokens. Large
// tiles: the sparse product 256 rows x 128 tokens per workgroup (each X fragment serves 4
// row tiles), the dense one 128 x 256 (each weight fragment serves 16 token tiles); each was
// the fastest for its kernel. The sparse product takes 256 x 256 when that grid still has
// a workgroup per CU (14336 x 4096 x 2048: 247 against 294 us; with fewer workgroups it
// loses: 4096 x 4096 x 2048: 102 against 71 us). The small tile (64 x 64) serves problems
// whose large-tile grid would leave CUs idle.
using SparseHuge = Tile<4, 16, 64>;   // 256 rows x 256 tokens: when even this grid fills the CUs
using SparseLarge = Tile<4, 8, 64>;
using DenseLarge = Tile<2, 16, 64>;
using Small = Tile<1, 4, 64>;
constexpr int kDepth = 2;

template <typename T>
int64_t workgroups(int64_t rows, int64_t tokens) {
  return ceil_div(rows, T::kRows) * ceil_div(tokens, T::kTokens);
}

template <typename T>
bool use_large(int64_t rows, int64_t tokens, const DeviceInfo& dev) {
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  return workgroups<T>(rows, tokens) >= cus;
}

}  // namespace

bool prefill_fits(int64_t rows, int64_t cols, int64_t tokens) {
  // byte offsets inside one workgroup's slices are 32-bit; workgroup counts fit an int
  return cols <= kPrefillMaxCols && tokens <= kPrefillMaxTokens && workgroups<Small>(rows, tokens) <= INT32_MAX;
}

bool prefill_pattern(int n, int m) { return 2 * n == m && (n == 2 || n == 4 || n == 8); }

hipError_t launch_prefill_spmm(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                               int64_t rows, int64_t cols, int64_t tokens, int n, int m, hipStream_t stream,
                               const DeviceInfo& dev) {
  if (!prefill_fits(rows, cols, tokens) || !prefill_pattern(n, m)) return hipErrorInvalidValue;
  int r = int(rows), c = int(cols), t = int(tokens);
  void* args[] = {&values, &masks, &X, &Y, &r, &c, &t};
  const bool split = n != 2;
  if (use_large<SparseHuge>(rows, tokens, dev))
    return launch(split ? reinterpret_cast<const void*>(&prefill_split_kernel<4, 16, 64, kDepth>)
                        : reinterpret_cast<const void*>(&prefill_spmm_kernel<4, 16, 64, kDepth>),
                  dim3(unsigned(workgroups<SparseHuge>(rows, tokens))), dim3(kThreads), args, 0, stream, dev);
  if (use_large<SparseLarge>(rows, tokens, dev))
    return launch(split ? reinterpret_cast<const void*>(&prefill_split_kernel<4, 8, 64, kDepth>)
                        : reinterpret_cast<const void*>(&prefill_spmm_kernel<4, 8, 64, kDepth>),
                  dim3(unsigned(workgroups<SparseLarge>(rows, tokens))), dim3(kThreads), args, 0, stream, dev);
  return launch(split ? reinterpret_cast<const void*>(&prefill_split_kernel<1, 4, 64, kDepth>)
                      : reinterpret_cast<const void*>(&prefill_spmm_kernel<1, 4, 64, kDepth>),
                dim3(unsigned(workgroups<Small>(rows, tokens))), dim3(kThreads), args, 0, stream, dev);
}

hipError_t launch_prefill_gemm(const uint16_t* W, const uint16_t* X, uint16_t* Y, int64_t rows, int64_t cols,
                               int64_t tokens, hipStream_t stream, const DeviceInfo& dev) {
  if (!prefill_fits(rows, cols, tokens)) return hipErrorInvalidValue;
  int r = int(rows), c = int(cols), t = int(tokens);
  void* args[] = {&W, &X, &Y, &r, &c, &t};
  if (use_large<DenseLarge>(rows, tokens, dev))
    return launch(reinterpret_cast<const void*>(&prefill_gemm_kernel<2, 16, 64, kDepth>),
                  dim3(unsigned(workgroups<DenseLarge>(rows, tokens))), dim3(kThreads), args, 0, stream, dev);
  return launch(reinterpret_cast<const void*>(&prefill_gemm_kernel<1, 4, 64, kDepth>),
                dim3(unsigned(workgroups<Small>(rows, tokens))), dim3(kThreads), args, 0, stream, dev);
}

const char* prefill_variant(int64_t rows, int64_t tokens, bool sparse, const DeviceInfo& dev, bool split) {
  if (sparse && split)
    return use_large<SparseHuge>(rows, tokens, dev)    ? "prefill_split_kernel<4, 16, 64, 2>"
           : use_large<SparseLarge>(rows, tokens, dev) ? "prefill_split_kernel<4, 8, 64, 2>"
                                                       : "prefill_split_kernel<1, 4, 64, 2>";
  if (sparse)
    return use_large<SparseHuge>(rows, tokens, dev)    ? "prefill_spmm_kernel<4, 16, 64, 2>"
           : use_large<SparseLarge>(rows, tokens, dev) ? "prefill_spmm_kernel<4, 8, 64, 2>"
                                                       : "prefill_spmm_kernel<1, 4, 64, 2>";
  return use_large<DenseLarge>(rows, tokens, dev) ? "prefill_gemm_kernel<2, 16, 64, 2>"
                                                  : "prefill_gemm_kernel<1, 4, 64, 2>";
}

}  // namespace nm
