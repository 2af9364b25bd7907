// nm_gemv_dense launcher; the kernels and their description are in nm_gemv_impl.h.
#include "nm_gemv_impl.h"

namespace nm {
namespace {

constexpr int kRG = 1;       // one row group of 8 rows per workgroup
constexpr int kCS = 8;       // 8 waves splitting the columns
constexpr int kBatch = 4;
constexpr bool kNT = true;   // W streams once, a whole 128-byte line per instruction

}  // namespace

hipError_t launch_gemv(const uint16_t* W, const uint16_t* x, uint16_t* y, int64_t rows,
                       int64_t cols, hipStream_t stream, const DeviceInfo& dev) {
  const uint4* w4 = reinterpret_cast<const uint4*>(W);
  const uint4* x4 = reinterpret_cast<const uint4*>(x);
  int r = int(rows), c = int(cols);
  void* args[] = {&w4, &x4, &y, &r, &c};
  const dim3 grid((r + 8 * kRG - 1) / (8 * kRG));
  const size_t lds = size_t(c) * 2 + spmv_detail::line_reduction_bytes(kRG * kCS);
  return launch(reinterpret_cast<const void*>(&gemv_detail::gemv_line_kernel<kRG, kCS, kBatch, kNT>), grid,
                dim3(64 * kRG * kCS), args, lds, stream, dev);
}

}  // namespace nm
