// nm_gemv_dense launcher; the kernel and its description are in nm_gemv_impl.h.
#include <algorithm>

#include "nm_gemv_impl.h"

namespace nm {
namespace {

constexpr int kBatch = 4;
constexpr bool kNT = true;   // W streams once, a whole 128-byte line per instruction

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroup shape of the dense product, from its own sweep on MI355X over the same
// projection shapes as the sparse rule (rows per workgroup 1..56, 2..16 waves per row
// group); within 1.1% of the best shape per layer on average, 3.6% at worst. A step is
// 64 columns (128 bytes of W per row).
//   * narrow layers (at most 8 rows per CU): a few rows per workgroup, about 8 steps per
//     wave;
//   * otherwise: about 8 rows per workgroup (balanced over the CUs) and 8..16 waves per
//     row, about 16 steps each. Unlike the sparse kernel, the dense one gains nothing from
//     taller workgroups on long rows: it streams twice the bytes per row for the same x.
WorkgroupShape gemv_shape(int64_t rows, int64_t cols, const DeviceInfo& dev) {
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int64_t steps = ceil_div(cols, 64);
  WorkgroupShape s;
  if (rows <= 8 * cus) {
    s.rpb = int(std::min<int64_t>(8, ceil_div(rows, cus)));
    s.cs = int(std::min<int64_t>(16, ceil_div(steps, 8)));
  } else {
    s.rpb = int(ceil_div(rows, cus * ceil_div(rows, 8 * cus)));
    s.cs = int(std::min<int64_t>(16, std::max<int64_t>(8, ceil_div(steps, 16))));
  }
  s.row_groups = int(ceil_div(s.rpb, 8));
  s.grid = ceil_div(rows, s.rpb);
  return s;
}

}  // namespace

WorkgroupShape dense_shape(int64_t rows, int64_t cols, const DeviceInfo& dev) { return gemv_shape(rows, cols, dev); }

hipError_t launch_gemv(const uint16_t* W, const uint16_t* x, uint16_t* y, int64_t rows,
                       int64_t cols, hipStream_t stream, const DeviceInfo& dev) {
  const WorkgroupShape s = gemv_shape(rows, cols, dev);
  const uint4* w4 = reinterpret_cast<const uint4*>(W);
  const uint4* x4 = reinterpret_cast<const uint4*>(x);
  int r = int(rows), c = int(cols), rpb = s.rpb, cs = s.cs;
  void* args[] = {&w4, &x4, &y, &r, &c, &rpb, &cs};
  return launch(reinterpret_cast<const void*>(&gemv_detail::gemv_kernel<kBatch, kNT>), dim3(unsigned(s.grid)),
                dim3(unsigned(64 * s.row_groups * s.cs)), args, gemv_detail::lds_bytes(c), stream, dev);
}

}  // namespace nm
