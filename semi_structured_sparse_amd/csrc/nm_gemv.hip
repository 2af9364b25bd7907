// nm_gemv_dense launcher; the kernel and its description are in nm_gemv_impl.h. The
// workgroup shape follows the same rule as the sparse product, applied to the dense
// row length (64 columns = 128 bytes of W per step).
#include "nm_gemv_impl.h"

namespace nm {
namespace {

constexpr int kBatch = 4;
constexpr bool kNT = true;   // W streams once, a whole 128-byte line per instruction

}  // namespace

hipError_t launch_gemv(const uint16_t* W, const uint16_t* x, uint16_t* y, int64_t rows,
                       int64_t cols, hipStream_t stream, const DeviceInfo& dev) {
  const WorkgroupShape s = workgroup_shape(rows, (cols + 63) / 64, dev);
  const uint4* w4 = reinterpret_cast<const uint4*>(W);
  const uint4* x4 = reinterpret_cast<const uint4*>(x);
  int r = int(rows), c = int(cols), rpb = s.rpb, cs = s.cs;
  void* args[] = {&w4, &x4, &y, &r, &c, &rpb, &cs};
  return launch(reinterpret_cast<const void*>(&gemv_detail::gemv_kernel<kBatch, kNT>), dim3(unsigned(s.grid)),
                dim3(unsigned(64 * s.row_groups * s.cs)), args, gemv_detail::lds_bytes(c), stream, dev);
}

}  // namespace nm
