// nm_spmm / nm_gemm_dense launchers: decoder, interleave, phase width and workgroup
// shape for a batch of 1..8 activation vectors. The kernels are in nm_spmm_impl.h.
#include <algorithm>

#include "nm_spmm_impl.h"

namespace nm {
namespace {

using namespace spmm_detail;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int N, int B, int DEC>
hipError_t launch_sparse(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                         int rows, int cols, hipStream_t stream, const DeviceInfo& dev) {
  // widest phase that fits, no wider than the row (rounded up to a whole step)
  const int cap = max_phase_cols<B, DEC>(size_t(dev.max_lds_per_block));
  if (cap < 128) return hipErrorInvalidValue;
  const int phase = int(std::min<int64_t>(cap, ceil_div(cols, 128) * 128));
  WorkgroupShape s = spmv_shape(rows, cols, dev);
  if (s.row_groups * s.cs > max_waves<N, B>()) s.cs = std::max(1, max_waves<N, B>() / s.row_groups);
  const uint4* v4 = reinterpret_cast<const uint4*>(values);
  int rpb = s.rpb, cs = s.cs;
  void* args[] = {&v4, &masks, &X, &Y, &rows, &cols, &rpb, &cs, const_cast<int*>(&phase)};
  return launch(reinterpret_cast<const void*>(&spmm_kernel<N, B, DEC>), dim3(unsigned(s.grid)),
                dim3(unsigned(64 * s.row_groups * s.cs)), args, lds_bytes<B, DEC>(phase), stream, dev);
}

template <int B>
hipError_t launch_sparse_b(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                           int rows, int cols, int N, hipStream_t stream, const DeviceInfo& dev) {
  switch (N) {
    case 2: return launch_sparse<2, B, kByteLut>(values, masks, X, Y, rows, cols, stream, dev);
    case 4: return launch_sparse<4, B, kByteLut>(values, masks, X, Y, rows, cols, stream, dev);
    case 8: return launch_sparse<8, B, kByteLut>(values, masks, X, Y, rows, cols, stream, dev);
    case 16: return launch_sparse<16, B, kBitWalk>(values, masks, X, Y, rows, cols, stream, dev);
    default: return hipErrorInvalidValue;
  }
}

template <int B>
hipError_t launch_dense_b(const uint16_t* W, const uint16_t* X, uint16_t* Y, int rows, int cols,
                          hipStream_t stream, const DeviceInfo& dev) {
  const size_t cap_bytes = size_t(dev.max_lds_per_block);
  if (cap_bytes <= dense_lds_bytes(B, 0)) return hipErrorInvalidValue;
  const int cap = int((cap_bytes - dense_lds_bytes(B, 0)) / (2 * B) / 64 * 64);
  if (cap < 64) return hipErrorInvalidValue;
  const int phase = int(std::min<int64_t>(cap, ceil_div(cols, 64) * 64));
  const WorkgroupShape s = dense_shape(rows, cols, dev);
  const uint4* w4 = reinterpret_cast<const uint4*>(W);
  int rpb = s.rpb, cs = s.cs;
  void* args[] = {&w4, &X, &Y, &rows, &cols, &rpb, &cs, const_cast<int*>(&phase)};
  return launch(reinterpret_cast<const void*>(&gemm_kernel<B>), dim3(unsigned(s.grid)),
                dim3(unsigned(64 * s.row_groups * s.cs)), args, dense_lds_bytes(B, phase), stream, dev);
}

}  // namespace

hipError_t launch_spmm(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                       int64_t rows, int64_t cols, int batch, int N, int M, hipStream_t stream,
                       const DeviceInfo& dev) {
  // one vector: the single-vector kernel (x staged whole) whenever x fits
  if (batch == 1 && cols <= max_cols_for(dev)) return launch_spmv(values, masks, X, Y, rows, cols, N, M, stream, dev);
  const int r = int(rows), c = int(cols);
  switch (batch) {
    case 1: return launch_sparse_b<1>(values, masks, X, Y, r, c, N, stream, dev);
    case 2: return launch_sparse_b<2>(values, masks, X, Y, r, c, N, stream, dev);
    case 3: return launch_sparse_b<3>(values, masks, X, Y, r, c, N, stream, dev);
    case 4: return launch_sparse_b<4>(values, masks, X, Y, r, c, N, stream, dev);
    case 5: return launch_sparse_b<5>(values, masks, X, Y, r, c, N, stream, dev);
    case 6: return launch_sparse_b<6>(values, masks, X, Y, r, c, N, stream, dev);
    case 7: return launch_sparse_b<7>(values, masks, X, Y, r, c, N, stream, dev);
    case 8: return launch_sparse_b<8>(values, masks, X, Y, r, c, N, stream, dev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(const uint16_t* W, const uint16_t* X, uint16_t* Y, int64_t rows, int64_t cols,
                       int batch, hipStream_t stream, const DeviceInfo& dev) {
  if (batch == 1 && cols <= max_cols_for(dev)) return launch_gemv(W, X, Y, rows, cols, stream, dev);
  const int r = int(rows), c = int(cols);
  switch (batch) {
    case 1: return launch_dense_b<1>(W, X, Y, r, c, stream, dev);
    case 2: return launch_dense_b<2>(W, X, Y, r, c, stream, dev);
    case 3: return launch_dense_b<3>(W, X, Y, r, c, stream, dev);
    case 4: return launch_dense_b<4>(W, X, Y, r, c, stream, dev);
    case 5: return launch_dense_b<5>(W, X, Y, r, c, stream, dev);
    case 6: return launch_dense_b<6>(W, X, Y, r, c, stream, dev);
    case 7: return launch_dense_b<7>(W, X, Y, r, c, stream, dev);
    case 8: return launch_dense_b<8>(W, X, Y, r, c, stream, dev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nm
