// nm_spmm / nm_gemm_dense launchers: decoder, interleave, phase width and workgroup
// shape for a batch of 1..8 activation vectors. The kernels are in nm_spmm_impl.h.
#include <algorithm>
#include <string>
#include <vector>

#include "nm_spmm_impl.h"

namespace nm {
namespace {

using namespace spmm_detail;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroup shape of the batch product, from a sweep on MI355X (batches 2, 4, 8; 2:4 and
// 16:32; 1024..28672 rows, 4096..14336 columns): every workgroup stages all B activation
// vectors (2*B*cols bytes from L2), so the product wants few, tall workgroups, about one
// per CU: up to 56 rows (7 groups of 8) and 16 / groups waves per group, 2..8 (48 rows
// when a workgroup may hold at most 12 waves). For 14336x4096 at B = 8 that is 22.5 us
// against 38.5 us with the single-vector rule's 8-row workgroups.
//
// Narrow layers (at most 4 rows per workgroup): the lanes of the 8 row slots of a wave would
// repeat rows, so the narrow kernel gives each row's slots CI = 2 (3..4 rows) or 4 (1..2
// rows) parts of the wave's columns instead (ci), when every part still holds a whole batch
// of 4 steps (1024 x 8192 and 1024 x 14336: 5-12% faster at 2..8 vectors; with fewer steps
// per part, 1024 x 4096, it was 2-9% slower, so those keep CI = 1).
WorkgroupShape spmm_shape_for(int64_t rows, int64_t cols, int maxw, const DeviceInfo& dev) {
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int64_t max_rpb = 8 * (maxw / 2);  // row groups of at least 2 waves
  WorkgroupShape s;
  const int64_t passes = ceil_div(rows, cus * max_rpb);
  s.rpb = int(std::max<int64_t>(1, ceil_div(rows, cus * passes)));
  s.row_groups = int(ceil_div(s.rpb, 8));
  s.cs = std::max(2, std::min(8, maxw / s.row_groups));
  if (s.row_groups * s.cs > maxw) s.cs = maxw / s.row_groups;
  s.grid = ceil_div(rows, s.rpb);
  const int64_t wave_steps = ceil_div(cols, 128) / s.cs;   // steps per wave (at least)
  for (int ci : {4, 2}) {
    if (s.rpb <= 8 / ci && wave_steps >= int64_t(4) * ci) {
      s.ci = ci;
      break;
    }
  }
  return s;
}

template <int N, int B>
WorkgroupShape spmm_shape(int64_t rows, int64_t cols, const DeviceInfo& dev) {
  return spmm_shape_for(rows, cols, max_waves<N, B>(), dev);
}

template <int N, int B, int DEC>
const void* spmm_kernel_for(int ci) {
  switch (ci) {
    case 2: return reinterpret_cast<const void*>(&spmm_narrow_kernel<N, B, DEC, 2>);
    case 4: return reinterpret_cast<const void*>(&spmm_narrow_kernel<N, B, DEC, 4>);
    default: return reinterpret_cast<const void*>(&spmm_kernel<N, B, DEC>);
  }
}

template <int N, int B, int DEC>
hipError_t launch_sparse(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                         int rows, int cols, hipStream_t stream, const DeviceInfo& dev) {
  // widest phase that fits, no wider than the row (rounded up to a whole step)
  const int cap = max_phase_cols<B, DEC>(size_t(dev.max_lds_per_block));
  if (cap < 128) return hipErrorInvalidValue;
  const int phase = int(std::min<int64_t>(cap, ceil_div(cols, 128) * 128));
  const WorkgroupShape s = spmm_shape<N, B>(rows, cols, dev);
  const uint4* v4 = reinterpret_cast<const uint4*>(values);
  int rpb = s.rpb, cs = s.cs;
  void* args[] = {&v4, &masks, &X, &Y, &rows, &cols, &rpb, &cs, const_cast<int*>(&phase)};
  return launch(spmm_kernel_for<N, B, DEC>(s.ci), dim3(unsigned(s.grid)), dim3(unsigned(64 * s.row_groups * s.cs)),
                args, lds_bytes<B, DEC>(phase), stream, dev);
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

// Workgroup shape of the dense batch product (B >= 2), from its own sweep over the same
// shapes and batches: balanced over the CUs, up to 16 rows per workgroup for B <= 4 and up
// to 40 for larger batches (staging B vectors per workgroup weighs more), with 16 waves
// (16 / groups per row group, at most 16 for the narrowest); narrow layers (at most 8 rows
// per CU) a few rows. The single-vector dense rule (8 rows, 8 waves) is up to 1.6x slower
// here (8192 x 8192 at B = 8: 44.1 us against 28.5 us), which would flatter the sparse
// product.
WorkgroupShape gemm_shape(int64_t rows, int batch, const DeviceInfo& dev) {
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int64_t max_rpb = batch <= 4 ? 16 : 40;
  WorkgroupShape s;
  if (rows <= 8 * cus) {
    s.rpb = int(std::min<int64_t>(8, ceil_div(rows, cus)));
  } else {
    s.rpb = int(ceil_div(rows, cus * ceil_div(rows, max_rpb * cus)));
  }
  s.row_groups = int(ceil_div(s.rpb, 8));
  s.cs = std::max(2, kMaxWaves / s.row_groups);
  s.grid = ceil_div(rows, s.rpb);
  return s;
}

template <int B>
hipError_t launch_dense_b(const uint16_t* W, const uint16_t* X, uint16_t* Y, int rows, int cols,
                          hipStream_t stream, const DeviceInfo& dev) {
  const size_t cap_bytes = size_t(dev.max_lds_per_block);
  if (cap_bytes <= dense_lds_bytes(B, 0)) return hipErrorInvalidValue;
  const int cap = int((cap_bytes - dense_lds_bytes(B, 0)) / (2 * B) / 64 * 64);
  if (cap < 64) return hipErrorInvalidValue;
  const int phase = int(std::min<int64_t>(cap, ceil_div(cols, 64) * 64));
  const WorkgroupShape s = B == 1 ? dense_shape(rows, cols, dev) : gemm_shape(rows, B, dev);
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

const char* spmm_variant(int64_t rows, int64_t cols, int N, int64_t batch, const DeviceInfo& dev) {
  const int n = N == 2 ? 0 : N == 4 ? 1 : N == 8 ? 2 : N == 16 ? 3 : -1;
  if (n < 0 || batch < 1 || batch > 8) return "";
  // the instantiations launch_sparse_b picks: byte table for N = 2, 4, 8, bit walk for 16
  const int b = int(batch);
  const int ci = spmm_shape_for(rows, cols, max_waves_of(N, b), dev).ci;
  if (ci > 1) {
    // spmm_narrow_kernel<N, B, DEC, CI> as profilers print it
    static const std::vector<std::string> narrow = [] {
      std::vector<std::string> v;
      for (int nn : {2, 4, 8, 16})
        for (int bb = 1; bb <= 8; ++bb)
          for (int cc : {2, 4})
            v.push_back("spmm_narrow_kernel<" + std::to_string(nn) + ", " + std::to_string(bb) + ", " +
                        std::to_string(nn == 16 ? int(kBitWalk) : int(kByteLut)) + ", " + std::to_string(cc) + ">");
      return v;
    }();
    return narrow[size_t((n * 8 + (b - 1)) * 2 + (ci == 4 ? 1 : 0))].c_str();
  }
  static const char* const kNames[4][8] = {
      {"spmm_kernel<2, 1, 2>", "spmm_kernel<2, 2, 2>", "spmm_kernel<2, 3, 2>", "spmm_kernel<2, 4, 2>", "spmm_kernel<2, 5, 2>", "spmm_kernel<2, 6, 2>", "spmm_kernel<2, 7, 2>", "spmm_kernel<2, 8, 2>"},
      {"spmm_kernel<4, 1, 2>", "spmm_kernel<4, 2, 2>", "spmm_kernel<4, 3, 2>", "spmm_kernel<4, 4, 2>", "spmm_kernel<4, 5, 2>", "spmm_kernel<4, 6, 2>", "spmm_kernel<4, 7, 2>", "spmm_kernel<4, 8, 2>"},
      {"spmm_kernel<8, 1, 2>", "spmm_kernel<8, 2, 2>", "spmm_kernel<8, 3, 2>", "spmm_kernel<8, 4, 2>", "spmm_kernel<8, 5, 2>", "spmm_kernel<8, 6, 2>", "spmm_kernel<8, 7, 2>", "spmm_kernel<8, 8, 2>"},
      {"spmm_kernel<16, 1, 0>", "spmm_kernel<16, 2, 0>", "spmm_kernel<16, 3, 0>", "spmm_kernel<16, 4, 0>", "spmm_kernel<16, 5, 0>", "spmm_kernel<16, 6, 0>", "spmm_kernel<16, 7, 0>", "spmm_kernel<16, 8, 0>"}};
  return kNames[n][batch - 1];
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
