// Dense fp16 matrix-vector product y = W x on gfx950: the kernel template of the
// same-GPU baseline the sparse product is measured against (aimodeling.com
// SparseDecoding article, "The Kernel Is the Other Half of the Answer", quotes every
// speedup against the dense product).
//
// It is built and tuned the same way as the sparse kernel so that the ratio is fair:
// a workgroup covers 8*RG rows with CS waves splitting the columns; in one step the 8
// lanes of a row each load 16 bytes of the row's next 128-byte line (64 columns), so a
// wave instruction consumes 8 whole lines and W can be streamed with nontemporal loads
// (NT), BATCH steps in flight; x is staged once in LDS and read back as 16-byte vectors;
// fp16 pairs are multiplied and summed in fp32 by v_dot2_f32_f16; rows are reduced with
// DPP across the row's 8 lanes and in LDS across waves, in a fixed order, and rounded
// once to fp16.
#pragma once

#include "nm_spmv_impl.h"

namespace nm {
namespace gemv_detail {

using spmv_detail::dpp_quad_sum;
using spmv_detail::half2_t;
using spmv_detail::load16;

__device__ __forceinline__ float dot8(uint4 w, uint4 xv, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.x), __builtin_bit_cast(half2_t, xv.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.y), __builtin_bit_cast(half2_t, xv.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.z), __builtin_bit_cast(half2_t, xv.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.w), __builtin_bit_cast(half2_t, xv.w), acc, false);
  return acc;
}

// Sum over 8 consecutive lanes: DPP quad sums, then row_half_mirror (lane i of each
// 8-lane group reads lane 7 - i, i.e. the other quad).
__device__ __forceinline__ float dpp_octet_sum(float v) {
  v = dpp_quad_sum(v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  return v;
}

// Full-line variant: 8 lanes per row, each step one whole 128-byte line (64 columns) of
// every row of the wave's 8 rows (nontemporal with NT); RG row groups x CS column
// splits per workgroup, as in the sparse full-line kernel.
template <int RG, int CS, int BATCH, bool NT>
__global__ __launch_bounds__(64 * RG * CS) void gemv_line_kernel(const uint4* __restrict__ W,
                                                                 const uint4* __restrict__ x,
                                                                 uint16_t* __restrict__ y, int rows, int cols) {
  constexpr int WAVES = RG * CS;
  constexpr int ROWS = 8 * RG;
  extern __shared__ uint4 lds[];
  float* red = reinterpret_cast<float*>(lds + (cols >> 3));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave / CS;
  const int cs = wave - rg * CS;
  const int u = lane & 7;
  const int row0 = blockIdx.x * ROWS;
  const unsigned r = unsigned(min(row0 + 8 * rg + (lane >> 3), rows - 1));

  const int words2 = cols >> 5;                 // 32-column chunks (4 lanes' worth)
  const int steps = (words2 + 1) >> 1;          // 64 columns of every row per step
  const int full_steps = words2 >> 1;
  const int s_beg = int((int64_t(steps) * cs) / CS);
  const int s_end = int((int64_t(steps) * (cs + 1)) / CS);
  const int s_main = min(s_end, full_steps);
  const uint4* __restrict__ wrow = W + size_t(r) * unsigned(cols >> 3);
  const uint4* __restrict__ wp = wrow + 8 * unsigned(s_beg) + unsigned(u);
  const uint4* xp = lds + 8 * unsigned(s_beg) + unsigned(u);
  const int n = s_main - s_beg;
  const int nfull = n / BATCH;
  const int rem = n - nfull * BATCH;

  uint4 wv[BATCH];
  if (nfull > 0) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i) wv[i] = load16<NT>(wp + 8 * i);
  }
  const int n16 = cols >> 3;
  for (int i = tid; i < n16; i += 64 * WAVES) lds[i] = x[i];
  __syncthreads();

  float part[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < nfull; ++b) {
    if (b > 0) {
#pragma unroll
      for (int i = 0; i < BATCH; ++i) wv[i] = load16<NT>(wp + 8 * i);
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) part[i & 3] = dot8(wv[i], xp[8 * i], part[i & 3]);
    wp += 8 * BATCH;
    xp += 8 * BATCH;
  }
  if (rem > 0) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i)
      if (i < rem) wv[i] = load16<NT>(wp + 8 * i);
#pragma unroll
    for (int i = 0; i < BATCH; ++i)
      if (i < rem) part[i & 3] = dot8(wv[i], xp[8 * i], part[i & 3]);
  }
  // cols % 64 == 32: the last step has 32 columns, held by lanes 0..3 of each row
  if (s_end > full_steps && u < 4) {
    const unsigned s = unsigned(full_steps);
    part[0] = dot8(load16<NT>(wrow + 8 * s + unsigned(u)), lds[8 * s + unsigned(u)], part[0]);
  }
  float acc = (part[0] + part[1]) + (part[2] + part[3]);

  acc = dpp_octet_sum(acc);
  if (u == 0) red[wave * 8 + (lane >> 3)] = acc;
  __syncthreads();
  if (tid < ROWS) {
    const int trg = tid >> 3, trow = tid & 7;
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < CS; ++k) t += red[(trg * CS + k) * 8 + trow];
    const int rr = row0 + tid;
    if (rr < rows) y[rr] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(t));
  }
}

}  // namespace gemv_detail
}  // namespace nm
