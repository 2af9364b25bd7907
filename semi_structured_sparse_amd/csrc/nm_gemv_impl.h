// Dense fp16 matrix-vector product y = W x on gfx950: the kernel template of the
// same-GPU baseline the sparse product is measured against (aimodeling.com
// SparseDecoding article, "The Kernel Is the Other Half of the Answer", quotes every
// speedup against the dense product).
//
// It is built and tuned the same way as the sparse kernel so that the ratio is fair:
// a workgroup covers a few rows with several waves splitting the columns; in one step the 8
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

// 8 lanes per row, each step one whole 128-byte line (64 columns) of every row of the
// wave's 8 rows (nontemporal with NT). The workgroup owns `rpb` consecutive rows in
// RG = ceil(rpb / 8) groups of 8, each with `cs_count` waves splitting the columns, as in
// the sparse kernel (same register budget, same prologue order: x chunks, then the first
// batch of W, then the LDS writes; same fixed-order reduction).
constexpr int kMaxWaves = spmv_detail::kMaxWaves;
constexpr int kRedUint4 = kMaxWaves * 8 * 4 / 16;  // reduction area, in uint4

template <int BATCH, bool NT>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(8))) void gemv_kernel(
    const uint4* __restrict__ W, const uint4* __restrict__ x, uint16_t* __restrict__ y, int rows, int cols,
    int rpb, int cs_count) {
  extern __shared__ uint4 lds[];
  float* red = reinterpret_cast<float*>(lds);
  uint4* xs = lds + kRedUint4;

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int CS = __builtin_amdgcn_readfirstlane(cs_count);
  const int rg = __builtin_amdgcn_readfirstlane(int(unsigned(wave) / unsigned(CS)));
  const int cs = wave - rg * CS;
  const int u = lane & 7;
  const int rsub = lane >> 3;
  const int row0 = blockIdx.x * rpb;
  const int row_end = min(row0 + rpb, rows);
  const unsigned r = unsigned(min(row0 + 8 * rg + rsub, row_end - 1));

  const int words2 = cols >> 5;                 // 32-column chunks (4 lanes' worth)
  const int steps = (words2 + 1) >> 1;          // 64 columns of every row per step
  const int full_steps = words2 >> 1;
  const int s_beg = int(unsigned(steps) * unsigned(cs) / unsigned(CS));
  const int s_end = int(unsigned(steps) * unsigned(cs + 1) / unsigned(CS));
  const int s_main = min(s_end, full_steps);
  const uint4* __restrict__ wrow = W + size_t(r) * unsigned(cols >> 3);
  const uint4* __restrict__ wp = wrow + 8 * unsigned(s_beg) + unsigned(u);
  const uint4* xp = xs + 8 * unsigned(s_beg) + unsigned(u);
  const int n = s_main - s_beg;
  const int nfull = n / BATCH;
  const int rem = n - nfull * BATCH;

  // prologue: x chunks, then the first batch of W (offsets clamped into the row, so the
  // loads are unconditional), then the LDS writes
  const int n16 = cols >> 3;
  const bool two_chunks = n16 > nthreads;
  const uint4 x0 = x[min(tid, n16 - 1)];
  uint4 x1 = make_uint4(0u, 0u, 0u, 0u);
  if (two_chunks) x1 = x[min(tid + nthreads, n16 - 1)];
  __builtin_amdgcn_sched_barrier(0);
  uint4 wv[BATCH];
  const unsigned wo = 8u * unsigned(s_beg) + unsigned(u), wlast = unsigned(cols >> 3) - 1u;
#pragma unroll
  for (int i = 0; i < BATCH; ++i) wv[i] = load16<NT>(wrow + min(wo + 8u * unsigned(i), wlast));
  if (tid < n16) xs[tid] = x0;
  if (two_chunks && tid + nthreads < n16) xs[tid + nthreads] = x1;
  for (int i = tid + 2 * nthreads; i < n16; i += nthreads) xs[i] = x[i];
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
    part[0] = dot8(load16<NT>(wrow + 8 * s + unsigned(u)), xs[8 * s + unsigned(u)], part[0]);
  }
  float acc = (part[0] + part[1]) + (part[2] + part[3]);

  acc = dpp_octet_sum(acc);
  if (u == 0) red[wave * 8 + rsub] = acc;
  __syncthreads();
  if (tid < row_end - row0) {
    const int trg = tid >> 3, trow = tid & 7;
    float t = 0.f;
    for (int k = 0; k < CS; ++k) t += red[(trg * CS + k) * 8 + trow];
    y[row0 + tid] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(t));
  }
}

constexpr size_t lds_bytes(int cols) { return size_t(kRedUint4) * 16 + size_t(cols) * 2; }

}  // namespace gemv_detail
}  // namespace nm
