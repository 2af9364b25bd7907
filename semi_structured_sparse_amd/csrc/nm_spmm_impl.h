// Small-batch N:M sparse matrix product Y = X W'^T on gfx950: the kernel template, and
// the dense counterpart it is measured against.
//
// Method (pages: news.bitwarelabs.com "SparseDecoding: decoding-aware pruning for
// accurate and fast LLM generation", "What's new", which separates batch-one decoding
// (sparse matrix-vector products) from prefill and larger batches (sparse matrix-matrix
// products); aimodeling.com SparseDecoding article, "The Kernel Is the Other Half of the
// Answer", for the bitmask format): for a batch of B <= 8 activation vectors the packed
// weights are still read once, so the product stays bound by HBM bandwidth while the
// useful work grows B-fold. The format and its decoding are those of the single-vector
// kernel; only x changes.
//
// Work mapping: as spmv_kernel (8 lanes per row, each step one whole 128-byte line of
// packed values = 4 mask words = 128 columns of the row, nontemporal loads, RG groups of
// 8 rows x CS waves splitting the columns). X ([B][cols], one activation vector per row)
// is staged in LDS interleaved by column: the SB >= B halves of column c (B activations,
// zero padding) are adjacent, so one ds_read_b32/b64/b128 returns all B activations a
// kept weight meets, and one v_fma_mix_f32 (fp16 x fp16 product, exact in fp32, fp32
// accumulator) per activation does the rest.
//
// When 2 * SB * cols bytes exceed the LDS budget the columns are processed in phases of
// `phase_cols` columns: stage that part of X, let every wave take its share of the
// phase's steps, and move on; the partial sums stay in registers across phases. Each
// phase loads its x chunks, then its first batch of values, then writes LDS, as the
// single-vector prologue does.
//
// Decoders: the byte LUT (2:4 and 4:8 have exactly 4 kept columns per mask byte, 8:16 a
// variable count concatenated by a 64-bit shift), with offsets pre-scaled by the
// interleave stride; for 16:32 the bit walk (the high-half lane walks the bit-reversed
// word from the window's end, with its values reversed by v_perm).
#pragma once

#include "nm_gemv_impl.h"
#include "nm_spmv_impl.h"

namespace nm {
namespace spmm_detail {

using gemv_detail::dot8;

using spmv_detail::dpp_quad_sum;
using spmv_detail::half2_t;
using spmv_detail::kByteLut;
using spmv_detail::kBitWalk;
using spmv_detail::kMaxWaves;
using spmv_detail::kPad;
using spmv_detail::lds_address;
using spmv_detail::load16;
using spmv_detail::reverse_half_word;
using spmv_detail::row8_sum;

constexpr int kMaxBatch = 8;

// halves per column in LDS for a batch of B: the next power of two
template <int B>
constexpr int stride_of() {
  return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8;
}

constexpr size_t kLutBytes = 2 * 256 * 8;
constexpr size_t kRedBytes = size_t(kMaxWaves) * 8 * kMaxBatch * sizeof(float);  // 4 KiB
constexpr int kXOffset = int(kRedBytes) + kPad;

// LDS bytes of one launch: reduction area, padded x buffer, then the byte-LUT tables.
template <int B, int DEC>
constexpr size_t lds_bytes(int phase_cols) {
  return size_t(kXOffset) + size_t(phase_cols) * 2 * stride_of<B>() + kPad +
         (DEC == kByteLut ? kLutBytes : 0);
}

// Widest phase (a multiple of 128 columns) that fits `lds_cap` bytes.
template <int B, int DEC>
constexpr int max_phase_cols(size_t lds_cap) {
  const size_t fixed = lds_bytes<B, DEC>(0);
  return lds_cap <= fixed ? 0 : int((lds_cap - fixed) / (2 * stride_of<B>()) / 128 * 128);
}

typedef __attribute__((address_space(3))) const unsigned int lds_u32_t;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x2_t lds_u32x2_t;
typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;

// The SB activations of one column, read from LDS byte address a, as SB/2 dwords.
template <int SB>
struct XCol {
  uint32_t d[SB < 2 ? 1 : SB / 2];
  __device__ __forceinline__ void read(uint32_t a) {
    if constexpr (SB == 1) {  // one 16-bit activation (2-byte aligned)
      d[0] = __builtin_bit_cast(uint16_t, spmv_detail::lds_half(a));
    } else if constexpr (SB == 2) {
      d[0] = *reinterpret_cast<lds_u32_t*>(uintptr_t(a));
    } else if constexpr (SB == 4) {
      const u32x2_t t = *reinterpret_cast<lds_u32x2_t*>(uintptr_t(a));
      d[0] = t.x;
      d[1] = t.y;
    } else {
      const u32x4_t t = *reinterpret_cast<lds_u32x4_t*>(uintptr_t(a));
      d[0] = t.x;
      d[1] = t.y;
      d[2] = t.z;
      d[3] = t.w;
    }
  }
  __device__ __forceinline__ _Float16 at(int b) const {
    const half2_t h = __builtin_bit_cast(half2_t, d[b >> 1]);
    return (b & 1) ? h.y : h.x;
  }
};

// acc[b] += w * x_b for the B activations of one kept weight.
template <int B, int SB>
__device__ __forceinline__ void fma_col(_Float16 w, const XCol<SB>& xc, float (&acc)[B]) {
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = __builtin_fmaf(float(w), float(xc.at(b)), acc[b]);
}

// Value k (0..7) of a lane's 16-byte chunk of packed values.
__device__ __forceinline__ _Float16 value_at(const uint4& v, int k) {
  const uint32_t d = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
  const half2_t h = __builtin_bit_cast(half2_t, d);
  return (k & 1) ? h.y : h.x;
}

// Byte-LUT tables for interleave stride SB: for each mask byte, the LDS byte offsets
// (column p of the byte -> 2*SB*p) of its set bits, lowest first, unused entries 0; the
// second table adds 8 columns (the byte's columns 8..15 of a half-word).
template <int SB>
__device__ __forceinline__ void stage_lut(uint2* lut, int tid, int nthreads) {
  for (int b = tid; b < 256; b += nthreads) {
    uint64_t lo = 0, hi = 0;
    int k = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if ((b >> p) & 1) {
        lo |= uint64_t(2 * SB * p) << (8 * k);
        hi |= uint64_t(2 * SB * (p + 8)) << (8 * k);
        ++k;
      }
    }
    lut[b] = make_uint2(uint32_t(lo), uint32_t(lo >> 32));
    lut[256 + b] = make_uint2(uint32_t(hi), uint32_t(hi >> 32));
  }
}

// One step of one lane: 8 kept values `v` of its half-word of mask word `m`.
//   LUT:  `xh` = LDS byte address of the half-word's first column, `lut` the tables.
//   bits: `xw` = LDS byte address of the word's first column.
template <int N, int B, int SB, int DEC>
__device__ __forceinline__ void step(const uint4& v, uint32_t m, int half, uint32_t xh, uint32_t xw,
                                     uint32_t lut, float (&acc)[B]) {
  if constexpr (DEC == kByteLut) {
    const uint32_t sh16 = 16u * unsigned(half);
    const uint32_t b0 = __builtin_amdgcn_ubfe(m, sh16, 8);
    const uint32_t b1 = __builtin_amdgcn_ubfe(m, sh16 + 8, 8);
    const uint2 l0 = spmv_detail::lds_u2(lut + 8u * b0);
    const uint2 l1 = spmv_detail::lds_u2(lut + 2048u + 8u * b1);
    uint32_t lo, hi;
    if constexpr (N <= 4) {  // exactly 4 kept columns in every mask byte
      lo = l0.x;
      hi = l1.x;
    } else {
      const uint64_t q = (uint64_t(l0.y) << 32 | l0.x) |
                         ((uint64_t(l1.y) << 32 | l1.x) << (8u * uint32_t(__builtin_popcount(b0))));
      lo = uint32_t(q);
      hi = uint32_t(q >> 32);
    }
    // four kept values at a time: their x reads, then their fmas
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t offs = h ? hi : lo;
      XCol<SB> xc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) xc[k].read(xh + ((offs >> (8 * k)) & 0xFFu));
#pragma unroll
      for (int k = 0; k < 4; ++k) fma_col<B, SB>(value_at(v, 4 * h + k), xc[k], acc);
      if (SB >= 4) __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // 2:4..8:16: the low-half lane walks the word's 8 lowest set bits, the high-half lane
    // those of the high 16 columns; 16:32: the high-half lane walks the bit-reversed word
    // from the window's last column down, and its values are reversed to match.
    const bool rev = N == 16 && half;
    uint32_t bits = N == 16 ? (half ? __builtin_bitreverse32(m) : m) : (half ? (m & 0xFFFF0000u) : m);
    const int stepb = rev ? -2 * SB : 2 * SB;
    const uint32_t base = rev ? xw + uint32_t(31 * 2 * SB) : xw;
    const uint4 vv = N == 16 ? reverse_half_word(v, rev ? 0x05040706u : 0x03020100u) : v;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      XCol<SB> xc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int p = __builtin_ctz(bits);  // exhausted word: -1, one column outside, still in the pad
        bits &= bits - 1;
        xc[k].read(base + uint32_t(stepb * p));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) fma_col<B, SB>(value_at(vv, 4 * h + k), xc[k], acc);
      if (SB >= 4) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Writes column group g (8 columns) of the current phase: x_b[i] for b < B, zero padding
// up to SB, at LDS byte address xbuf + (8g + i) * 2 * SB.
template <int B, int SB>
__device__ __forceinline__ void store_group(const uint4 (&xg)[B], int g, char* xbuf) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t d[SB < 2 ? 1 : SB / 2];
#pragma unroll
    for (int j = 0; j < (SB < 2 ? 1 : SB / 2); ++j) {
      uint32_t lo = 0, hi = 0;
      if (2 * j < B) {
        const uint32_t w = (i >> 1) == 0 ? xg[2 * j].x : (i >> 1) == 1 ? xg[2 * j].y : (i >> 1) == 2 ? xg[2 * j].z : xg[2 * j].w;
        lo = (i & 1) ? (w >> 16) : (w & 0xFFFFu);
      }
      if (2 * j + 1 < B) {
        const uint32_t w = (i >> 1) == 0 ? xg[2 * j + 1].x : (i >> 1) == 1 ? xg[2 * j + 1].y : (i >> 1) == 2 ? xg[2 * j + 1].z : xg[2 * j + 1].w;
        hi = (i & 1) ? (w >> 16) : (w & 0xFFFFu);
      }
      d[j] = lo | (hi << 16);
    }
    char* dst = xbuf + size_t(8 * g + i) * 2 * SB;
    if constexpr (SB == 1) {
      *reinterpret_cast<uint16_t*>(dst) = uint16_t(d[0]);
    } else if constexpr (SB == 2) {
      *reinterpret_cast<uint32_t*>(dst) = d[0];
    } else if constexpr (SB == 4) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(d[0], d[1]);
    } else {
      *reinterpret_cast<uint4*>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
    }
  }
}

// Loads column group g of X (columns c0 + 8g .. +8) for every b < B.
template <int B>
__device__ __forceinline__ void load_group(const uint16_t* __restrict__ X, int cols, int c, uint4 (&xg)[B]) {
#pragma unroll
  for (int b = 0; b < B; ++b)
    xg[b] = *reinterpret_cast<const uint4*>(X + size_t(b) * unsigned(cols) + unsigned(c));
}

// Register budget per batch size, the largest occupancy without spills: 6 waves per SIMD
// (80 VGPRs) for B = 1, 5 (96) for B = 2..5, 4 (128) for B = 6..8, 3 (168) for 16:32 at
// B = 6..8 (its high-half lanes also hold their values reversed): the B accumulators and
// the x reads of a step (SB/2 dwords per kept value) grow with B.
constexpr int waves_per_eu_of(int N, int B) { return B <= 1 ? 6 : B <= 5 ? 5 : (N == 16 ? 3 : 4); }
template <int N, int B>
constexpr int waves_per_eu() {
  return waves_per_eu_of(N, B);
}

// Largest workgroup: 16 waves, but 12 where 3 waves per SIMD are needed (a 16-wave
// workgroup needs 4 per SIMD, i.e. at most 128 VGPRs).
constexpr int max_waves_of(int N, int B) { return waves_per_eu_of(N, B) < 4 ? 12 : kMaxWaves; }
template <int N, int B>
constexpr int max_waves() {
  return max_waves_of(N, B);
}

// The dense kernel holds no decode state: 8 waves per SIMD up to B = 4, 6 up to 6, 4 above.
template <int B>
constexpr int dense_waves_per_eu() {
  return B <= 4 ? 8 : B <= 6 ? 6 : 4;
}

// CI > 1 (narrow layers, rpb <= RPW = 8 / CI rows per workgroup, one row group): the lanes
// of row slot s take row s % RPW and the (s / RPW)-th of CI near-equal, contiguous parts of
// the wave's steps, so that no lane repeats another lane's row (with 8-row slots and 4-row
// workgroups half of every wave would); the CI partial sums of a row are added across lanes
// before the LDS reduction.
template <int N, int B, int DEC, int CI>
__device__ __forceinline__ void spmm_body(const uint4* __restrict__ values, const uint32_t* __restrict__ masks,
                                          const uint16_t* __restrict__ X, uint16_t* __restrict__ Y, int rows,
                                          int cols, int rpb, int cs_count, int phase_cols) {
  static_assert(DEC == kByteLut || (DEC == kBitWalk), "byte LUT or bit walk");
  static_assert(DEC != kByteLut || N <= 8, "the byte LUT needs at most 8 kept columns per mask half-word");
  static_assert(CI == 1 || CI == 2 || CI == 4, "column parts per wave: 1, 2 or 4");
  constexpr int RPW = 8 / CI;                      // rows per wave
  constexpr int SB = stride_of<B>();
  constexpr int BATCH = 4;
  extern __shared__ uint4 lds[];
  char* lds_b = reinterpret_cast<char*>(lds);
  float* red = reinterpret_cast<float*>(lds_b);
  char* xbuf = lds_b + kXOffset;
  char* lut_p = xbuf + size_t(phase_cols) * 2 * SB + kPad;

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int CS = __builtin_amdgcn_readfirstlane(cs_count);
  const int rg = __builtin_amdgcn_readfirstlane(int(unsigned(wave) / unsigned(CS)));
  const int cs = wave - rg * CS;
  const int rsub = (lane & 31) >> 2;               // row slot within the wave's 8
  const int rrow = rsub % RPW;                     // its row within the wave's RPW rows
  const int cpart = rsub / RPW;                    // its part of the wave's steps
  const int u = ((lane >> 5) << 2) | (lane & 3);
  const int half = u & 1;
  const int wsel = u >> 1;
  const int row0 = blockIdx.x * rpb;
  const int row_end = min(row0 + rpb, rows);
  const unsigned r = unsigned(min(row0 + 8 * rg + rrow, row_end - 1));

  const int words = cols >> 5;
  const int steps = (words + 3) >> 2;
  const int full_steps = words >> 2;
  const int psteps = phase_cols >> 7;
  const uint4* __restrict__ vrow = values + size_t(r) * unsigned(cols >> 4);
  const uint32_t* __restrict__ mrow = masks + size_t(r) * unsigned(words);
  const uint32_t xbase = lds_address(xbuf);
  const uint32_t lut = lds_address(lut_p);

  if constexpr (DEC == kByteLut) stage_lut<SB>(reinterpret_cast<uint2*>(lut_p), tid, nthreads);

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.f;

  for (int p0 = 0; p0 < steps; p0 += psteps) {
    const int p1 = min(steps, p0 + psteps);
    const int pn = p1 - p0;
    const int w_beg = p0 + int(unsigned(pn) * unsigned(cs) / unsigned(CS));
    const int w_end = p0 + int(unsigned(pn) * unsigned(cs + 1) / unsigned(CS));
    // this lane's part of the wave's steps (the whole range when CI == 1)
    const int s_beg = w_beg + int(unsigned(w_end - w_beg) * unsigned(cpart) / unsigned(CI));
    const int s_end = w_beg + int(unsigned(w_end - w_beg) * unsigned(cpart + 1) / unsigned(CI));
    const int s_main = min(s_end, full_steps);
    const int n = max(0, s_main - s_beg);
    const int nfull = n / BATCH;
    const int rem = n - nfull * BATCH;
    const int c0 = p0 << 7;                               // first column of the phase
    const int ngroups = (min(cols, p1 << 7) - c0) >> 3;   // 8-column groups of the phase

    if (p0 > 0) __syncthreads();  // every wave is done with the previous phase's x

    // prologue: x chunks, then the first value batch, then the LDS writes
    uint4 xg[B];
    load_group<B>(X, cols, c0 + 8 * min(tid, ngroups - 1), xg);
    __builtin_amdgcn_sched_barrier(0);
    spmv_detail::Batch<BATCH, true, 8, 4, 768, 256> A;
    A.load_clamped(vrow, 8u * unsigned(s_beg) + unsigned(u), unsigned(cols >> 4) - 1u, mrow,
                   4u * unsigned(s_beg) + unsigned(wsel), unsigned(words) - 1u);
    if (tid < ngroups) store_group<B, SB>(xg, tid, xbuf);
    for (int g = tid + nthreads; g < ngroups; g += nthreads) {
      uint4 xo[B];
      load_group<B>(X, cols, c0 + 8 * g, xo);
      store_group<B, SB>(xo, g, xbuf);
    }
    __syncthreads();

    // LDS byte address of this lane's word window in the batch's first step
    uint32_t xw = xbase + uint32_t((s_beg - p0) * 128 + 32 * wsel) * 2u * SB;
    const uint32_t xhalf = 16u * 2u * SB * unsigned(half);
    const uint4* __restrict__ vp = vrow + 8 * unsigned(s_beg) + unsigned(u);
    const uint32_t* __restrict__ mp = mrow + 4 * unsigned(s_beg) + unsigned(wsel);
    for (int bt = 0; bt < nfull; ++bt) {
      if (bt > 0) A.load(vp, mp, BATCH);
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        step<N, B, SB, DEC>(A.v[i], A.m[i], half, xw + 128u * 2u * SB * i + xhalf, xw + 128u * 2u * SB * i, lut, acc);
        // one step's x reads live at a time (8 columns x SB/2 dwords), not the batch's
        __builtin_amdgcn_sched_barrier(0);
      }
      vp += 8 * BATCH;
      mp += 4 * BATCH;
      xw += 128u * 2u * SB * BATCH;
    }
    if (rem > 0) {
      spmv_detail::Batch<BATCH, true, 8, 4, 768, 256> R;
      R.load(vp, mp, rem);
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        if (i < rem)
          step<N, B, SB, DEC>(R.v[i], R.m[i], half, xw + 128u * 2u * SB * i + xhalf, xw + 128u * 2u * SB * i, lut, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // last step of the row with 1..3 words: lanes whose word exists
    if (s_end > full_steps && wsel < (words & 3)) {
      const unsigned s = unsigned(full_steps);
      spmv_detail::Batch<1, true, 8, 4, 768, 256> T;
      T.load(vrow + 8 * s + unsigned(u), mrow + 4 * s + unsigned(wsel), 1);
      const uint32_t xt = xbase + uint32_t((int(s) - p0) * 128 + 32 * wsel) * 2u * SB;
      step<N, B, SB, DEC>(T.v[0], T.m[0], half, xt + xhalf, xt, lut, acc);
    }
  }

  // row sums: DPP inside the quad and the partner half-wave, the CI parts (row slots
  // rrow + k * RPW, lanes 4 * RPW apart), then LDS across the CS waves
#pragma unroll
  for (int b = 0; b < B; ++b) {
    float s = row8_sum(acc[b]);
#pragma unroll
    for (int d = 4 * RPW; d < 32; d <<= 1) s += __shfl_xor(s, d);
    if (u == 0 && cpart == 0) red[(wave * 8 + rrow) * kMaxBatch + b] = s;
  }
  __syncthreads();
  const int nr = row_end - row0;
  if (tid < B * rpb) {
    const int b = tid / rpb, rr = tid - b * rpb;
    if (rr < nr) {
      const int trg = rr >> 3, trow = rr & 7;
      float t = 0.f;
      for (int k = 0; k < CS; ++k) t += red[((trg * CS + k) * 8 + trow) * kMaxBatch + b];
      Y[size_t(b) * unsigned(rows) + unsigned(row0 + rr)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(t));
    }
  }
}

template <int N, int B, int DEC>
__global__ __launch_bounds__((64 * max_waves<N, B>())) __attribute__((amdgpu_waves_per_eu((waves_per_eu<N, B>())))) void spmm_kernel(
    const uint4* __restrict__ values, const uint32_t* __restrict__ masks, const uint16_t* __restrict__ X,
    uint16_t* __restrict__ Y, int rows, int cols, int rpb, int cs_count, int phase_cols) {
  spmm_body<N, B, DEC, 1>(values, masks, X, Y, rows, cols, rpb, cs_count, phase_cols);
}

template <int N, int B, int DEC, int CI>
__global__ __launch_bounds__((64 * max_waves<N, B>())) __attribute__((amdgpu_waves_per_eu((waves_per_eu<N, B>())))) void spmm_narrow_kernel(
    const uint4* __restrict__ values, const uint32_t* __restrict__ masks, const uint16_t* __restrict__ X,
    uint16_t* __restrict__ Y, int rows, int cols, int rpb, int cs_count, int phase_cols) {
  spmm_body<N, B, DEC, CI>(values, masks, X, Y, rows, cols, rpb, cs_count, phase_cols);
}

// ---------------------------------------------------------------- dense counterpart
// Y = X W^T for the dense fp16 W: the gemv_kernel mapping (8 lanes per row, one 128-byte
// line of 64 columns per step, nontemporal loads), with X staged per phase as B separate
// vectors ([b][c]: the 8 lanes of a row read the same 16-byte chunks of every vector, and
// the 8 rows of a wave share them). Per 8 weights and activation vector: 4 v_dot2_f32_f16.
constexpr size_t dense_lds_bytes(int B, int phase_cols) {
  return kRedBytes + size_t(B) * size_t(phase_cols) * 2;
}

template <int B>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(dense_waves_per_eu<B>()))) void gemm_kernel(
    const uint4* __restrict__ W, const uint16_t* __restrict__ X, uint16_t* __restrict__ Y, int rows, int cols,
    int rpb, int cs_count, int phase_cols) {
  constexpr int BATCH = 4;
  extern __shared__ uint4 lds[];
  float* red = reinterpret_cast<float*>(lds);
  uint4* xs = lds + kRedBytes / 16;  // [B][phase_cols / 8] uint4

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

  const int words2 = cols >> 5;
  const int steps = (words2 + 1) >> 1;          // 64 columns per step
  const int full_steps = words2 >> 1;
  const int psteps = phase_cols >> 6;
  const int pc16 = phase_cols >> 3;             // uint4 per staged vector
  const uint4* __restrict__ wrow = W + size_t(r) * unsigned(cols >> 3);

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.f;

  for (int p0 = 0; p0 < steps; p0 += psteps) {
    const int p1 = min(steps, p0 + psteps);
    const int pn = p1 - p0;
    const int s_beg = p0 + int(unsigned(pn) * unsigned(cs) / unsigned(CS));
    const int s_end = p0 + int(unsigned(pn) * unsigned(cs + 1) / unsigned(CS));
    const int s_main = min(s_end, full_steps);
    const int n = max(0, s_main - s_beg);
    const int nfull = n / BATCH;
    const int rem = n - nfull * BATCH;
    const int c0 = p0 << 6;
    const int n16 = (min(cols, p1 << 6) - c0) >> 3;   // uint4 per vector in this phase
    const int total = B * n16;

    if (p0 > 0) __syncthreads();

    // prologue: the first x chunk, then the first batch of W (clamped), then LDS writes
    const int i0 = min(tid, total - 1);
    const int b0 = i0 / n16;
    const uint4 x0 = *reinterpret_cast<const uint4*>(X + size_t(b0) * unsigned(cols) + unsigned(c0 + 8 * (i0 - b0 * n16)));
    __builtin_amdgcn_sched_barrier(0);
    uint4 wv[BATCH];
    const unsigned wo = 8u * unsigned(s_beg) + unsigned(u), wlast = unsigned(cols >> 3) - 1u;
#pragma unroll
    for (int i = 0; i < BATCH; ++i) wv[i] = load16<true>(wrow + min(wo + 8u * unsigned(i), wlast));
    if (tid < total) xs[b0 * pc16 + (i0 - b0 * n16)] = x0;
    for (int i = tid + nthreads; i < total; i += nthreads) {
      const int b = i / n16, j = i - b * n16;
      xs[b * pc16 + j] = *reinterpret_cast<const uint4*>(X + size_t(b) * unsigned(cols) + unsigned(c0 + 8 * j));
    }
    __syncthreads();

    const uint4* __restrict__ wp = wrow + 8 * unsigned(s_beg) + unsigned(u);
    int xo = 8 * (s_beg - p0) + u;  // uint4 index of this lane's 8 columns within the phase
    for (int bt = 0; bt < nfull; ++bt) {
      if (bt > 0) {
#pragma unroll
        for (int i = 0; i < BATCH; ++i) wv[i] = load16<true>(wp + 8 * i);
      }
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = dot8(wv[i], xs[b * pc16 + xo + 8 * i], acc[b]);
      wp += 8 * BATCH;
      xo += 8 * BATCH;
    }
    if (rem > 0) {
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        if (i < rem) wv[i] = load16<true>(wp + 8 * i);
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        if (i < rem)
#pragma unroll
          for (int b = 0; b < B; ++b) acc[b] = dot8(wv[i], xs[b * pc16 + xo + 8 * i], acc[b]);
    }
    // cols % 64 == 32: the row's last step has 32 columns, held by lanes 0..3
    if (s_end > full_steps && u < 4) {
      const int s = full_steps;
      const uint4 wt = load16<true>(wrow + 8 * unsigned(s) + unsigned(u));
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = dot8(wt, xs[b * pc16 + 8 * (s - p0) + u], acc[b]);
    }
  }

#pragma unroll
  for (int b = 0; b < B; ++b) {
    float s = dpp_quad_sum(acc[b]);
    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x141, 0xF, 0xF, true));
    if (u == 0) red[(wave * 8 + rsub) * kMaxBatch + b] = s;
  }
  __syncthreads();
  const int nr = row_end - row0;
  if (tid < B * rpb) {
    const int b = tid / rpb, rr = tid - b * rpb;
    if (rr < nr) {
      const int trg = rr >> 3, trow = rr & 7;
      float t = 0.f;
      for (int k = 0; k < CS; ++k) t += red[((trg * CS + k) * 8 + trow) * kMaxBatch + b];
      Y[size_t(b) * unsigned(rows) + unsigned(row0 + rr)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(t));
    }
  }
}

}  // namespace spmm_detail
}  // namespace nm
