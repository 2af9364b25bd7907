// Batch-one N:M sparse matrix-vector product y = W x on gfx950: the kernel template.
//
// Method (pages: news.bitwarelabs.com "SparseDecoding: decoding-aware pruning for
// accurate and fast LLM generation", "What's new"; aimodeling.com SparseDecoding
// article, "The Kernel Is the Other Half of the Answer"): the weights are read once
// per product, so the kernel is bound by HBM bandwidth; a 32-bit mask word indexes 32
// input columns and carries exactly 16 kept values at 50% density, so the values of
// word w start at a fixed offset 16*w and the traversal of a word is a fixed number
// of steps with no prefix scan.
//
// Work mapping (one workgroup = 16 rows x all columns, WAVES waves):
//   * A "step" covers 64 columns (2 mask words) of every row of the tile. In one step
//     each row's 64 bytes of packed values are split over 4 lanes: lane u of the row
//     loads one 16-byte dwordx4 holding 8 values, the half h = u & 1 of word
//     2*step + (u >> 1). The 16 rows x 4 lanes fill the 64 lanes of a wave, and a
//     wave's consecutive steps walk each row 64 bytes at a time (the two halves of a
//     128-byte line are read by consecutive instructions of the same wave).
//   * The WAVES waves split the steps of the row range evenly (contiguous ranges) and
//     their partial sums are combined in LDS in a fixed order.
//   * Loads of packed values and masks are issued BATCH steps at a time.
//   * Products are fp16 x fp16 (exact in fp32) accumulated in fp32 by v_dot2_f32_f16
//     on pairs of values, reduced across the row's 4 lanes with DPP, then across waves
//     in LDS, and rounded once to fp16.
//
// Two ways to find the x of each kept value (the "decoder"):
//   * Bit walk (any pattern): x is staged in LDS and every kept value gathers its x
//     with one 16-bit LDS read at the position of the next set bit of its mask bits
//     (find-lowest-set-bit, then clear it: a fixed 8 steps per lane). For 2:4, 4:8 and
//     8:16 each 16-column half of a word holds exactly 8 kept columns, so the lane
//     owning half h walks the set bits of (mask & half h); for 16:32 the lane with the
//     low 8 values walks the lowest 8 set bits and the lane with the high 8 values
//     first clears the lowest 8. In one wave instruction the 32 lanes of a half-wave
//     touch at most two adjacent mask words, i.e. 32 consecutive dwords of x, so the
//     gathers hit distinct banks or broadcast.
//   * Pair table (2:4 only): every aligned group of 4 columns keeps exactly 2, one of
//     6 patterns, and the two kept values of a group are one fp16 pair of the packed
//     row. The workgroup stages, for each group, the 6 possible x pairs (24 bytes) in
//     LDS, in the order of the pattern's nibble n (slot (n >> 1) - 1 for n = 3, 5, 6,
//     9, 10, 12). One 32-bit LDS read then returns the x pair of a value pair, and one
//     v_dot2 consumes it: a 3-bit field extract, an address add, one LDS read and one
//     dot per two values.
//   Both decoders stay inside the LDS allocation for any mask bits (a malformed mask
//   gives an unspecified y, never an out-of-bounds access): the data region has 64
//   bytes of padding on each side, more than the furthest a bad mask can reach.
#pragma once

#include "nm_internal.h"

namespace nm {
namespace spmv_detail {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

enum Decoder { kBitWalk = 0, kPairTable = 1 };

constexpr int kPad = 64;  // bytes of LDS padding on each side of the x data

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if constexpr (NT) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
  } else {
    return *p;
  }
}

template <bool NT>
__device__ __forceinline__ uint32_t load4(const uint32_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

__device__ __forceinline__ float dpp_quad_sum(float v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of a quad ends with the quad's sum.
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  return v;
}

__device__ __forceinline__ float dot2(uint32_t v, half2_t x, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v), x, acc, false);
}

// LDS layout: [reduction: WAVES x 16 floats][pad][x data][pad].
constexpr int data_offset(int waves) { return int(reduction_lds_bytes(waves)) + kPad; }

template <int DEC>
constexpr size_t data_bytes(int cols) {
  return DEC == kPairTable ? size_t(cols) / 4 * 24 : size_t(cols) * 2;
}

template <int DEC>
constexpr size_t lds_bytes(int cols, int waves) {
  return size_t(data_offset(waves)) + data_bytes<DEC>(cols) + kPad;
}

// ---------------------------------------------------------------- bit-walk decoder
// Set bits of the mask word that belong to this lane's 8 values.
template <int N>
__device__ __forceinline__ uint32_t lane_bits(uint32_t m, int half, uint32_t keep_high) {
  if constexpr (N < 16) {
    // keep_high is 0xFFFFFFFF for the low-half lane (it walks only the 8 lowest set bits,
    // which are exactly the low half's), 0xFFFF0000 for the high-half lane.
    (void)half;
    return m & keep_high;
  } else {
    (void)keep_high;
    uint32_t hi = m;
#pragma unroll
    for (int i = 0; i < 8; ++i) hi &= hi - 1;  // clear the 8 lowest set bits
    return half ? hi : m;
  }
}

// 32-bit LDS byte address of an LDS object, and 16-bit loads from such addresses (LDS
// addresses wrap modulo 2^32, so a step of -2 bytes stays a plain 32-bit add).
typedef __attribute__((address_space(3))) const char lds_char_t;
typedef __attribute__((address_space(3))) const _Float16 lds_half_t;

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_char_t*)(p)));  // generic -> LDS address space
}

__device__ __forceinline__ _Float16 lds_half(uint32_t a) {
  return *reinterpret_cast<lds_half_t*>(uintptr_t(a));
}

// x pairs of this lane's 8 kept columns: `bits` holds the columns as set bits relative to
// xw, the LDS byte address of the mask word's x window (v_ffbl of an exhausted word is
// -1: one element before the window, still inside the padded LDS data region).
__device__ __forceinline__ void gather_bits(uint32_t bits, uint32_t xw, half2_t (&xp)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t p0 = uint32_t(__builtin_ctz(bits));
    bits &= bits - 1;
    const uint32_t p1 = uint32_t(__builtin_ctz(bits));
    bits &= bits - 1;
    xp[k].x = lds_half(xw + 2u * p0);
    xp[k].y = lds_half(xw + 2u * p1);
  }
}

// ---------------------------------------------------------------- pair-table decoder
// Slot of a 2:4 nibble n in its group's 6 pairs: (n >> 1) - 1, i.e. 0..5 for
// n = 3 (cols 0,1), 5 (0,2), 6 (1,2), 9 (0,3), 10 (1,3), 12 (2,3).
__device__ __forceinline__ void stage_pair_table(const uint4* __restrict__ x, uint32_t* __restrict__ tbl,
                                                 int cols, int tid, int nthreads) {
  const int pairs_of_groups = cols >> 3;  // 8 columns = 2 groups per uint4 of x
  for (int i = tid; i < pairs_of_groups; i += nthreads) {
    const uint4 v = x[i];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const uint32_t lo = d[2 * gg], hi = d[2 * gg + 1];  // (x0, x1), (x2, x3)
      const uint32_t x0 = lo & 0xFFFFu, x1 = lo >> 16, x2 = hi & 0xFFFFu, x3 = hi >> 16;
      uint32_t* t = tbl + 6 * (2 * i + gg);
      t[0] = lo;                   // n = 3:  (x0, x1)
      t[1] = x0 | (x2 << 16);      // n = 5:  (x0, x2)
      t[2] = x1 | (x2 << 16);      // n = 6:  (x1, x2)
      t[3] = x0 | (x3 << 16);      // n = 9:  (x0, x3)
      t[4] = x1 | (x3 << 16);      // n = 10: (x1, x3)
      t[5] = hi;                   // n = 12: (x2, x3)
    }
  }
}

// ---------------------------------------------------------------- batches
// One batch of BATCH steps for one lane. Per step the lane's values advance VSTEP uint4s,
// its mask MSTEP words, its pair-table position TSTEP bytes and its x window XSTEP bytes.
template <int BATCH, bool NTV, int VSTEP, int MSTEP, int TSTEP, int XSTEP>
struct Batch {
  uint4 v[BATCH];
  uint32_t m[BATCH];

  // Loads `count` steps starting at vp / mp (count == BATCH: no guards). Values may be
  // nontemporal (NTV); masks are plain loads (a mask line is shared by several steps).
  __device__ __forceinline__ void load(const uint4* __restrict__ vp, const uint32_t* __restrict__ mp,
                                       int count) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      if (i < count) {
        v[i] = load16<NTV>(vp + VSTEP * i);
        m[i] = mp[MSTEP * i];
      }
    }
  }

  // Bit walk: `xw` is the LDS byte address of the x window of this lane's word in the
  // batch's first step.
  template <int N>
  __device__ __forceinline__ void compute_bits(uint32_t xw, int half, uint32_t keep_high, int count,
                                               float (&part)[4]) const {
    half2_t xp[BATCH][4];
#pragma unroll
    for (int i = 0; i < BATCH; ++i)
      if (i < count) gather_bits(lane_bits<N>(m[i], half, keep_high), xw + uint32_t(XSTEP) * i, xp[i]);
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      if (i < count) {
        float a = part[i & 3];
        a = dot2(v[i].x, xp[i][0], a);
        a = dot2(v[i].y, xp[i][1], a);
        a = dot2(v[i].z, xp[i][2], a);
        a = dot2(v[i].w, xp[i][3], a);
        part[i & 3] = a;
      }
    }
  }

  // Pair table: `tb` points 4 bytes before the table entries of this lane's half-word in
  // the batch's first step; `sh` = 16*half + 1 is the bit offset of the slot field of the
  // lane's first nibble.
  __device__ __forceinline__ void compute_pairs(const char* __restrict__ tb, uint32_t sh, int count,
                                                float (&part)[4]) const {
    uint32_t xp[BATCH][4];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      if (i < count) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // (nibble >> 1) of the lane's nibble g: 1..6 for the valid 2:4 nibbles
          const uint32_t slot = __builtin_amdgcn_ubfe(m[i], sh + 4 * g, 3);
          xp[i][g] = *reinterpret_cast<const uint32_t*>(tb + 4 * slot + (TSTEP * i + 24 * g));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      if (i < count) {
        float a = part[i & 3];
        a = dot2(v[i].x, __builtin_bit_cast(half2_t, xp[i][0]), a);
        a = dot2(v[i].y, __builtin_bit_cast(half2_t, xp[i][1]), a);
        a = dot2(v[i].z, __builtin_bit_cast(half2_t, xp[i][2]), a);
        a = dot2(v[i].w, __builtin_bit_cast(half2_t, xp[i][3]), a);
        part[i & 3] = a;
      }
    }
  }
};

// Stages x (bit walk) or its pair table in the LDS data region.
template <int DEC>
__device__ __forceinline__ void stage_x(const uint4* __restrict__ x, char* data, int cols, int tid, int nthreads) {
  if constexpr (DEC == kPairTable) {
    stage_pair_table(x, reinterpret_cast<uint32_t*>(data), cols, tid, nthreads);
  } else {
    uint4* xs4 = reinterpret_cast<uint4*>(data);
    const int n16 = cols >> 3;
    for (int i = tid; i < n16; i += nthreads) xs4[i] = x[i];
  }
}

template <int N, int WAVES, int BATCH, bool NT, int DEC>
__global__ __launch_bounds__(64 * WAVES) void spmv_kernel(const uint4* __restrict__ values,
                                                          const uint32_t* __restrict__ masks,
                                                          const uint4* __restrict__ x,
                                                          uint16_t* __restrict__ y, int rows, int cols) {
  static_assert(DEC == kBitWalk || N == 2, "the pair table decodes 2:4 only");
  extern __shared__ uint4 lds[];
  char* lds_b = reinterpret_cast<char*>(lds);
  float* red = reinterpret_cast<float*>(lds_b);
  char* data = lds_b + data_offset(WAVES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps loop bounds scalar
  const int u = lane & 3;          // lane within the row's quad
  const int half = u & 1;          // which 8 values of the word
  const int wsel = u >> 1;         // which of the step's 2 words
  const int row0 = blockIdx.x * kRowsPerBlock;
  // Lanes past the last row read the last row again; their sums are never stored.
  const unsigned r = unsigned(min(row0 + (lane >> 2), rows - 1));

  const int words = cols >> 5;
  const int steps = (words + 1) >> 1;
  const int full_steps = words >> 1;
  const int s_beg = int((int64_t(steps) * wave) / WAVES);
  const int s_end = int((int64_t(steps) * (wave + 1)) / WAVES);
  const int s_main = min(s_end, full_steps);

  const uint4* __restrict__ vrow = values + size_t(r) * unsigned(cols >> 4);
  const uint32_t* __restrict__ mrow = masks + size_t(r) * unsigned(words);
  const uint32_t keep_high = half ? 0xFFFF0000u : 0xFFFFFFFFu;

  // Per step the lane's values advance 64 bytes (4 x uint4) and its mask 2 words.
  const uint4* __restrict__ vp = vrow + 4 * unsigned(s_beg) + unsigned(u);
  const uint32_t* __restrict__ mp = mrow + 2 * unsigned(s_beg) + unsigned(wsel);
  const int n = s_main - s_beg;      // wave-uniform
  const int nfull = n / BATCH;
  const int rem = n - nfull * BATCH;

  using B = Batch<BATCH, NT, 4, 2, 384, 128>;
  B A;
  if (nfull > 0) A.load(vp, mp, BATCH);  // first batch in flight while x is staged

  // Stage x (or its pair table) in LDS.
  stage_x<DEC>(x, data, cols, tid, 64 * WAVES);
  __syncthreads();

  // This lane's x data position in the first step of its range; a step is 64 columns.
  uint32_t xw = lds_address(data) + 128u * unsigned(s_beg) + 64u * unsigned(wsel);
  const char* tb = data - 4 + 384 * unsigned(s_beg) + 192 * unsigned(wsel) + 96 * unsigned(half);
  const uint32_t sh = 16u * unsigned(half) + 1u;

  float part[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < nfull; ++b) {
    if (b > 0) A.load(vp, mp, BATCH);
    if constexpr (DEC == kPairTable) A.compute_pairs(tb, sh, BATCH, part);
    else A.template compute_bits<N>(xw, half, keep_high, BATCH, part);
    vp += 4 * BATCH;
    mp += 2 * BATCH;
    xw += 128u * BATCH;
    tb += 384 * BATCH;
  }
  if (rem > 0) {  // fewer than BATCH full steps left
    B R;
    R.load(vp, mp, rem);
    if constexpr (DEC == kPairTable) R.compute_pairs(tb, sh, rem, part);
    else R.template compute_bits<N>(xw, half, keep_high, rem, part);
  }
  // Odd word count: the last step holds a single word, owned by the lanes with wsel == 0.
  if (s_end > full_steps && wsel == 0) {
    const unsigned s = unsigned(full_steps);
    Batch<1, NT, 4, 2, 384, 128> T;
    T.load(vrow + 4 * s + unsigned(u), mrow + 2 * s, 1);
    if constexpr (DEC == kPairTable)
      T.compute_pairs(data - 4 + 384 * s + 96 * unsigned(half), sh, 1, part);
    else
      T.template compute_bits<N>(lds_address(data) + 128u * s, half, keep_high, 1, part);
  }
  float acc = (part[0] + part[1]) + (part[2] + part[3]);

  acc = dpp_quad_sum(acc);
  if (u == 0) red[wave * kRowsPerBlock + (lane >> 2)] = acc;
  __syncthreads();
  if (tid < kRowsPerBlock) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < WAVES; ++k) t += red[k * kRowsPerBlock + tid];
    const int rr = row0 + tid;
    if (rr < rows) y[rr] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(t));
  }
}

// ---------------------------------------------------------------- full-line variant
// Same method, with 8 lanes per row: in one step the 8 lanes of a row load the row's next
// 128 bytes of packed values (one whole cache line, 4 mask words = 128 columns), so every
// line is consumed by a single wave instruction and the values can be streamed with
// nontemporal loads (NTV). A wave instruction covers 8 rows; a workgroup has RG row
// groups of 8 rows and CS waves splitting the columns of each row group (RG*CS waves).
// Row sums: DPP inside the quad, row_half_mirror across the two quads of the row, then
// LDS across the CS waves, in a fixed order.
__device__ __forceinline__ float dpp_octet_sum(float v) {
  v = dpp_quad_sum(v);
  // row_half_mirror: lane i of each 8-lane half-row reads lane 7 - i (the other quad)
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  return v;
}

constexpr size_t line_reduction_bytes(int waves) { return size_t(waves) * 8 * sizeof(float); }
constexpr int line_data_offset(int waves) { return int(line_reduction_bytes(waves)) + kPad; }

template <int DEC>
constexpr size_t line_lds_bytes(int cols, int waves) {
  return size_t(line_data_offset(waves)) + data_bytes<DEC>(cols) + kPad;
}

template <int N, int RG, int CS, int BATCH, bool NTV, int DEC>
__global__ __launch_bounds__(64 * RG * CS) void spmv_line_kernel(const uint4* __restrict__ values,
                                                                 const uint32_t* __restrict__ masks,
                                                                 const uint4* __restrict__ x,
                                                                 uint16_t* __restrict__ y, int rows, int cols) {
  static_assert(DEC == kBitWalk || N == 2, "the pair table decodes 2:4 only");
  constexpr int WAVES = RG * CS;
  constexpr int ROWS = 8 * RG;
  extern __shared__ uint4 lds[];
  char* lds_b = reinterpret_cast<char*>(lds);
  float* red = reinterpret_cast<float*>(lds_b);
  char* data = lds_b + line_data_offset(WAVES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave / CS;
  const int cs = wave - rg * CS;
  const int u = lane & 7;          // lane within the row's octet: half-word u of the step
  const int half = u & 1;
  const int wsel = u >> 1;         // which of the step's 4 words
  const int row0 = blockIdx.x * ROWS;
  const unsigned r = unsigned(min(row0 + 8 * rg + (lane >> 3), rows - 1));

  const int words = cols >> 5;
  const int steps = (words + 3) >> 2;
  const int full_steps = words >> 2;
  const int s_beg = int((int64_t(steps) * cs) / CS);
  const int s_end = int((int64_t(steps) * (cs + 1)) / CS);
  const int s_main = min(s_end, full_steps);

  const uint4* __restrict__ vrow = values + size_t(r) * unsigned(cols >> 4);
  const uint32_t* __restrict__ mrow = masks + size_t(r) * unsigned(words);
  const uint32_t keep_high = half ? 0xFFFF0000u : 0xFFFFFFFFu;

  const uint4* __restrict__ vp = vrow + 8 * unsigned(s_beg) + unsigned(u);
  const uint32_t* __restrict__ mp = mrow + 4 * unsigned(s_beg) + unsigned(wsel);
  const int n = s_main - s_beg;
  const int nfull = n / BATCH;
  const int rem = n - nfull * BATCH;

  using B = Batch<BATCH, NTV, 8, 4, 768, 256>;
  B A;
  if (nfull > 0) A.load(vp, mp, BATCH);  // first batch in flight while x is staged

  stage_x<DEC>(x, data, cols, tid, 64 * WAVES);
  __syncthreads();

  uint32_t xw = lds_address(data) + 256u * unsigned(s_beg) + 64u * unsigned(wsel);
  const char* tb = data - 4 + 768 * unsigned(s_beg) + 192 * unsigned(wsel) + 96 * unsigned(half);
  const uint32_t sh = 16u * unsigned(half) + 1u;

  float part[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < nfull; ++b) {
    if (b > 0) A.load(vp, mp, BATCH);
    if constexpr (DEC == kPairTable) A.compute_pairs(tb, sh, BATCH, part);
    else A.template compute_bits<N>(xw, half, keep_high, BATCH, part);
    vp += 8 * BATCH;
    mp += 4 * BATCH;
    xw += 256u * BATCH;
    tb += 768 * BATCH;
  }
  if (rem > 0) {
    B R;
    R.load(vp, mp, rem);
    if constexpr (DEC == kPairTable) R.compute_pairs(tb, sh, rem, part);
    else R.template compute_bits<N>(xw, half, keep_high, rem, part);
  }
  // Last step with 1..3 words (cols not a multiple of 128): lanes whose word exists.
  if (s_end > full_steps && wsel < (words & 3)) {
    const unsigned s = unsigned(full_steps);
    Batch<1, NTV, 8, 4, 768, 256> T;
    T.load(vrow + 8 * s + unsigned(u), mrow + 4 * s + unsigned(wsel), 1);
    if constexpr (DEC == kPairTable)
      T.compute_pairs(data - 4 + 768 * s + 192 * unsigned(wsel) + 96 * unsigned(half), sh, 1, part);
    else
      T.template compute_bits<N>(lds_address(data) + 256u * s + 64u * unsigned(wsel), half, keep_high, 1, part);
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

}  // namespace spmv_detail
}  // namespace nm
