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
// Work mapping (spmv_kernel below): a workgroup covers 8*RG rows x all columns;
// its RG*CS waves take RG groups of 8 rows, and CS waves split each row group's
// columns into contiguous ranges. In one "step" the 8 lanes of a row each load 16 bytes
// (8 values, half a mask word) of the row's next 128-byte line of packed values (4 mask
// words, 128 columns), so a wave instruction consumes 8 whole cache lines. Loads are
// issued BATCH steps at a time. Products are fp16 x fp16 (exact in fp32) accumulated in
// fp32 by v_dot2_f32_f16 on pairs of values, reduced across the row's 8 lanes, then across
// the CS waves in LDS in a fixed order, and rounded once to fp16.
//
// Four ways to find the x of each kept value (the "decoder"), all with a fixed number
// of steps per mask word and no prefix scan:
//   * Pair table (2:4): every aligned group of 4 columns keeps exactly 2, one of 6
//     patterns, and the two kept values of a group are one fp16 pair of the packed row.
//     The workgroup stages, for each group, the 6 possible x pairs (24 bytes) in LDS in
//     the order of the pattern's nibble n (slot (n >> 1) - 1 for n = 3, 5, 6, 9, 10, 12).
//     One 32-bit LDS read returns the x pair of a value pair and one v_dot2 consumes it:
//     a 3-bit field extract, an address add, one LDS read and one dot per two values.
//   * Byte LUT (4:8, 8:16): x is staged in LDS with two 256-entry tables giving, for a
//     mask byte, the byte offsets of its set bits. The two bytes of a lane's half-word
//     give its 8 offsets (for 8:16 concatenated with one 64-bit shift by 8 * popcount of
//     the low byte); each value then costs one SDWA byte-select add and one 16-bit LDS read.
//   * Reversed walk (16:32): x is staged with a copy in which each mask word's 32
//     elements are reversed. The low-half lane walks the 8 lowest set bits of the word
//     (find-lowest-set-bit, clear it); the high-half lane walks the 8 lowest set bits of
//     the bit-reversed word, i.e. the 8 highest columns, in the reversed copy, with its
//     values reversed by one v_perm per pair.
//   * Bit walk (any pattern; used when the larger tables do not fit in LDS): as above on
//     the plain copy; for 16:32 the high-half lane walks down from the window's end.
//   Every decoder stays inside the LDS allocation for any mask bits (a malformed mask
//   gives an unspecified y, never an out-of-bounds access): the data region has 64
//   bytes of padding on each side, more than the furthest a bad mask can reach.
#pragma once

#include "nm_internal.h"

namespace nm {
namespace spmv_detail {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

enum Decoder { kBitWalk = 0, kPairTable = 1, kByteLut = 2, kRevWalk = 3 };

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

// Byte-LUT tables: for each mask byte b, the byte offsets 2p of its set bits p (lowest
// first, unused entries 0), once as is and once +16 (the byte's columns 8..15 of a half-word).
constexpr size_t kLutBytes = 2 * 256 * 8;

// kRevWalk (16:32) stages x and, after it, a copy with every mask word's 32 elements in
// reverse order, which the high-half lanes walk.
template <int DEC>
constexpr size_t data_bytes(int cols) {
  return DEC == kPairTable ? size_t(cols) / 4 * 24
       : DEC == kByteLut   ? size_t(cols) * 2 + kLutBytes
       : DEC == kRevWalk   ? size_t(cols) * 4
                           : size_t(cols) * 2;
}

// ---------------------------------------------------------------- bit-walk decoder
// Set bits of the mask word that belong to this lane's 8 values, lowest first.
// For 2:4, 4:8 and 8:16 every 16-column half of a word holds exactly 8 kept columns:
// keep_high is 0xFFFFFFFF for the low-half lane (it walks only the 8 lowest set bits,
// which are exactly the low half's) and 0xFFFF0000 for the high-half lane. For 16:32 the
// high-half lane walks the bit-reversed word instead, so that its 8 values are the 8
// lowest set bits of that (see reverse_half_word for its values).
template <int N>
__device__ __forceinline__ uint32_t lane_bits(uint32_t m, int half, uint32_t keep_high) {
  if constexpr (N < 16) {
    (void)half;
    return m & keep_high;
  } else {
    (void)keep_high;
    return half ? __builtin_bitreverse32(m) : m;
  }
}

// The high-half lane of a 16:32 word meets its values from the highest column down, so
// its 8 values are reversed: pair j becomes (v[15-2j], v[14-2j]) of the word. One v_perm
// per pair with a lane-dependent selector (identity for the low-half lane).
__device__ __forceinline__ uint4 reverse_half_word(uint4 v, uint32_t sel) {
  return make_uint4(__builtin_amdgcn_perm(v.w, v.x, sel), __builtin_amdgcn_perm(v.z, v.y, sel),
                    __builtin_amdgcn_perm(v.y, v.z, sel), __builtin_amdgcn_perm(v.x, v.w, sel));
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

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x2_t lds_u2_t;
__device__ __forceinline__ uint2 lds_u2(uint32_t a) {
  const u32x2_t t = *reinterpret_cast<lds_u2_t*>(uintptr_t(a));
  return make_uint2(t.x, t.y);
}

// x pairs of this lane's 8 kept columns: `bits` holds the columns as set bits; column p
// sits at LDS byte address xw + step * p (step = 2, or -2 from the window's last element
// for a bit-reversed 16:32 word). v_ffbl of an exhausted word is -1: one element outside
// the window, still inside the padded LDS data region. The 8 addresses come first, then the
// 8 reads, then the pairs, so that the step's reads are in flight together (one LDS round
// trip per step rather than one per pair).
__device__ __forceinline__ void gather_bits(uint32_t bits, uint32_t xw, int step, half2_t (&xp)[4]) {
  uint32_t a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int p0 = __builtin_ctz(bits);
    bits &= bits - 1;
    a[k] = xw + uint32_t(step * p0);
  }
  _Float16 h[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) h[k] = lds_half(a[k]);
#pragma unroll
  for (int k = 0; k < 4; ++k) xp[k] = half2_t{h[2 * k], h[2 * k + 1]};
}

// Byte-LUT gather for 4:8 and 8:16: the half-word's two mask bytes give their set-bit
// offsets from the tables (one 64-bit LDS read each); the two lists are concatenated with
// one 64-bit shift by 8 * popcount(low byte), modulo 64 (for 4:8 the low byte always holds 4); byte k
// of the result is the offset of value k from xh, the half-word's x window. The 8 reads are
// issued before the pairs are formed, as in gather_bits.
template <int N>
__device__ __forceinline__ void gather_lut(uint32_t m, uint32_t sh16, uint32_t lut, uint32_t xh,
                                           half2_t (&xp)[4]) {
  const uint32_t b0 = __builtin_amdgcn_ubfe(m, sh16, 8);
  const uint32_t b1 = __builtin_amdgcn_ubfe(m, sh16 + 8, 8);
  const uint2 l0 = lds_u2(lut + 8u * b0);
  const uint2 l1 = lds_u2(lut + 2048u + 8u * b1);
  uint32_t lo, hi;
  if constexpr (N == 4) {
    lo = l0.x;
    hi = l1.x;
  } else {
    // A valid half-word keeps 8 values, so when the low byte keeps all 8 (a shift of 64) the
    // high byte keeps none and its list is 0: the shift amount is taken modulo 64, which keeps
    // the shift defined and leaves the result unchanged.
    const uint32_t shift = (8u * uint32_t(__builtin_popcount(b0))) & 63u;
    const uint64_t q = (uint64_t(l0.y) << 32 | l0.x) | ((uint64_t(l1.y) << 32 | l1.x) << shift);
    lo = uint32_t(q);
    hi = uint32_t(q >> 32);
  }
  _Float16 h[8];
  h[0] = lds_half(xh + (lo & 0xFFu));
  h[1] = lds_half(xh + ((lo >> 8) & 0xFFu));
  h[2] = lds_half(xh + ((lo >> 16) & 0xFFu));
  h[3] = lds_half(xh + (lo >> 24));
  h[4] = lds_half(xh + (hi & 0xFFu));
  h[5] = lds_half(xh + ((hi >> 8) & 0xFFu));
  h[6] = lds_half(xh + ((hi >> 16) & 0xFFu));
  h[7] = lds_half(xh + (hi >> 24));
#pragma unroll
  for (int k = 0; k < 4; ++k) xp[k] = half2_t{h[2 * k], h[2 * k + 1]};
}

// Builds the two byte-LUT tables (256 entries of 8 bytes each) at `lut`.
__device__ __forceinline__ void stage_byte_lut(uint2* lut, int tid, int nthreads) {
  for (int b = tid; b < 256; b += nthreads) {
    uint64_t lo = 0, hi = 0;
    int k = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if ((b >> p) & 1) {
        lo |= uint64_t(2 * p) << (8 * k);
        hi |= uint64_t(2 * p + 16) << (8 * k);
        ++k;
      }
    }
    lut[b] = make_uint2(uint32_t(lo), uint32_t(lo >> 32));
    lut[256 + b] = make_uint2(uint32_t(hi), uint32_t(hi >> 32));
  }
}

// ---------------------------------------------------------------- pair-table decoder
// Slot of a 2:4 nibble n in its group's 6 pairs: (n >> 1) - 1, i.e. 0..5 for
// n = 3 (cols 0,1), 5 (0,2), 6 (1,2), 9 (0,3), 10 (1,3), 12 (2,3). The table itself is
// written by store_x_chunk.

// ---------------------------------------------------------------- batches
// One batch of BATCH steps for one lane. Per step the lane's values advance VSTEP uint4s,
// its mask MSTEP words, its pair-table position TSTEP bytes and its x window XSTEP bytes.
template <int BATCH, bool NTV, int VSTEP, int MSTEP, int TSTEP, int XSTEP>
struct Batch {
  uint4 v[BATCH];
  uint32_t m[BATCH];

  // Loads a whole batch unconditionally, every offset clamped to the row's last uint4 of
  // values (vlast) and last mask word (mlast): when the batch lies inside the row the
  // clamps change nothing; otherwise the lane reads valid data it will not use. Being
  // branch-free, these loads let the compiler wait for earlier loads with an exact count.
  __device__ __forceinline__ void load_clamped(const uint4* __restrict__ vrow, unsigned vo, unsigned vlast,
                                               const uint32_t* __restrict__ mrow, unsigned mo, unsigned mlast) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      v[i] = load16<NTV>(vrow + min(vo + unsigned(VSTEP * i), vlast));
      m[i] = mrow[min(mo + unsigned(MSTEP * i), mlast)];
    }
  }

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
  // batch's first step. 16:32 high-half lanes walk the bit-reversed word: with XR their
  // `xw` points into the reversed copy of x (step +2); without it they walk the plain
  // window from its last element down (step -2).
  template <int N, bool XR>
  __device__ __forceinline__ void compute_bits(uint32_t xw, int half, uint32_t keep_high, int count,
                                               float (&part)[4]) const {
    const bool rev = N == 16 && half;
    const int step = (rev && !XR) ? -2 : 2;
    const uint32_t xoff = (rev && !XR) ? 62u : 0u;
    const uint32_t sel = rev ? 0x05040706u : 0x03020100u;
    half2_t xp[BATCH][4];
#pragma unroll
    for (int i = 0; i < BATCH; ++i)
      if (i < count) gather_bits(lane_bits<N>(m[i], half, keep_high), xw + uint32_t(XSTEP) * i + xoff, step, xp[i]);
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      if (i < count) {
        const uint4 vv = N == 16 ? reverse_half_word(v[i], sel) : v[i];
        float a = part[i & 3];
        a = dot2(vv.x, xp[i][0], a);
        a = dot2(vv.y, xp[i][1], a);
        a = dot2(vv.z, xp[i][2], a);
        a = dot2(vv.w, xp[i][3], a);
        part[i & 3] = a;
      }
    }
  }

  // Byte LUT (4:8, 8:16): `xh` is the LDS byte address of this lane's half-word x window
  // in the batch's first step, `lut` the tables, `sh16` = 16 * half.
  template <int N>
  __device__ __forceinline__ void compute_lut(uint32_t xh, uint32_t lut, uint32_t sh16, int count,
                                              float (&part)[4]) const {
    half2_t xp[BATCH][4];
#pragma unroll
    for (int i = 0; i < BATCH; ++i)
      if (i < count) gather_lut<N>(m[i], sh16, lut, xh + uint32_t(XSTEP) * i, xp[i]);
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

// Writes chunk i of x (elements 8i..8i+7, one uint4) into the LDS data region in the
// decoder's form: the plain copy; for the pair table the 6 x pairs of each of its two
// 4-column groups; for the reversed walk also the reversed copy, in which quarter q of
// every mask word's 32 elements holds quarter 3 - q of x, elements reversed.
template <int DEC>
__device__ __forceinline__ void store_x_chunk(uint4 v, int i, char* data, int cols) {
  if constexpr (DEC == kPairTable) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const uint32_t lo = d[2 * gg], hi = d[2 * gg + 1];  // (x0, x1), (x2, x3)
      const uint32_t x0 = lo & 0xFFFFu, x1 = lo >> 16, x2 = hi & 0xFFFFu, x3 = hi >> 16;
      uint32_t* t = reinterpret_cast<uint32_t*>(data) + 6 * (2 * i + gg);
      t[0] = lo;                   // n = 3:  (x0, x1)
      t[1] = x0 | (x2 << 16);      // n = 5:  (x0, x2)
      t[2] = x1 | (x2 << 16);      // n = 6:  (x1, x2)
      t[3] = x0 | (x3 << 16);      // n = 9:  (x0, x3)
      t[4] = x1 | (x3 << 16);      // n = 10: (x1, x3)
      t[5] = hi;                   // n = 12: (x2, x3)
    }
  } else {
    reinterpret_cast<uint4*>(data)[i] = v;
    if constexpr (DEC == kRevWalk) {
      const int j = (i & ~3) | (3 - (i & 3));  // the quarter that mirrors chunk i in its word
      reinterpret_cast<uint4*>(data + size_t(cols) * 2)[j] =
          make_uint4(__builtin_amdgcn_alignbit(v.w, v.w, 16), __builtin_amdgcn_alignbit(v.z, v.z, 16),
                     __builtin_amdgcn_alignbit(v.y, v.y, 16), __builtin_amdgcn_alignbit(v.x, v.x, 16));
    }
  }
  (void)cols;
}

// ---------------------------------------------------------------- kernel
// 8 lanes per row: in one step the 8 lanes of a row load the row's next 128 bytes of
// packed values (one whole cache line, 4 mask words = 128 columns), so every line is
// consumed by a single wave instruction and the values can be streamed with nontemporal
// loads (NTV). A wave instruction covers 8 rows. Lanes are ordered so that each half-wave
// holds the same half of every row's line: lanes 4r..4r+3 take half-words 0..3 (words 0,
// 1) of row r and lanes 32+4r..32+4r+3 half-words 4..7 (words 2, 3), so the LDS reads of
// a half-wave touch only 2 consecutive mask words' x data (no bank conflicts for the bit
// walk; 8 table groups for the pair table).
//
// Sum over the 8 lanes of a row (lanes 4r..4r+3 and 32+4r..32+4r+3): DPP inside the
// quad, then the partner half-wave's quad (lane ^ 32).
__device__ __forceinline__ float row8_sum(float v) {
  v = dpp_quad_sum(v);
  v += __shfl_xor(v, 32);
  return v;
}

constexpr int kMaxWaves = 16;  // 1024 threads per workgroup at most
constexpr size_t kReductionBytes = size_t(kMaxWaves) * 8 * sizeof(float);
constexpr int kDataOffset = int(kReductionBytes) + kPad;

template <int DEC>
constexpr size_t lds_bytes(int cols) {
  return size_t(kDataOffset) + data_bytes<DEC>(cols) + kPad;
}

// Workgroup shape, chosen per launch: the workgroup owns `rpb` consecutive rows (any
// count; the grid is ceil(rows / rpb)), split into RG = ceil(rpb / 8) groups of 8 rows;
// each group has `cs` waves that split the columns into contiguous ranges of whole steps
// (blockDim.x == 64 * RG * cs <= 1024). Lanes of rows past the workgroup's last row load
// that last row again (same addresses, no extra memory traffic) and their sums are dropped.
// Row sums: DPP inside the quad, the partner half-wave, then the cs waves in LDS in a
// fixed order.
//
// Order of the prologue: each thread first loads its (up to two) chunks of x, then the
// first batch of its values, and only then writes x to LDS, so that the wait for x does
// not include the wait for the value batch (loads complete in order) and the staging
// overlaps the value stream.
//
// CI > 1 (narrow layers of RPW = 8 / CI rows per workgroup, cols a multiple of 128): a wave
// covers RPW rows and the lanes of row slot s take row s % RPW and the (s / RPW)-th of CI
// equal, contiguous column ranges inside the wave's range, so that no lane repeats another
// lane's row; the launcher picks CS = steps / (BATCH * CI), so that every lane has exactly
// one batch of whole steps, which the prologue loads. The CI partial sums of a row are added
// across lanes before the LDS reduction.
//
// `block` is the workgroup's index within the product (blockIdx.x for a single product).
template <int N, int BATCH, bool NTV, int DEC, int CI>
__device__ __forceinline__ void spmv_body(
    const uint4* __restrict__ values, const uint32_t* __restrict__ masks, const uint4* __restrict__ x,
    uint16_t* __restrict__ y, int rows, int cols, int rpb, int cs_count, int block) {
  static_assert((DEC != kPairTable || N == 2) && (DEC != kByteLut || N == 4 || N == 8) &&
                    (DEC != kRevWalk || N == 16),
                "pair table: 2:4 only; byte LUT: 4:8 and 8:16 only; reversed walk: 16:32 only");
  extern __shared__ uint4 lds[];
  char* lds_b = reinterpret_cast<char*>(lds);
  float* red = reinterpret_cast<float*>(lds_b);
  char* data = lds_b + kDataOffset;

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int CS = __builtin_amdgcn_readfirstlane(cs_count);
  const int rg = __builtin_amdgcn_readfirstlane(int(unsigned(wave) / unsigned(CS)));
  const int cs = wave - rg * CS;
  static_assert(CI == 1 || CI == 2 || CI == 4 || CI == 8, "column parts per wave: 1, 2, 4 or 8");
  constexpr int RPW = 8 / CI;                      // rows per wave
  const int rsub = (lane & 31) >> 2;               // row slot within the wave's 8
  const int rrow = rsub % RPW;                     // its row within the wave's RPW rows
  const int cpart = rsub / RPW;                    // its column range of the wave's CI
  const int u = ((lane >> 5) << 2) | (lane & 3);   // half-word u of the step's 8
  const int half = u & 1;
  const int wsel = u >> 1;                         // which of the step's 4 words
  const int row0 = block * rpb;
  const int row_end = min(row0 + rpb, rows);
  const unsigned r = unsigned(min(row0 + 8 * rg + rrow, row_end - 1));

  const int words = cols >> 5;
  const int steps = (words + 3) >> 2;
  const int full_steps = words >> 2;
  // steps * (cs + 1) < 2^23 * 16: 32-bit arithmetic is exact (cols <= 2^30)
  // CI > 1: every lane has `len` == BATCH whole steps (steps == full_steps)
  const int len = steps / (CS * CI);
  const int s_beg = CI == 1 ? int(unsigned(steps) * unsigned(cs) / unsigned(CS)) : len * (cs * CI + cpart);
  const int s_end = CI == 1 ? int(unsigned(steps) * unsigned(cs + 1) / unsigned(CS)) : s_beg + len;
  const int s_main = min(s_end, full_steps);

  const uint4* __restrict__ vrow = values + size_t(r) * unsigned(cols >> 4);
  const uint32_t* __restrict__ mrow = masks + size_t(r) * unsigned(words);
  const uint32_t keep_high = half ? 0xFFFF0000u : 0xFFFFFFFFu;

  const uint4* __restrict__ vp = vrow + 8 * unsigned(s_beg) + unsigned(u);
  const uint32_t* __restrict__ mp = mrow + 4 * unsigned(s_beg) + unsigned(wsel);
  const int n = CI == 1 ? s_main - s_beg : len;    // wave-uniform
  const int nfull = n / BATCH;
  const int rem = n - nfull * BATCH;

  // prologue: x chunks, then the first value batch, then the LDS writes (all loads
  // unconditional, see load_clamped)
  const int n16 = cols >> 3;
  const int i0 = tid, i1 = tid + nthreads;
  const bool two_chunks = n16 > nthreads;  // workgroup-uniform
  const uint4 x0 = x[min(i0, n16 - 1)];
  uint4 x1 = make_uint4(0u, 0u, 0u, 0u);
  if (two_chunks) x1 = x[min(i1, n16 - 1)];
  __builtin_amdgcn_sched_barrier(0);  // keep the x loads ahead of the value batch
  using B = Batch<BATCH, NTV, 8, 4, 768, 256>;
  B A;
  A.load_clamped(vrow, 8u * unsigned(s_beg) + unsigned(u), unsigned(cols >> 4) - 1u, mrow,
                 4u * unsigned(s_beg) + unsigned(wsel), unsigned(words) - 1u);
  if constexpr (DEC == kByteLut) stage_byte_lut(reinterpret_cast<uint2*>(data + size_t(cols) * 2), tid, nthreads);
  if (i0 < n16) store_x_chunk<DEC>(x0, i0, data, cols);
  if (two_chunks && i1 < n16) store_x_chunk<DEC>(x1, i1, data, cols);
  for (int i = i1 + nthreads; i < n16; i += nthreads) store_x_chunk<DEC>(x[i], i, data, cols);
  __syncthreads();

  uint32_t xw = lds_address(data) + 256u * unsigned(s_beg) + 64u * unsigned(wsel);
  const char* tb = data - 4 + 768 * unsigned(s_beg) + 192 * unsigned(wsel) + 96 * unsigned(half);
  const uint32_t sh = 16u * unsigned(half) + 1u;
  const uint32_t sh16 = 16u * unsigned(half);
  const uint32_t xhalf = 32u * unsigned(half);                      // byte offset of the half-word's x
  const uint32_t lut = lds_address(data) + 2u * unsigned(cols);     // byte-LUT tables after x
  // 16:32 high-half lanes read the reversed copy of x, which follows x
  const uint32_t xrev = (DEC == kRevWalk && half) ? 2u * unsigned(cols) : 0u;

  float part[4] = {0.f, 0.f, 0.f, 0.f};
  // products of one batch whose first step's x window / pair table sit at xw_ / tb_
  auto compute = [&](const B& S, uint32_t xw_, const char* tb_, int count) {
    if constexpr (DEC == kPairTable) S.compute_pairs(tb_, sh, count, part);
    else if constexpr (DEC == kByteLut) S.template compute_lut<N>(xw_ + xhalf, lut, sh16, count, part);
    else S.template compute_bits<N, DEC == kRevWalk>(xw_ + xrev, half, keep_high, count, part);
  };
  if constexpr (CI > 1) {
    // every lane has exactly one batch (the launcher sets len == BATCH): the prologue's
    compute(A, xw, tb, BATCH);
  } else {
    for (int b = 0; b < nfull; ++b) {
      if (b > 0) A.load(vp, mp, BATCH);
      compute(A, xw, tb, BATCH);
      vp += 8 * BATCH;
      mp += 4 * BATCH;
      xw += 256u * BATCH;
      tb += 768 * BATCH;
    }
    if (rem > 0) {
      B R;
      R.load(vp, mp, rem);
      compute(R, xw, tb, rem);
    }
  }
  // Last step with 1..3 words (cols not a multiple of 128): lanes whose word exists.
  if (s_end > full_steps && wsel < (words & 3)) {
    const unsigned s = unsigned(full_steps);
    Batch<1, NTV, 8, 4, 768, 256> T;
    T.load(vrow + 8 * s + unsigned(u), mrow + 4 * s + unsigned(wsel), 1);
    if constexpr (DEC == kPairTable)
      T.compute_pairs(data - 4 + 768 * s + 192 * unsigned(wsel) + 96 * unsigned(half), sh, 1, part);
    else if constexpr (DEC == kByteLut)
      T.template compute_lut<N>(lds_address(data) + 256u * s + 64u * unsigned(wsel) + xhalf, lut, sh16, 1, part);
    else
      T.template compute_bits<N, DEC == kRevWalk>(lds_address(data) + 256u * s + 64u * unsigned(wsel) + xrev, half, keep_high, 1, part);
  }
  float acc = (part[0] + part[1]) + (part[2] + part[3]);

  acc = row8_sum(acc);
  // CI > 1: add the row's CI column ranges (row slots rrow + k * RPW, lanes 4 * RPW apart)
#pragma unroll
  for (int d = 4 * RPW; d < 32; d <<= 1) acc += __shfl_xor(acc, d);
  if (u == 0 && cpart == 0) red[wave * 8 + rsub] = acc;
  __syncthreads();
  if (tid < row_end - row0) {
    const int trg = tid >> 3, trow = tid & 7;
    float t = 0.f;
    for (int k = 0; k < CS; ++k) t += red[(trg * CS + k) * 8 + trow];
    y[row0 + tid] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(t));
  }
}

// Register budget: 64 VGPRs, so that 8 waves fit on each SIMD (two 16-wave workgroups per
// CU). At 65..72 VGPRs only 7 fit and a CU holds a single 16-wave workgroup, which leaves
// nothing to overlap one workgroup's staging of x and its final reduction with. (The body
// is a separate inlined function: the kernel compiled this way was measured 1-7% faster
// for 4:8 and 8:16 on layers of 4096 columns than with the body written in the kernel.)
template <int N, int BATCH, bool NTV, int DEC>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(8))) void spmv_kernel(
    const uint4* __restrict__ values, const uint32_t* __restrict__ masks, const uint4* __restrict__ x,
    uint16_t* __restrict__ y, int rows, int cols, int rpb, int cs_count) {
  spmv_body<N, BATCH, NTV, DEC, 1>(values, masks, x, y, rows, cols, rpb, cs_count, int(blockIdx.x));
}

// Narrow layers (at most 8 rows per CU, at most 64 steps per row): rows per workgroup
// 8 / CI with CI column ranges per wave, the same register budget.
template <int N, int BATCH, bool NTV, int DEC, int CI>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(8))) void spmv_narrow_kernel(
    const uint4* __restrict__ values, const uint32_t* __restrict__ masks, const uint4* __restrict__ x,
    uint16_t* __restrict__ y, int rows, int cols, int rpb, int cs_count) {
  spmv_body<N, BATCH, NTV, DEC, CI>(values, masks, x, y, rows, cols, rpb, cs_count, int(blockIdx.x));
}

// Several products that share x and one workgroup shape, in one launch (for example q, k
// and v, or gate and up, stored as separate matrices): product k owns workgroups
// [block0[k], block0[k + 1]) of the grid and runs the single-product body on them, so its y
// is the one a launch of spmv_kernel with the same rows per workgroup and waves gives. One
// launch fills and drains the memory pipeline once for all of them.
constexpr int kMaxGroup = 8;
struct GroupArgs {
  const uint4* x;
  int cols;
  int cs;   // waves per workgroup (one row group)
  int rpb;  // rows per workgroup
  int count;
  int block0[kMaxGroup + 1];
  const uint4* values[kMaxGroup];
  const uint32_t* masks[kMaxGroup];
  uint16_t* y[kMaxGroup];
  int rows[kMaxGroup];
};

template <int N, int BATCH, bool NTV, int DEC>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(8))) void spmv_group_kernel(
    const GroupArgs a) {
  const int b = int(blockIdx.x);
  // the product this workgroup serves: the number of product starts at or below b (static
  // indices, so the starts come in one scalar load rather than a chain of dependent ones)
  int k = 0;
#pragma unroll
  for (int j = 1; j < kMaxGroup; ++j) k += (j < a.count && b >= a.block0[j]) ? 1 : 0;
  spmv_body<N, BATCH, NTV, DEC, 1>(a.values[k], a.masks[k], a.x, a.y[k], a.rows[k], a.cols, a.rpb, a.cs,
                                   b - a.block0[k]);
}

// ---------------------------------------------------------------- 25% density
// The same method for N:M with N/M = 1/4 (1:4, 2:8, 4:16, 8:32): every mask word keeps 8
// values (16 bytes), so each of a row's 8 lanes takes one whole word per step (the step
// still covers one 128-byte line of the row's values, now 8 words = 256 columns; lanes
// 4r..4r+3 words 0..3, lanes 32+4r..32+4r+3 words 4..7) and walks its 8 set bits with a
// fixed number of steps (find-lowest-set-bit, clear it), gathering x from the word's
// 32-column window of the staged copy. The pattern only fixes how the 8 bits are spread,
// not the work, so one kernel serves all four. Workgroup shape, prologue order, register
// budget and reduction are those of spmv_kernel.
template <int BATCH, bool NTV>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(8))) void spmv_quarter_kernel(
    const uint4* __restrict__ values, const uint32_t* __restrict__ masks, const uint4* __restrict__ x,
    uint16_t* __restrict__ y, int rows, int cols, int rpb, int cs_count) {
  extern __shared__ uint4 lds[];
  char* lds_b = reinterpret_cast<char*>(lds);
  float* red = reinterpret_cast<float*>(lds_b);
  char* data = lds_b + kDataOffset;

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int CS = __builtin_amdgcn_readfirstlane(cs_count);
  const int rg = __builtin_amdgcn_readfirstlane(int(unsigned(wave) / unsigned(CS)));
  const int cs = wave - rg * CS;
  const int rsub = (lane & 31) >> 2;
  const int u = ((lane >> 5) << 2) | (lane & 3);   // the step's word u of 8
  const int row0 = blockIdx.x * rpb;
  const int row_end = min(row0 + rpb, rows);
  const unsigned r = unsigned(min(row0 + 8 * rg + rsub, row_end - 1));

  const int words = cols >> 5;
  const int steps = (words + 7) >> 3;
  const int full_steps = words >> 3;
  const int s_beg = int(unsigned(steps) * unsigned(cs) / unsigned(CS));
  const int s_end = int(unsigned(steps) * unsigned(cs + 1) / unsigned(CS));
  const int s_main = min(s_end, full_steps);

  const uint4* __restrict__ vrow = values + size_t(r) * unsigned(cols >> 5);   // 8 values per word
  const uint32_t* __restrict__ mrow = masks + size_t(r) * unsigned(words);
  const uint4* __restrict__ vp = vrow + 8 * unsigned(s_beg) + unsigned(u);
  const uint32_t* __restrict__ mp = mrow + 8 * unsigned(s_beg) + unsigned(u);
  const int n = s_main - s_beg;
  const int nfull = n / BATCH;
  const int rem = n - nfull * BATCH;

  // prologue: x chunks, then the first batch (clamped into the row), then the LDS writes
  const int n16 = cols >> 3;
  const int i0 = tid, i1 = tid + nthreads;
  const bool two_chunks = n16 > nthreads;
  const uint4 x0 = x[min(i0, n16 - 1)];
  uint4 x1 = make_uint4(0u, 0u, 0u, 0u);
  if (two_chunks) x1 = x[min(i1, n16 - 1)];
  __builtin_amdgcn_sched_barrier(0);
  using B = Batch<BATCH, NTV, 8, 8, 0, 512>;
  B A;
  A.load_clamped(vrow, 8u * unsigned(s_beg) + unsigned(u), unsigned(cols >> 5) - 1u, mrow,
                 8u * unsigned(s_beg) + unsigned(u), unsigned(words) - 1u);
  if (i0 < n16) store_x_chunk<kBitWalk>(x0, i0, data, cols);
  if (two_chunks && i1 < n16) store_x_chunk<kBitWalk>(x1, i1, data, cols);
  for (int i = i1 + nthreads; i < n16; i += nthreads) store_x_chunk<kBitWalk>(x[i], i, data, cols);
  __syncthreads();

  // LDS byte address of this lane's word window (32 columns) in the batch's first step
  uint32_t xw = lds_address(data) + 512u * unsigned(s_beg) + 64u * unsigned(u);
  constexpr uint32_t kAll = 0xFFFFFFFFu;  // the lane walks all 8 set bits of its word
  float part[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < nfull; ++b) {
    if (b > 0) A.load(vp, mp, BATCH);
    A.template compute_bits<2, false>(xw, 0, kAll, BATCH, part);
    vp += 8 * BATCH;
    mp += 8 * BATCH;
    xw += 512u * BATCH;
  }
  if (rem > 0) {
    B R;
    R.load(vp, mp, rem);
    R.template compute_bits<2, false>(xw, 0, kAll, rem, part);
  }
  // last step with 1..7 words (cols not a multiple of 256): lanes whose word exists
  if (s_end > full_steps && u < (words & 7)) {
    const unsigned s = unsigned(full_steps);
    Batch<1, NTV, 8, 8, 0, 512> T;
    T.load(vrow + 8 * s + unsigned(u), mrow + 8 * s + unsigned(u), 1);
    T.template compute_bits<2, false>(lds_address(data) + 512u * s + 64u * unsigned(u), 0, kAll, 1, part);
  }
  float acc = (part[0] + part[1]) + (part[2] + part[3]);

  acc = row8_sum(acc);
  if (u == 0) red[wave * 8 + rsub] = acc;
  __syncthreads();
  if (tid < row_end - row0) {
    const int trg = tid >> 3, trow = tid & 7;
    float t = 0.f;
    for (int k = 0; k < CS; ++k) t += red[(trg * CS + k) * 8 + trow];
    y[row0 + tid] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(t));
  }
}

}  // namespace spmv_detail
}  // namespace nm
