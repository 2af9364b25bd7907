// Prefill-sized products on the gfx950 matrix cores: the 2:4 sparse product on the sparse
// matrix instruction and its dense counterpart on the dense one, from one kernel skeleton.
//
// Y [tokens][rows] = X [tokens][cols] W'^T, W' the pruned weight (packed: kept values in
// row order, one 32-bit mask word per 32 columns) or the dense weight.
//
// Prefill is compute-bound and runs sparse matrix-matrix products (news.bitwarelabs.com
// "SparseDecoding: decoding-aware pruning for accurate and fast LLM generation", "What's
// new"), the regime where 2:4 sparse matrix hardware pays off (aimodeling.com SparseDecoding
// article, "The Kernel Is the Other Half of the Answer": 1.31 to 1.46x over dense in
// prefill on the pages' GPU). On gfx950 that hardware is v_smfmac_f32_16x16x64_f16:
// D[16 x 16] += A[16 x 64] B[64 x 16] with A 2:4 sparse along K, given as its 32 kept
// values plus per lane a 16-bit index word of 2-bit positions, at twice the dense rate.
//
// Lane layout of the sparse instruction (measured on gfx950 by multiplying one-hot
// compressed A operands with a labelled B):
//   A: lane l holds row l % 16. With q = l / 16 its 8 halves are the kept pairs (ascending
//      column) of the 4-column groups b_q + {0, 1, 4, 5} of the instruction's K, b_q =
//      8 (q & 1) + 2 (q >> 1). Nibble i of the index word is the pair's position code
//      p0 | p1 << 2 (p0 < p1, positions 0..3 in the group) for the i-th of those groups.
//   B: lane l holds token l % 16 at K = 16 (l / 16) + j, j = 0..15.
//   D: lane l holds token l % 16, rows 4 (l / 16) + e, e = 0..3.
// The instruction's K order is free as long as A and B agree, so it is permuted to suit
// the packed format: lane q's groups are the actual column groups 4q .. 4q+3 of the
// 64-column step. Its 8 values are then packed values 8q .. 8q+7 of the step (one 16-byte
// load; a 2:4 group keeps exactly two values, adjacent in the packed row) and its index
// word comes from the 16 mask bits of those groups (half q & 1 of mask word q >> 1). The
// B lane with q = l / 16 then holds actual columns 8q .. 8q+7 and 32+8q .. 32+8q+7.
//
// Dense instruction v_mfma_f32_16x16x32_f16: A lane l holds row l % 16, K 8 (l / 16) + j;
// B lane l holds token l % 16, K 8 (l / 16) + j; D as above.
//
// Work mapping: a workgroup of 4 waves takes 4 * 16 * TR rows x 16 * TT tokens; each wave
// TR x TT output tiles of 16 x 16 (its own rows, all the workgroup's tokens). Per step of
// KS columns the workgroup stages the X tile (16 * TT tokens x 2 KS bytes) in LDS
// (double-buffered; 16-byte chunks XOR-swizzled by token so the fragment reads are free of
// bank conflicts) and each wave loads its own weight fragments straight into registers;
// both kinds of load are issued D steps ahead, as range-checked buffer loads. Per 64
// columns a wave issues TR * TT sparse instructions (2 * TR * TT dense ones) and reads TT
// X fragments from LDS, each one token tile ahead of its products. Workgroups are mapped
// to output tiles XCD by XCD (tile_of).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace nm {
namespace prefill_detail {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h16_t __attribute__((ext_vector_type(16)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u8_t __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;     // waves per workgroup, stacked along rows
constexpr int kThreads = 64 * kWaves;

// KS = columns per main-loop step (64 or 128).
template <int TR, int TT, int KS>
struct Tile {
  static constexpr int kRows = kWaves * 16 * TR;      // rows per workgroup
  static constexpr int kTokens = 16 * TT;             // tokens per workgroup
  static constexpr int kRowBytes = 2 * KS;            // one token's X slice per step
  static constexpr int kXBytes = kTokens * kRowBytes; // one X buffer
  static constexpr int kXChunks = kTokens * KS / 8;   // its 16-byte chunks
  static constexpr int kXPerThread = kXChunks / kThreads;
  static constexpr int kSub = KS / 64;                // 64-column sub-steps
  static_assert(KS == 64 || KS == 128, "step of 64 or 128 columns");
  static_assert(kXChunks % kThreads == 0, "X tile must split evenly over the workgroup");
};

// 2:4 position code (p0 | p1 << 2) of each 4-bit mask nibble with two set bits, as a
// 16-entry table of nibbles (the definition pair_codes32 is checked against).
constexpr uint64_t kPairCodes = (0x4ull << (4 * 0x3)) | (0x8ull << (4 * 0x5)) | (0x9ull << (4 * 0x6)) |
                                (0xCull << (4 * 0x9)) | (0xDull << (4 * 0xA)) | (0xEull << (4 * 0xC));

// The position codes of all 8 nibbles of a mask word at once (nibble i of the result is the
// code of nibble i), by bit operations: for a nibble with exactly two set bits b_p0, b_p1
// (p0 < p1), p0 = 0 iff b0, 1 iff !b0 & b1, else 2; p1 = 3 iff b3, 2 iff !b3 & b2, else 1. So
// code bit 0 = !b0 & b1, bit 1 = !b0 & !b1, bit 2 = b3 | !b2, bit 3 = b3 | b2. The table above
// on every nibble with two set bits (checked below at compile time); other nibbles
// (zero-filled tails, malformed masks) get some code, and their values are zero or the
// result is unspecified anyway.
__host__ __device__ constexpr uint32_t pair_codes32(uint32_t m) {
  const uint32_t t = m >> 1;
  return (~m & t & 0x11111111u) | ((~(m | t) & 0x11111111u) << 1) | ((t | ~m) & 0x44444444u) |
         ((m | (m << 1)) & 0x88888888u);
}

constexpr bool pair_codes_match_table() {
  for (uint32_t n = 0; n < 16; ++n) {
    if (__builtin_popcount(n) != 2) continue;
    for (int i = 0; i < 8; ++i)
      if (((pair_codes32(n << (4 * i)) >> (4 * i)) & 0xFu) != ((kPairCodes >> (4 * n)) & 0xFu)) return false;
  }
  return true;
}
static_assert(pair_codes_match_table(), "bitwise position codes disagree with the table");

// ---- 4:8 and 8:16 on the 2:4 instruction (split operands) ----
// These patterns keep exactly 8 values in every 16 aligned columns, so a lane's 16-byte
// load holds the kept values of its 16 columns (4 groups), but a 4-column group may keep
// 0 .. 4 of them. Each group is split in two: its first two kept values (ascending column)
// form a pair of a 2:4 operand A, the third and fourth a pair of a 2:4 operand B, with
// zeros where a group keeps fewer; A and B go through the sparse instruction with the same
// X fragment into the same accumulator. Moving the values into place is a per-lane shuffle
// that depends only on the lane's 16 mask bits: a table indexed by (side, mask byte) gives
// for each output dword two byte selectors (one over values 0..3, one over values 4..7,
// v_perm_b32, results ORed) and the pairs' 2-bit position codes. The low mask byte's values
// are ranks 0 .. c-1 of the lane's 8 and the high byte's the last ones, 8 - c' .. 7 (c, c'
// their bit counts), so each byte's entry depends on that byte alone.
//
// ---- split tables (4:8, 8:16) ----
// Entry (side, byte), side 0 for the low mask byte of a lane's 16 bits, 1 for the high one:
// sel[4 g + {0, 1}] = selectors of operand A's pair for the byte's group g (over values 0..3,
// over values 4..7), sel[4 g + {2, 3}] the same for operand B; idx bits 4 g .. 4 g + 3 = A's
// position code for group g, bits 8 + 4 g .. = B's. Selector byte 0x0C gives a zero byte.
constexpr int kSplitEntries = 512;
constexpr uint32_t kSplitSelBytes = kSplitEntries * 32;
constexpr uint32_t kSplitLutBytes = kSplitSelBytes + kSplitEntries * 2;   // + 16-bit codes

struct SplitEntry {
  uint32_t sel[8];
  uint32_t idx;
};

// selector bytes placing value `rank` of the lane's 8 (-1: zero) as one fp16 half, for the
// operand pair (values 0..3) when !high, (values 4..7) when high
__host__ __device__ constexpr uint32_t split_half_sel(int rank, bool high) {
  if (rank < 0 || (rank >= 4) != high) return 0x0C0Cu;
  const uint32_t b = 2u * uint32_t(rank & 3);
  return b | (b + 1u) << 8;
}

__host__ __device__ constexpr SplitEntry split_entry(int side, int byte) {
  SplitEntry e{};
  const int c = __builtin_popcount(unsigned(byte));
  int rank = side ? 8 - c : 0;                       // rank of the byte's first kept value
  uint32_t idx = 0;
  for (int g = 0; g < 2; ++g) {
    const int nib = (byte >> (4 * g)) & 15;
    int p[4] = {0, 0, 0, 0}, k = 0;
    for (int b = 0; b < 4; ++b)
      if ((nib >> b) & 1) p[k++] = b;
    // pairs as (rank of the value at the lower position, at the higher), -1 = zero; the
    // positions stay distinct and ascending
    int a0 = -1, a1 = -1, b0 = -1, b1 = -1, ca = 0x4, cb = 0x4;
    if (k >= 2) { a0 = rank; a1 = rank + 1; ca = p[0] | p[1] << 2; }
    else if (k == 1) {
      if (p[0] < 3) { a0 = rank; ca = p[0] | 3 << 2; } else { a1 = rank; ca = 2 | 3 << 2; }
    }
    if (k == 4) { b0 = rank + 2; b1 = rank + 3; cb = 2 | 3 << 2; }
    else if (k == 3) {
      if (p[2] < 3) { b0 = rank + 2; cb = p[2] | 3 << 2; } else { b1 = rank + 2; cb = 2 | 3 << 2; }
    }
    e.sel[4 * g + 0] = split_half_sel(a0, false) | split_half_sel(a1, false) << 16;
    e.sel[4 * g + 1] = split_half_sel(a0, true) | split_half_sel(a1, true) << 16;
    e.sel[4 * g + 2] = split_half_sel(b0, false) | split_half_sel(b1, false) << 16;
    e.sel[4 * g + 3] = split_half_sel(b0, true) | split_half_sel(b1, true) << 16;
    idx |= uint32_t(ca) << (4 * g) | uint32_t(cb) << (8 + 4 * g);
    rank += k;
  }
  e.idx = idx;
  return e;
}

// The tables as laid out in LDS (17 KiB): entry e's selectors at 32 e, its codes at
// kSplitSelBytes + 2 e. Built at compile time; each workgroup copies them to LDS once.
struct SplitTable {
  uint4 sel[2 * kSplitEntries];
  uint16_t idx[kSplitEntries];
};
static_assert(sizeof(SplitTable) == kSplitLutBytes, "split table layout");

__host__ __device__ constexpr SplitTable make_split_table() {
  SplitTable t{};
  for (int e = 0; e < kSplitEntries; ++e) {
    const SplitEntry x = split_entry(e >> 8, e & 255);
    t.sel[2 * e] = uint4{x.sel[0], x.sel[1], x.sel[2], x.sel[3]};
    t.sel[2 * e + 1] = uint4{x.sel[4], x.sel[5], x.sel[6], x.sel[7]};
    t.idx[e] = uint16_t(x.idx);
  }
  return t;
}

__device__ const SplitTable kSplitTable = make_split_table();

// ---- 16:32 on the dense matrix instruction (expanded fragments) ----
// A 16:32 word keeps 16 values anywhere in its 32 columns, so no fixed share of them lands in
// a lane's columns and no 2:4 split fits. The dense 16 x 16 x 32 instruction takes the word
// as it is: lane (row, q) supplies the 8 dense halves of columns 8q .. 8q+7, i.e. mask byte q.
// Its kept values are the word's packed values pc .. pc+c-1 (pc the bit count of the word
// below byte q, c the byte's): the lane reads the 8 halves from pc on into 4 dwords w0..w3,
// and a table indexed by the mask byte gives, per output dword (columns 2d, 2d+1), two
// v_perm_b32 byte selectors, one over w0:w1 and one over w2:w3, whose results are ORed:
// the value of rank r = (bits of the byte below column j) for a set bit j, a zero byte pair
// for a clear one. Selector byte 0x0C gives a zero byte.
constexpr int kExpandEntries = 256;
constexpr uint32_t kExpandBytes = kExpandEntries * 32;

// selector bytes placing half `rank` of the 8-half window (-1: zero) in one output half,
// for the perm over w0:w1 when !high (halves 0..3), over w2:w3 when high (halves 4..7)
__host__ __device__ constexpr uint32_t expand_half_sel(int rank, bool high) {
  if (rank < 0 || (rank >= 4) != high) return 0x0C0Cu;
  const uint32_t b = 2u * uint32_t(rank & 3);
  return b | (b + 1u) << 8;
}

struct ExpandTable {
  uint4 sel[2 * kExpandEntries];   // entry b: sel[2b] = (lo0, hi0, lo1, hi1), sel[2b+1] = (lo2, hi2, lo3, hi3)
};
static_assert(sizeof(ExpandTable) == kExpandBytes, "expand table layout");

__host__ __device__ constexpr ExpandTable make_expand_table() {
  ExpandTable t{};
  for (int b = 0; b < kExpandEntries; ++b) {
    uint32_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int rank = 0;
    int r[8] = {-1, -1, -1, -1, -1, -1, -1, -1};
    for (int j = 0; j < 8; ++j)
      if ((b >> j) & 1) r[j] = rank++;
    for (int d = 0; d < 4; ++d) {
      v[2 * d] = expand_half_sel(r[2 * d], false) | expand_half_sel(r[2 * d + 1], false) << 16;
      v[2 * d + 1] = expand_half_sel(r[2 * d], true) | expand_half_sel(r[2 * d + 1], true) << 16;
    }
    t.sel[2 * b] = uint4{v[0], v[1], v[2], v[3]};
    t.sel[2 * b + 1] = uint4{v[4], v[5], v[6], v[7]};
  }
  return t;
}

__device__ const ExpandTable kExpandTable = make_expand_table();

// Buffer loads: a resource spans one workgroup's slice of an operand and the hardware
// returns zero for offsets at or past its end, so lanes with nothing to load (tokens or
// rows past the end, columns past the row) take kOutOfRange instead of a branch.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, raw (untyped) access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcWord3);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
  const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u2_t __attribute__((ext_vector_type(2)));
  const u2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Partial tiles of column splits cross workgroups on different XCDs, whose L2 caches are
// not coherent with each other: buffer accesses with the SC1 cache-policy bit are (the form
// the compiler gives device-scope atomic loads and stores), so no fence has to write back or
// invalidate a whole L2.
constexpr int kCoherentAux = 16;   // SC1

__device__ __forceinline__ void coherent_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
  const u4_t u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, off, 0, kCoherentAux);
}

__device__ __forceinline__ float4 coherent_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
  const u4_t u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentAux);
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}

// LDS byte offset of 16-byte chunk c of token t in an X buffer with rb bytes per token:
// the low 3 bits of the chunk index are XORed with the token's, so the 8 tokens one
// fragment read touches at a time land on 8 different 16-byte bank groups.
template <int RB>
__device__ __forceinline__ uint32_t x_offset(int t, int c) { return uint32_t(t * RB + ((c ^ (t & 7)) << 4)); }

__device__ __forceinline__ uint4 lds_read16(const char* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

// The X chunks this thread stages: chunk k = tid + kThreads * j is token k / (KS / 8),
// column chunk k % (KS / 8) of the step. Tokens past the end and columns past the row
// read as zero.
template <int TR, int TT, int KS>
struct XStager {
  using T = Tile<TR, TT, KS>;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[T::kXPerThread];  // byte offset of the chunk in step 0
  int col[T::kXPerThread];
  uint32_t dst[T::kXPerThread];

  __device__ __forceinline__ void init(const uint16_t* __restrict__ X, int tokens, int cols, int t0, int tid) {
    rsrc = make_rsrc(X + size_t(t0) * unsigned(cols), int64_t(min(T::kTokens, tokens - t0)) * cols * 2);
#pragma unroll
    for (int j = 0; j < T::kXPerThread; ++j) {
      const int k = tid + kThreads * j;
      const int t = k / (KS / 8), c = k % (KS / 8);
      col[j] = 8 * c;
      off[j] = uint32_t(t) * uint32_t(cols) * 2u + uint32_t(16 * c);
      dst[j] = x_offset<T::kRowBytes>(t, c);
    }
  }
  __device__ __forceinline__ void load(uint4 (&r)[T::kXPerThread], int c0, int cols) const {
#pragma unroll
    for (int j = 0; j < T::kXPerThread; ++j)
      r[j] = buf_load16(rsrc, c0 + col[j] < cols ? off[j] + 2u * uint32_t(c0) : kOutOfRange);
  }
  __device__ __forceinline__ void store(const uint4 (&r)[T::kXPerThread], char* buf) const {
#pragma unroll
    for (int j = 0; j < T::kXPerThread; ++j) *reinterpret_cast<uint4*>(buf + dst[j]) = r[j];
  }
};

// Output tile of a workgroup. Workgroups go to the 8 XCDs in turn (workgroup b to XCD
// b % 8), each XCD with its own L2, so workgroup b is given tile L: the tiles are cut into
// 8 contiguous runs, one per XCD, and ordered in bands of kGroup row tiles (token tile
// outer, row tile inner within a band) so that a run is a compact block of row tiles x
// token tiles whose weight and X slices the XCD's L2 serves to all of them. Workgroups
// past the last multiple of 8 keep their own index.
constexpr int kGroup = 8;

struct TileCoord {
  int rx, ty;
};

__host__ __device__ __forceinline__ TileCoord tile_of(int b, int nrx, int nty) {
  const int nwg = nrx * nty;
  const int full = nwg - nwg % 8;
  const int L = b < full ? (b % 8) * (full / 8) + b / 8 : b;
  const int band = L / (kGroup * nty);
  const int gh = min(kGroup, nrx - band * kGroup);
  const int idx = L - band * kGroup * nty;
  return {band * kGroup + idx % gh, idx / gh};
}

// Writes one 16 x 16 output tile's lane share: 4 consecutive rows of one token.
__device__ __forceinline__ void store_tile(const f4_t& d, uint16_t* __restrict__ Y, int rows, int tokens, int row,
                                           int tok, bool vec) {
  if (tok >= tokens || row >= rows) return;
  uint16_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(d[e]));
  uint16_t* out = Y + size_t(tok) * unsigned(rows) + unsigned(row);
  if (vec && row + 4 <= rows) {
    *reinterpret_cast<uint2*>(out) = make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (row + e < rows) out[e] = h[e];
  }
}

template <int TR, int TT>
__device__ __forceinline__ void zero(f4_t (&acc)[TR][TT]) {
#pragma unroll
  for (int a = 0; a < TR; ++a)
#pragma unroll
    for (int b = 0; b < TT; ++b) acc[a][b] = f4_t{0.f, 0.f, 0.f, 0.f};
}

template <int TR, int TT>
__device__ __forceinline__ void store_all(const f4_t (&acc)[TR][TT], uint16_t* __restrict__ Y, int rows, int tokens,
                                          int r0, int t0, int lane) {
  const int q = lane >> 4, li = lane & 15;
  const bool vec = (rows & 3) == 0 && (reinterpret_cast<uintptr_t>(Y) & 7) == 0;
#pragma unroll
  for (int a = 0; a < TR; ++a)
#pragma unroll
    for (int b = 0; b < TT; ++b) store_tile(acc[a][b], Y, rows, tokens, r0 + 16 * a + 4 * q, t0 + 16 * b + li, vec);
}

// The workgroup's output tile written as whole lines: each lane's 16 x 16 tiles leave 4 rows
// of one token (8 bytes), so a direct store touches 16 tokens x 8 bytes per row tile and the
// memory writes a line several times. Instead the tile (kRows rows x kTokens tokens) goes
// through LDS (the X buffers, free after the main loop) in P = ceil(TR / 2) passes of
// kTokens / P tokens, each token's kRows fp16 in 16-byte chunks XOR-swizzled by its low 3
// bits, and leaves in 16-byte stores of 8 consecutive rows of one token, consecutive lanes
// covering a token's rows. Needs rows % 8 == 0 and a 16-byte aligned Y (store_all else).
template <int TR, int TT, int KS>
__device__ __forceinline__ void store_lines(const f4_t (&acc)[TR][TT], uint16_t* __restrict__ Y, int rows,
                                            int tokens, int wg_r0, int t0, int wave, int lane, char* buf) {
  using T = Tile<TR, TT, KS>;
  constexpr int P = (TR + 1) / 2;
  constexpr int kPassTok = T::kTokens / P;
  constexpr int kTokBytes = T::kRows * 2;
  constexpr int kChunks = kTokBytes / 16;
  constexpr int kPassChunks = kPassTok * kChunks;
  static_assert(kPassTok % 16 == 0 && kChunks % 8 == 0, "whole token tiles and swizzle groups per pass");
  static_assert(kPassTok * kTokBytes <= 2 * T::kXBytes, "a pass fits in the two X buffers");
  static_assert(kPassChunks % kThreads == 0, "the chunks of a pass split evenly over the workgroup");
  const int q = lane >> 4, li = lane & 15;
  const int tid = threadIdx.x;
  __syncthreads();   // every wave's last reads of the X buffers are done
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int b = 0; b < TT; ++b) {
      if (16 * b < p * kPassTok || 16 * b >= (p + 1) * kPassTok) continue;
      const int tl = 16 * b + li - p * kPassTok;
#pragma unroll
      for (int a = 0; a < TR; ++a) {
        const int rl = wave * 16 * TR + 16 * a + 4 * q;
        const uint32_t off = uint32_t(tl * kTokBytes + (((rl >> 3) ^ (tl & 7)) << 4) + 8 * ((rl >> 2) & 1));
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[a][b][e]));
        *reinterpret_cast<uint2*>(buf + off) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPassChunks / kThreads; ++j) {
      const int k = tid + kThreads * j;
      const int tl = k / kChunks, c = k % kChunks;
      const int tok = t0 + p * kPassTok + tl, row = wg_r0 + 8 * c;
      const uint4 v = *reinterpret_cast<const uint4*>(buf + tl * kTokBytes + ((c ^ (tl & 7)) << 4));
      if (tok < tokens && row < rows)   // rows % 8 == 0: a chunk's 8 rows are all in or all out
        *reinterpret_cast<uint4*>(Y + size_t(tok) * unsigned(rows) + unsigned(row)) = v;
    }
    if (p + 1 < P) __syncthreads();
  }
}

template <int TR, int TT, int KS>
__device__ __forceinline__ void store_out(const f4_t (&acc)[TR][TT], uint16_t* __restrict__ Y, int rows,
                                          int tokens, int wg_r0, int t0, int wave, int lane, char* buf) {
  if ((rows & 7) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0)
    store_lines<TR, TT, KS>(acc, Y, rows, tokens, wg_r0, t0, wave, lane, buf);
  else
    store_all(acc, Y, rows, tokens, wg_r0 + wave * 16 * TR, t0, lane);
}

// Weight values of one step for the sparse product: per row tile and 64-column sub-step,
// this lane's 8 kept values. (The mask words travel separately, a block of steps at a time.)
template <int TR, int SUB>
struct SparseA {
  uint4 v[TR][SUB];
};

// Weight fragments of one step for the dense product: per row tile and 32-column slice.
template <int TR, int SUB>
struct DenseA {
  uint4 v[TR][2 * SUB];
};

// The dense product's main loop. X goes global -> registers -> LDS (two buffers), weights
// global -> registers, D steps ahead. Step s: barrier; write X of step s + 1 (its loads were
// issued D - 1 steps earlier) into buffer (s + 1) & 1, last read in step s - 1, which every
// wave has finished by the barrier; take this step's weight set; issue the loads of step
// s + D into the freed register sets; compute on buffer s & 1. Steps are unrolled D at a
// time so every register set has a fixed name; the steps past the last one (up to D - 1)
// skip only the math, and their loads repeat the last step, so the loads and waits stay
// the same in every step.
template <int TR, int TT, int KS, int D, typename AFrag, typename LoadA, typename Compute>
__device__ __forceinline__ void dense_main_loop(const XStager<TR, TT, KS>& xst,
                                                char (*xs)[Tile<TR, TT, KS>::kXBytes], int cols, LoadA load_a,
                                                Compute compute) {
  using T = Tile<TR, TT, KS>;
  const int steps = (cols + KS - 1) / KS;
  const int last = (steps - 1) * KS;
  uint4 xr[D][T::kXPerThread];
  AFrag af[D];
#pragma unroll
  for (int p = 0; p < D; ++p) {
    const int c = min(p * KS, last);
    xst.load(xr[p], c, cols);
    load_a(af[p], c);
  }
  xst.store(xr[0], xs[0]);
  for (int s0 = 0; s0 < steps; s0 += D) {
#pragma unroll
    for (int p = 0; p < D; ++p) {
      const int s = s0 + p;
      __syncthreads();
      xst.store(xr[(p + 1) % D], xs[(s + 1) & 1]);
      const AFrag cur = af[p];
      const int cn = min((s + D) * KS, last);
      xst.load(xr[p], cn, cols);
      load_a(af[p], cn);
      if (s < steps) compute(cur, xs[s & 1]);
    }
  }
}

// Calls f(integral_constant<int, P>) for P = P0 .. U - 1, in order.
template <int P0, int U, typename F>
__device__ __forceinline__ void unroll_slots(F& f) {
  if constexpr (P0 < U) {
    f(std::integral_constant<int, P0>());
    unroll_slots<P0 + 1, U>(f);
  }
}

// The sparse product's main loop over columns c_beg .. c_end - 1 (c_beg a multiple of U *
// KS, so that step s of the range is step s of its mask block): the dense one's schedule,
// unrolled U steps at a time (U a multiple of D) so that every slot of a mask block has a
// fixed name, with a hook per slot (run after the slot's loads are issued) for the
// mask-block loads, and a stage callback run once after the first loads are issued (LDS
// writes of data loaded before them). Steps past the last one (up to U - 1) skip only the
// math.
template <int TR, int TT, int KS, int D, int U, typename AFrag, typename LoadA, typename Hook, typename Compute,
          typename Stage>
__device__ __forceinline__ void sparse_main_loop(const XStager<TR, TT, KS>& xst,
                                                 char (*xs)[Tile<TR, TT, KS>::kXBytes], int cols, int c_beg,
                                                 int c_end, LoadA load_a, Hook hook, Compute compute, Stage stage) {
  static_assert(U % D == 0, "unroll must be a multiple of the load depth");
  using T = Tile<TR, TT, KS>;
  const int steps = (c_end - c_beg + KS - 1) / KS;
  const int last = c_beg + (steps - 1) * KS;
  uint4 xr[D][T::kXPerThread];
  AFrag af[D];
#pragma unroll
  for (int p = 0; p < D; ++p) {
    const int c = min(c_beg + p * KS, last);
    xst.load(xr[p], c, cols);
    load_a(af[p], c);
  }
  stage();
  xst.store(xr[0], xs[0]);
  for (int s0 = 0; s0 < steps; s0 += U) {
    auto slot = [&](auto pc) {
      constexpr int P = decltype(pc)::value;
      const int s = s0 + P;
      __syncthreads();
      xst.store(xr[(P + 1) % D], xs[(s + 1) & 1]);
      const AFrag cur = af[P % D];
      const int cn = min(c_beg + (s + D) * KS, last);
      xst.load(xr[P % D], cn, cols);
      load_a(af[P % D], cn);
      hook(pc, s0);
      if (s < steps) compute(cur, xs[s & 1], pc);
    };
    unroll_slots<0, U>(slot);
  }
}

// ---- column splits (mid-size batches) ----
// With a few hundred tokens or fewer the grid of output tiles leaves most CUs idle while each
// workgroup walks every column in turn, so the columns of a tile can go to `splits`
// consecutive workgroups, each taking whole blocks of kColBlock columns (one block of mask
// words per row). Each leaves its fp32 partial tile in part (per tile, per split, one float4
// per lane and 16 x 16 tile: kThreads * TR * TT float4) and counts itself in cnt[tile]; the
// last to arrive sums the partials in split order (the same order whichever arrives last),
// resets the count to zero and stores the tile. Consecutive workgroups land on different
// XCDs, so with 8 splits each XCD takes one column range of every tile and its L2 serves that
// range of X to all of them.
constexpr int kColBlock = 512;
constexpr int kMaxColSplits = 8;

// Partial tiles the last workgroup of a tile loads at once in the hand-off (split_handoff): 32
// float4 per lane in flight, so all 8 of a 64 x 64 tile at once, 2 at a time for 128 x 128 and
// one at a time for 256 x 128 (tiles = 16 x 16 output tiles per wave, TR * TT). Two at a time
// for 256 x 128 (64 float4 per lane; the kernel runs one wave per SIMD anyway) measured within
// +-3% of one.
constexpr int handoff_slots(int tiles) {
  return tiles >= 32 ? 1 : (32 / tiles < kMaxColSplits ? 32 / tiles : kMaxColSplits);
}

struct ColSplit {
  float4* part;
  unsigned* cnt;
  int splits, tile, split;
  unsigned* flag;   // one LDS word: the count this workgroup's arrival saw
};

// Hands the partial tile over; true in the workgroup that then holds the tile's sum in acc.
template <int TR, int TT>
__device__ __forceinline__ bool split_handoff(f4_t (&acc)[TR][TT], const ColSplit& cs) {
  constexpr int kPer = kThreads * TR * TT;   // float4 per partial tile
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t pr =
      make_rsrc(cs.part + size_t(cs.tile) * unsigned(cs.splits) * unsigned(kPer), int64_t(cs.splits) * kPer * 16);
#pragma unroll
  for (int a = 0; a < TR; ++a)
#pragma unroll
    for (int b = 0; b < TT; ++b)
      coherent_store16(pr, uint32_t((cs.split * TR * TT + a * TT + b) * kThreads + tid) * 16u,
                       make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]));
  // every wave's partial has reached the device's coherence point before the count moves
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) *cs.flag = atomicAdd(cs.cnt + cs.tile, 1u);
  __syncthreads();
  if (*cs.flag != unsigned(cs.splits - 1)) return false;
  // the tile's last workgroup: every split's partial is complete. The partials are loaded R
  // splits at a time (one memory round trip per R) and summed in split order; slots past the
  // last split are outside the resource and read zero, and adding zero after the last split
  // leaves the sum as it is.
  constexpr int R = handoff_slots(TR * TT);
  zero(acc);
  for (int k0 = 0; k0 < cs.splits; k0 += R) {
    float4 v[R][TR][TT];
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
      for (int a = 0; a < TR; ++a)
#pragma unroll
        for (int b = 0; b < TT; ++b)
          v[k][a][b] = coherent_load16(pr, uint32_t(((k0 + k) * TR * TT + a * TT + b) * kThreads + tid) * 16u);
#pragma unroll
    for (int k = 0; k < R; ++k) {
#pragma unroll
      for (int a = 0; a < TR; ++a)
#pragma unroll
        for (int b = 0; b < TT; ++b) {
          acc[a][b][0] += v[k][a][b].x;
          acc[a][b][1] += v[k][a][b].y;
          acc[a][b][2] += v[k][a][b].z;
          acc[a][b][3] += v[k][a][b].w;
        }
    }
  }
  if (tid == 0) atomicExch(cs.cnt + cs.tile, 0u);
  return true;
}

// How the sparse body turns a lane's packed values and mask bits into matrix operands:
// 2:4 directly on the sparse instruction; 4:8 and 8:16 split into two 2:4 operands (the
// split tables); 16:32 expanded to dense fragments for the dense instruction (the expansion
// table), one per 32-column word.
constexpr int kPfDirect = 0, kPfSplit = 1, kPfExpand = 2;
// EXPAND: LDS bytes of one wave's value area per row tile: the step's values of its 16 rows
// (64 bytes each) and room for a window read past the last row's second word
constexpr uint32_t kPfAreaBytes = 16 * 64 + 64;

// The sparse products: values [rows][cols / 2] fp16, masks [rows][cols / 32]; MODE as above
// (lut: the pattern's table in LDS; area: EXPAND's per-wave value areas, TR per wave).
// COLS: one of a tile's column splits (columns c_beg .. c_end - 1; the hand-off to the
// tile's last workgroup in split_handoff), else the whole row (c_beg = 0, c_end = cols).
template <int TR, int TT, int KS, int D, int MODE, bool COLS>
__device__ __forceinline__ void prefill_sparse_body(const uint16_t* __restrict__ values,
                                                    const uint32_t* __restrict__ masks,
                                                    const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                    int rows, int cols, int tokens,
                                                    char (*xs)[Tile<TR, TT, KS>::kXBytes], char* lut, char* area,
                                                    TileCoord tc, int c_beg, int c_end, const ColSplit& cs) {
  constexpr bool SPLIT = MODE == kPfSplit, EXPAND = MODE == kPfExpand;
  using T = Tile<TR, TT, KS>;
  constexpr int SUB = T::kSub;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, li = lane & 15;
  const int r0 = tc.rx * T::kRows + wave * 16 * TR;
  const int t0 = tc.ty * T::kTokens;
  const int words = cols >> 5;

  // SPLIT, EXPAND: this thread's 16-byte chunks of the pattern's table, loaded before
  // anything else and written to LDS with the first X chunks (the wait for those covers them)
  constexpr int kLutChunks = int((EXPAND ? kExpandBytes : kSplitLutBytes) / 16);
  constexpr int kLutPer = SPLIT || EXPAND ? (kLutChunks + kThreads - 1) / kThreads : 1;
  uint4 lreg[kLutPer];
  if constexpr (SPLIT || EXPAND) {
    const uint4* tab = EXPAND ? reinterpret_cast<const uint4*>(&kExpandTable)
                              : reinterpret_cast<const uint4*>(&kSplitTable);
#pragma unroll
    for (int j = 0; j < kLutPer; ++j) lreg[j] = tab[min(tid + kThreads * j, kLutChunks - 1)];
  }
  auto stage = [&] {
    if constexpr (SPLIT || EXPAND) {
#pragma unroll
      for (int j = 0; j < kLutPer; ++j)
        if (tid + kThreads * j < kLutChunks) reinterpret_cast<uint4*>(lut)[tid + kThreads * j] = lreg[j];
    }
  };

  XStager<TR, TT, KS> xst;
  xst.init(X, tokens, cols, t0, tid);

  // weight slices of the workgroup's rows; this lane's row in tile a is 16 a + li of its wave
  const int wg_rows = min(T::kRows, rows - tc.rx * T::kRows);
  const size_t wg_r0 = size_t(tc.rx) * T::kRows;
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(values + wg_r0 * unsigned(cols >> 1), int64_t(wg_rows) * cols);
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(masks + wg_r0 * unsigned(words), int64_t(wg_rows) * words * 4);
  uint32_t voff[TR], moff[TR];
#pragma unroll
  for (int a = 0; a < TR; ++a) {
    const uint32_t rl = uint32_t(wave * 16 * TR + 16 * a + li);
    voff[a] = rl * uint32_t(cols) + 16u * uint32_t(q);          // values 8q.. of the step
    moff[a] = rl * uint32_t(words) * 4u + 16u * uint32_t(q);     // mask words 4q .. 4q + 3 of a block
  }
  const int qcol = 32 * (q >> 1);  // first column of this lane's mask word in a sub-step
  const int mshift = 16 * (q & 1);
  using AF = SparseA<TR, SUB>;
  auto load_a = [&](AF& f, int c0) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int c = c0 + 64 * u;
      const bool ok = c + qcol < cols;
#pragma unroll
      for (int a = 0; a < TR; ++a) f.v[a][u] = buf_load16(vr, ok ? voff[a] + uint32_t(c) : kOutOfRange);
    }
  };

  // Mask words, a block of kMaskSteps 64-column steps (2 kMaskSteps words of each row) at
  // a time: lane q of row li holds words 4q .. 4q + 3 of the block (one 16-byte load per
  // row tile per block instead of one 4-byte load per step; a load touches the same 16
  // rows either way, so fewer, wider loads cost less). At step j of the block the lane
  // needs word 2j + (q >> 1), which lane li + 16 (j / 2) holds as its word 2 (j % 2) +
  // (q >> 1); a cross-lane permute fetches it. The block for the next steps is loaded
  // kMaskSteps - D steps into the current one, D steps ahead like the values.
  constexpr int kMaskSteps = 8;
  static_assert(KS == 64, "mask blocks are laid out for 64-column steps");
  static_assert(kMaskSteps * KS == kColBlock, "column splits cover whole mask blocks");
  const int steps = (c_end - c_beg + KS - 1) / KS;
  const int first_block = c_beg / kColBlock, last_block = (steps - 1) / kMaskSteps;
  uint4 mcur[TR], mnext[TR];
  auto load_masks = [&](int blk) {   // blk counts from the range's first block
#pragma unroll
    for (int a = 0; a < TR; ++a)
      mnext[a] = buf_load16(mr, moff[a] + uint32_t(64 * (first_block + min(blk, last_block))));
  };
  load_masks(0);
  auto hook = [&](auto pc, int s0) {
    constexpr int P = decltype(pc)::value;
    if constexpr (P == 0) {   // 2:4: the position codes of the block's words, once per block
#pragma unroll
      for (int a = 0; a < TR; ++a)
        mcur[a] = SPLIT || EXPAND
                      ? mnext[a]
                      : make_uint4(pair_codes32(mnext[a].x), pair_codes32(mnext[a].y), pair_codes32(mnext[a].z),
                                   pair_codes32(mnext[a].w));
    }
    if constexpr (P == kMaskSteps - D) load_masks(s0 / kMaskSteps + 1);
  };

  f4_t acc[TR][TT];
  zero(acc);
  // X fragment of token 16 b + li: column chunks q and 4 + q of the step
  const uint32_t b_lo = x_offset<T::kRowBytes>(li, q), b_hi = x_offset<T::kRowBytes>(li, 4 + q);
  // EXPAND: this wave's value areas (row tile a at a * kPfAreaBytes)
  char* const warea = EXPAND ? area + uint32_t(wave) * TR * kPfAreaBytes : nullptr;
  auto compute_expand = [&](const AF& f, const char* buf, auto pc) {
    constexpr int J = decltype(pc)::value;
    const int src = 4 * (li + 16 * (J >> 1));
    // the step's values of the wave's rows to its areas (row li at 64 li: word 0's 16 values,
    // then word 1's; lane q's 16 bytes at 16 q), visible to the wave's other lanes before
    // they read them back
#pragma unroll
    for (int a = 0; a < TR; ++a) *reinterpret_cast<uint4*>(warea + a * kPfAreaBytes + 64 * li + 16 * q) = f.v[a][0];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane (q, li): the dense halves of columns 8q .. 8q+7 of each word of row li: the 8
    // halves from its mask byte's first kept value on, placed by the expansion table
    uint4 dense[TR][2];
#pragma unroll
    for (int a = 0; a < TR; ++a) {
      const uint32_t w0 = uint32_t(__builtin_amdgcn_ds_bpermute(src, int((J & 1) ? mcur[a].z : mcur[a].x)));
      const uint32_t w1 = uint32_t(__builtin_amdgcn_ds_bpermute(src, int((J & 1) ? mcur[a].w : mcur[a].y)));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t wi = i ? w1 : w0;
        const uint32_t byte = __builtin_amdgcn_ubfe(wi, 8u * uint32_t(q), 8);
        // first kept value of the byte among the word's 16 (clamped: any mask keeps the
        // window inside the areas)
        const uint32_t first = min(uint32_t(__builtin_popcount(wi & ((1u << (8 * q)) - 1u))), 16u);
        const uint32_t off = uint32_t(a) * kPfAreaBytes + 64u * uint32_t(li) + 32u * uint32_t(i) + 2u * first;
        const uint32_t* wd = reinterpret_cast<const uint32_t*>(warea + (off & ~3u));
        const uint32_t sh = (off & 2u) * 8u;   // 16 when the window starts mid-dword
        const uint32_t r0 = wd[0], r1 = wd[1], r2 = wd[2], r3 = wd[3], r4 = wd[4];
        const uint32_t v0 = __builtin_amdgcn_alignbit(r1, r0, sh), v1 = __builtin_amdgcn_alignbit(r2, r1, sh);
        const uint32_t v2 = __builtin_amdgcn_alignbit(r3, r2, sh), v3 = __builtin_amdgcn_alignbit(r4, r3, sh);
        const uint4 s0 = *reinterpret_cast<const uint4*>(lut + 32u * byte);
        const uint4 s1 = *reinterpret_cast<const uint4*>(lut + 32u * byte + 16u);
        auto pick = [&](uint32_t lo_sel, uint32_t hi_sel) {
          return __builtin_amdgcn_perm(v1, v0, lo_sel) | __builtin_amdgcn_perm(v3, v2, hi_sel);
        };
        dense[a][i] = make_uint4(pick(s0.x, s0.y), pick(s0.z, s0.w), pick(s1.x, s1.y), pick(s1.z, s1.w));
      }
    }
    // every lane has read the areas before the next step writes them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // X fragments (chunks q and 4 + q: the columns of word 0, word 1), one token tile ahead
    uint4 lo[2], hi[2];
    lo[0] = lds_read16(buf, b_lo);
    hi[0] = lds_read16(buf, b_hi);
#pragma unroll
    for (int b = 0; b < TT; ++b) {
      if (b + 1 < TT) {
        const char* tb = buf + (b + 1) * 16 * T::kRowBytes;
        lo[(b + 1) & 1] = lds_read16(tb, b_lo);
        hi[(b + 1) & 1] = lds_read16(tb, b_hi);
      }
#pragma unroll
      for (int a = 0; a < TR; ++a) {
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, dense[a][0]),
                                                           __builtin_bit_cast(h8_t, lo[b & 1]), acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, dense[a][1]),
                                                           __builtin_bit_cast(h8_t, hi[b & 1]), acc[a][b], 0, 0, 0);
      }
    }
  };
  auto compute_sparse = [&](const AF& f, const char* buf, auto pc) {
    constexpr int J = decltype(pc)::value;           // step within the mask block
    const int src = 4 * (li + 16 * (J >> 1));        // byte address of lane li + 16 (J / 2)
    h8_t av[TR], bv[SPLIT ? TR : 1];
    int idx[TR], idb[SPLIT ? TR : 1];
#pragma unroll
    for (int a = 0; a < TR; ++a) {
      const uint32_t w0 = uint32_t(__builtin_amdgcn_ds_bpermute(src, int((J & 1) ? mcur[a].z : mcur[a].x)));
      const uint32_t w1 = uint32_t(__builtin_amdgcn_ds_bpermute(src, int((J & 1) ? mcur[a].w : mcur[a].y)));
      const uint32_t m16 = __builtin_amdgcn_ubfe((q >> 1) ? w1 : w0, uint32_t(mshift), 16);
      if constexpr (SPLIT) {
        // the lane's 16 mask bits select the table entries of its two bytes
        const uint32_t e0 = 32u * (m16 & 0xFFu), e1 = 32u * (256u + (m16 >> 8));
        const uint4 s0 = *reinterpret_cast<const uint4*>(lut + e0);
        const uint4 s1 = *reinterpret_cast<const uint4*>(lut + e0 + 16);
        const uint4 s2 = *reinterpret_cast<const uint4*>(lut + e1);
        const uint4 s3 = *reinterpret_cast<const uint4*>(lut + e1 + 16);
        const uint16_t* codes = reinterpret_cast<const uint16_t*>(lut + kSplitSelBytes);
        const uint32_t i0 = codes[m16 & 0xFFu], i1 = codes[256u + (m16 >> 8)];
        const uint4 v = f.v[a][0];
        auto pick = [&](uint32_t lo_sel, uint32_t hi_sel) {
          return __builtin_amdgcn_perm(v.y, v.x, lo_sel) | __builtin_amdgcn_perm(v.w, v.z, hi_sel);
        };
        av[a] = __builtin_bit_cast(
            h8_t, make_uint4(pick(s0.x, s0.y), pick(s1.x, s1.y), pick(s2.x, s2.y), pick(s3.x, s3.y)));
        bv[a] = __builtin_bit_cast(
            h8_t, make_uint4(pick(s0.z, s0.w), pick(s1.z, s1.w), pick(s2.z, s2.w), pick(s3.z, s3.w)));
        idx[a] = int(__builtin_amdgcn_perm(i1, i0, 0x0C0C0400u));   // A codes of groups 0..3
        idb[a] = int(__builtin_amdgcn_perm(i1, i0, 0x0C0C0501u));   // B codes
      } else {
        av[a] = __builtin_bit_cast(h8_t, f.v[a][0]);
        idx[a] = int(m16);
      }
    }
    // X fragments are read one token tile ahead of the math that uses them
    uint4 lo[2], hi[2];
    lo[0] = lds_read16(buf, b_lo);
    hi[0] = lds_read16(buf, b_hi);
#pragma unroll
    for (int b = 0; b < TT; ++b) {
      if (b + 1 < TT) {
        const char* tb = buf + (b + 1) * 16 * T::kRowBytes;
        lo[(b + 1) & 1] = lds_read16(tb, b_lo);
        hi[(b + 1) & 1] = lds_read16(tb, b_hi);
      }
      const uint4 l = lo[b & 1], h = hi[b & 1];
      const u8_t xv = {l.x, l.y, l.z, l.w, h.x, h.y, h.z, h.w};
      const h16_t bf = __builtin_bit_cast(h16_t, xv);
#pragma unroll
      for (int a = 0; a < TR; ++a) {
        acc[a][b] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(av[a], bf, acc[a][b], idx[a], 0, 0);
        if constexpr (SPLIT) acc[a][b] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(bv[a], bf, acc[a][b], idb[a], 0, 0);
      }
    }
  };
  auto compute = [&](const AF& f, const char* buf, auto pc) {
    if constexpr (EXPAND)
      compute_expand(f, buf, pc);
    else
      compute_sparse(f, buf, pc);
  };
  sparse_main_loop<TR, TT, KS, D, kMaskSteps, AF>(xst, xs, cols, c_beg, c_end, load_a, hook, compute, stage);
  if constexpr (COLS) {
    if (!split_handoff<TR, TT>(acc, cs)) return;
  }
  // (the split kernels keep the direct stores: with the staged ones their 256 x 256 tile
  // measured 8% slower on 14336 x 4096 x 2048, the 2:4 and dense kernels 2-6% faster)
  if constexpr (SPLIT)
    store_all(acc, Y, rows, tokens, r0, t0, lane);
  else
    store_out<TR, TT, KS>(acc, Y, rows, tokens, tc.rx * T::kRows, t0, wave, lane, xs[0]);
}

// 2:4 sparse product.
template <int TR, int TT, int KS, int D>
__global__ __launch_bounds__(kThreads) void prefill_spmm_kernel(const uint16_t* __restrict__ values,
                                                                const uint32_t* __restrict__ masks,
                                                                const uint16_t* __restrict__ X,
                                                                uint16_t* __restrict__ Y, int rows, int cols,
                                                                int tokens) {
  using T = Tile<TR, TT, KS>;
  __shared__ __attribute__((aligned(16))) char xs[2][T::kXBytes];
  const TileCoord tc = tile_of(int(blockIdx.x), (rows + T::kRows - 1) / T::kRows, (tokens + T::kTokens - 1) / T::kTokens);
  prefill_sparse_body<TR, TT, KS, D, kPfDirect, false>(values, masks, X, Y, rows, cols, tokens, xs, nullptr, nullptr,
                                                       tc, 0, cols, ColSplit{});
}

// 4:8 and 8:16 sparse product (split operands).
template <int TR, int TT, int KS, int D>
__global__ __launch_bounds__(kThreads) void prefill_split_kernel(const uint16_t* __restrict__ values,
                                                                 const uint32_t* __restrict__ masks,
                                                                 const uint16_t* __restrict__ X,
                                                                 uint16_t* __restrict__ Y, int rows, int cols,
                                                                 int tokens) {
  using T = Tile<TR, TT, KS>;
  __shared__ __attribute__((aligned(16))) char xs[2][T::kXBytes];
  __shared__ __attribute__((aligned(16))) char lut[kSplitLutBytes];
  const TileCoord tc = tile_of(int(blockIdx.x), (rows + T::kRows - 1) / T::kRows, (tokens + T::kTokens - 1) / T::kTokens);
  prefill_sparse_body<TR, TT, KS, D, kPfSplit, false>(values, masks, X, Y, rows, cols, tokens, xs, lut, nullptr, tc, 0,
                                                      cols, ColSplit{});
}

// 16:32 sparse product (fragments expanded for the dense instruction).
template <int TR, int TT, int KS, int D>
__global__ __launch_bounds__(kThreads) void prefill_expand_kernel(const uint16_t* __restrict__ values,
                                                                  const uint32_t* __restrict__ masks,
                                                                  const uint16_t* __restrict__ X,
                                                                  uint16_t* __restrict__ Y, int rows, int cols,
                                                                  int tokens) {
  using T = Tile<TR, TT, KS>;
  __shared__ __attribute__((aligned(16))) char xs[2][T::kXBytes];
  __shared__ __attribute__((aligned(16))) char lut[kExpandBytes];
  __shared__ __attribute__((aligned(16))) char area[kWaves * TR * kPfAreaBytes];
  const TileCoord tc = tile_of(int(blockIdx.x), (rows + T::kRows - 1) / T::kRows, (tokens + T::kTokens - 1) / T::kTokens);
  prefill_sparse_body<TR, TT, KS, D, kPfExpand, false>(values, masks, X, Y, rows, cols, tokens, xs, lut, area, tc, 0,
                                                       cols, ColSplit{});
}

// Column-split sparse products (2:4 when !SPLIT, 4:8 and 8:16 when SPLIT): workgroup b takes
// split b % splits of tile b / splits (row tile fastest), columns [split, split + 1) *
// blocks * kColBlock of the row.
template <int TR, int TT, int KS, int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) void prefill_colsplit_kernel(const uint16_t* __restrict__ values,
                                                                    const uint32_t* __restrict__ masks,
                                                                    const uint16_t* __restrict__ X,
                                                                    uint16_t* __restrict__ Y, int rows, int cols,
                                                                    int tokens, int splits, int blocks,
                                                                    float4* __restrict__ part,
                                                                    unsigned* __restrict__ cnt) {
  using T = Tile<TR, TT, KS>;
  __shared__ __attribute__((aligned(16))) char xs[2][T::kXBytes];
  __shared__ __attribute__((aligned(16))) char lut[SPLIT ? kSplitLutBytes : 16];
  __shared__ unsigned flag;
  const int b = int(blockIdx.x);
  const int tile = b / splits, split = b - tile * splits;
  const int nrx = (rows + T::kRows - 1) / T::kRows;
  const TileCoord tc{tile % nrx, tile / nrx};
  const int c_beg = split * blocks * kColBlock;
  const int c_end = min(cols, c_beg + blocks * kColBlock);
  prefill_sparse_body<TR, TT, KS, D, SPLIT ? kPfSplit : kPfDirect, true>(
      values, masks, X, Y, rows, cols, tokens, xs, SPLIT ? lut : nullptr, nullptr, tc, c_beg, c_end,
      ColSplit{part, cnt, splits, tile, split, &flag});
}

// The column-split 16:32 product (expanded fragments), laid out as prefill_colsplit_kernel.
template <int TR, int TT, int KS, int D>
__global__ __launch_bounds__(kThreads) void prefill_colsplit_expand_kernel(const uint16_t* __restrict__ values,
                                                                           const uint32_t* __restrict__ masks,
                                                                           const uint16_t* __restrict__ X,
                                                                           uint16_t* __restrict__ Y, int rows,
                                                                           int cols, int tokens, int splits,
                                                                           int blocks, float4* __restrict__ part,
                                                                           unsigned* __restrict__ cnt) {
  using T = Tile<TR, TT, KS>;
  __shared__ __attribute__((aligned(16))) char xs[2][T::kXBytes];
  __shared__ __attribute__((aligned(16))) char lut[kExpandBytes];
  __shared__ __attribute__((aligned(16))) char area[kWaves * TR * kPfAreaBytes];
  __shared__ unsigned flag;
  const int b = int(blockIdx.x);
  const int tile = b / splits, split = b - tile * splits;
  const int nrx = (rows + T::kRows - 1) / T::kRows;
  const TileCoord tc{tile % nrx, tile / nrx};
  const int c_beg = split * blocks * kColBlock;
  const int c_end = min(cols, c_beg + blocks * kColBlock);
  prefill_sparse_body<TR, TT, KS, D, kPfExpand, true>(values, masks, X, Y, rows, cols, tokens, xs, lut, area, tc,
                                                      c_beg, c_end, ColSplit{part, cnt, splits, tile, split, &flag});
}

// Dense product: W [rows][cols] fp16.
template <int TR, int TT, int KS, int D>
__global__ __launch_bounds__(kThreads) void prefill_gemm_kernel(const uint16_t* __restrict__ W,
                                                                const uint16_t* __restrict__ X,
                                                                uint16_t* __restrict__ Y, int rows, int cols,
                                                                int tokens) {
  using T = Tile<TR, TT, KS>;
  constexpr int SUB = T::kSub;
  __shared__ __attribute__((aligned(16))) char xs[2][T::kXBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, li = lane & 15;
  const TileCoord tc = tile_of(int(blockIdx.x), (rows + T::kRows - 1) / T::kRows, (tokens + T::kTokens - 1) / T::kTokens);
  const int r0 = tc.rx * T::kRows + wave * 16 * TR;
  const int t0 = tc.ty * T::kTokens;

  XStager<TR, TT, KS> xst;
  xst.init(X, tokens, cols, t0, tid);

  const int wg_rows = min(T::kRows, rows - tc.rx * T::kRows);
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(W + size_t(tc.rx) * T::kRows * unsigned(cols), int64_t(wg_rows) * cols * 2);
  uint32_t woff[TR];
#pragma unroll
  for (int a = 0; a < TR; ++a)
    woff[a] = uint32_t(wave * 16 * TR + 16 * a + li) * uint32_t(cols) * 2u + 16u * uint32_t(q);
  using AF = DenseA<TR, SUB>;
  auto load_a = [&](AF& f, int c0) {
#pragma unroll
    for (int g = 0; g < 2 * SUB; ++g) {
      const int c = c0 + 32 * g;
#pragma unroll
      for (int a = 0; a < TR; ++a) f.v[a][g] = buf_load16(wr, c < cols ? woff[a] + 2u * uint32_t(c) : kOutOfRange);
    }
  };

  f4_t acc[TR][TT];
  zero(acc);
  uint32_t b_off[2 * SUB];
#pragma unroll
  for (int g = 0; g < 2 * SUB; ++g) b_off[g] = x_offset<T::kRowBytes>(li, 4 * g + q);
  auto compute = [&](const AF& f, const char* buf) {
#pragma unroll
    for (int g = 0; g < 2 * SUB; ++g) {
      // X fragments are read one token tile ahead of the math that uses them
      uint4 xf[2];
      xf[0] = lds_read16(buf, b_off[g]);
#pragma unroll
      for (int b = 0; b < TT; ++b) {
        if (b + 1 < TT) xf[(b + 1) & 1] = lds_read16(buf + (b + 1) * 16 * T::kRowBytes, b_off[g]);
        const h8_t bf = __builtin_bit_cast(h8_t, xf[b & 1]);
#pragma unroll
        for (int a = 0; a < TR; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, f.v[a][g]), bf, acc[a][b], 0, 0, 0);
        // scheduling hint: LDS reads and matrix instructions in alternating groups (two
        // reads, then the TR products of this token tile), measured faster for this kernel
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TR, 0);
      }
    }
  };
  dense_main_loop<TR, TT, KS, D, AF>(xst, xs, cols, load_a, compute);
  store_out<TR, TT, KS>(acc, Y, rows, tokens, tc.rx * T::kRows, t0, wave, lane, xs[0]);
}

}  // namespace prefill_detail
}  // namespace nm
