// Small-batch 50% products on the gfx950 matrix instructions: Y [tokens][rows] =
// X [tokens][cols] W'^T for 1 <= tokens <= 16, W' given as the packed values and bitmask
// (the batch side of the SpMV / SpMM split the news.bitwarelabs.com page draws in "What's
// new"; bitmask format of the aimodeling.com page, "The Kernel Is the Other Half of the
// Answer").
//
// With at most 16 tokens the product is bound by reading the packed weights once, like the
// batch-one SpMV, so the kernels are laid out like the SpMV: a workgroup holds RG row groups
// of 16 rows, each split over CS waves along the columns (RG * CS <= 16; the other waves
// only help stage X); X of all tokens sits in LDS (in column phases when it does not fit);
// each wave streams its rows' values and masks with no barrier in its loop and multiplies
// them on a matrix instruction that covers every token at once, and the CS partial tiles of
// a row group are summed through LDS at the end.
//
// 2:4 (skinny_spmm_kernel<1, false>): the 2:4 sparse instruction (16 x 16 x 64) directly,
// with the position codes of the prefill kernel (nm_prefill_impl.h). 4:8 and 8:16
// (skinny_spmm_kernel<1, true>): these patterns keep exactly 8 values in every 16 aligned
// columns, so each 4-column group is split into two 2:4 operands (its first two kept values,
// and the rest) by the split tables of nm_prefill_impl.h, kept in LDS; both operands go
// through the sparse instruction with the same X fragment. Both read whole 128-byte lines
// per load (skinny_line_body).
//
// 16:32 (skinny_expand_kernel): a word's 16 kept values may sit anywhere in its 32 columns,
// so the dense 16 x 16 x 32 instruction takes each word, with the lanes' fragments expanded
// to dense columns: each wave writes the step's loaded values (16 rows x 64 bytes) to its
// own LDS area, and lane (row, q) reads the 8 halves from its mask byte's first kept value
// on and places them with the expansion table below (skinny_expand_body).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nm_prefill_impl.h"

namespace nm {
namespace skinny_detail {

using namespace prefill_detail;

constexpr int kMaxWaves = 16;
constexpr int kMaxTokens = 16;
constexpr int kThreadsFixed = 64 * kMaxWaves;           // every launch uses 16 waves
constexpr int kXChunksPerThread = 8;                    // X staged per phase: <= 8 x 16 B per thread
constexpr size_t kMaxXBytes = size_t(kThreadsFixed) * kXChunksPerThread * 16;   // 128 KiB

// LDS bytes of the X buffer for `tokens` rows of `phase_cols` columns, and of the reduction
// area for `waves` waves (one float4 per lane).
__host__ __device__ inline size_t x_bytes(int tokens, int phase_cols) { return size_t(tokens) * phase_cols * 2; }
__host__ __device__ inline size_t red_bytes(int waves) { return size_t(waves) * 64 * 16; }

// LDS byte offset of 16-byte chunk c of token t, rows of rb bytes: the low 3 bits of the
// chunk index are XORed with the token's (8 tokens read at a time land on 8 bank groups).
__device__ __forceinline__ uint32_t xoff(int t, int c, uint32_t rb) {
  return uint32_t(t) * rb + (uint32_t(c ^ (t & 7)) << 4);
}

// What the kernel does with the packed operand: 2:4 directly, 4:8 / 8:16 split, 16:32
// expanded.
constexpr int kModeDirect = 0, kModeSplit = 1, kModeExpand = 2;
// EXPAND: LDS bytes of one wave's area: the step's values of 16 rows (64 bytes each) and
// room for a window read past the last row's second word
constexpr uint32_t kExpandWaveBytes = 16 * 64 + 64;

// LDS bytes ahead of X: the split tables, or the expansion table and the waves' value areas.
template <int MODE>
__host__ __device__ constexpr uint32_t lead_bytes() {
  return MODE == kModeSplit ? kSplitLutBytes
       : MODE == kModeExpand ? kExpandBytes + uint32_t(kMaxWaves) * kExpandWaveBytes
                             : 0u;
}

// The workgroup's view of the launch: its rows, the wave's place in them, and the buffer
// resources of its slices of the packed matrix and of X. With `splits` > 1 the columns of
// each group of row tiles are split over that many consecutive workgroups (split = which).
struct Tile {
  int lane, wave, q, li, rg, cs;
  bool active;   // the wave owns rows (rg < rg_count)
  int wg_r0, words;
  int tile0, split;   // first 16-row tile of the workgroup; its part of the columns
  __amdgpu_buffer_rsrc_t vr, mr, xr;

  __device__ __forceinline__ Tile(const uint16_t* values, const uint32_t* masks, const uint16_t* X, int rows,
                                  int cols, int tokens, int rg_count, int cs_count, int splits = 1) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    // the wave index and everything derived from it are wave-uniform (scalar registers):
    // the loop bounds, the step offsets and the checks on them cost no vector instructions
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    q = lane >> 4;
    li = lane & 15;
    rg = wave / cs_count;
    cs = wave - rg * cs_count;
    // waves past rg_count * cs_count (when 16 is not a multiple of cs_count) stage X and
    // meet the barriers but own no rows
    active = rg < rg_count;
    const int wg_rows_max = rg_count * 16;
    // splits is 1, 2, 4 or 8: a shift, and none of it without a split
    const int sh = splits == 1 ? 0 : splits == 2 ? 1 : splits == 4 ? 2 : 3;
    const int wg = int(blockIdx.x) >> sh;
    split = int(blockIdx.x) & (splits - 1);
    tile0 = wg * rg_count;
    wg_r0 = wg * wg_rows_max;
    const int wg_rows = min(wg_rows_max, rows - wg_r0);
    words = cols >> 5;
    vr = make_rsrc(values + size_t(wg_r0) * unsigned(cols >> 1), int64_t(wg_rows) * cols);
    mr = make_rsrc(masks + size_t(wg_r0) * unsigned(words), int64_t(wg_rows) * words * 4);
    xr = make_rsrc(X, int64_t(tokens) * cols * 2);
  }
};

// X[0 .. tokens)[p0 .. p0 + chunks * 8) of one phase: flat chunk k = tid + kThreadsFixed * j
// of token t = k / chunks, chunk c = k % chunks (one division, then steps of kThreadsFixed).
// Chunks past the row load out of range (zero); chunks past the end are not written.
struct XStage {
  uint4 xs[kXChunksPerThread];
  uint32_t xdst[kXChunksPerThread];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t xr, int tokens, int cols, int p0, int chunks,
                                       uint32_t rb) {
    const int tid = threadIdx.x;
    const int nchunks = tokens * chunks;
    const int dt = kThreadsFixed / chunks, dc = kThreadsFixed - dt * chunks;
    int t = tid / chunks, c = tid - t * chunks;
#pragma unroll
    for (int j = 0; j < kXChunksPerThread; ++j) {
      const int k = tid + kThreadsFixed * j;
      const int col = p0 + 8 * c;
      const bool ok = k < nchunks && col < cols;
      xs[j] = buf_load16(xr, ok ? (uint32_t(t) * uint32_t(cols) + uint32_t(col)) * 2u : kOutOfRange);
      xdst[j] = k < nchunks ? xoff(t, c, rb) : 0xFFFFFFFFu;
      t += dt;
      c += dc;
      if (c >= chunks) { c -= chunks; ++t; }
    }
  }

  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int j = 0; j < kXChunksPerThread; ++j)
      if (xdst[j] != 0xFFFFFFFFu) *reinterpret_cast<uint4*>(lds + xdst[j]) = xs[j];
  }
};

// Column splits (splits > 1): each workgroup of a tile's group leaves its fp32 partial tile
// (one float4 per lane, 1 KiB per 16-row tile) in part[(tile * splits + split) * 64 + lane]
// and counts itself in cnt[tile]; the last one to arrive sums the splits' partials in split
// order (the same order whichever arrives last), rounds once, stores, and sets the count back
// to zero, so the counters are zero again after every launch.
constexpr int kMaxSplits = 8;

struct SplitWs {
  float4* part;
  unsigned* cnt;
  int splits;
};

// The CS partial tiles of each row group summed through LDS in a fixed order; the group's
// first wave rounds once and stores (with column splits, the last split's first wave). D
// layout of the instructions: lane (q, li) holds token li, rows 4q .. 4q+3 of the tile.
__device__ __forceinline__ void reduce_store(const Tile& w, f4_t acc, int cs_count, int rows, int tokens,
                                             uint16_t* __restrict__ Y, char* lds_base,
                                             const SplitWs& sw = SplitWs{nullptr, nullptr, 1}) {
  __syncthreads();
  float4* red = reinterpret_cast<float4*>(lds_base);
  red[w.wave * 64 + w.lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (w.cs != 0 || !w.active) return;
  float4 s = red[w.wave * 64 + w.lane];
  for (int k = 1; k < cs_count; ++k) {
    const float4 v = red[(w.wave + k) * 64 + w.lane];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (sw.splits > 1) {
    const int tile = w.tile0 + w.rg;
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(sw.part + size_t(tile) * unsigned(sw.splits) * 64u, int64_t(sw.splits) * 1024);
    coherent_store16(pr, uint32_t(w.split * 64 + w.lane) * 16u, s);
    // the partial has reached the device's coherence point before the count moves
    __builtin_amdgcn_s_waitcnt(0);
    unsigned old = 0;
    if (w.lane == 0) old = atomicAdd(sw.cnt + tile, 1u);
    old = unsigned(__shfl(int(old), 0));
    if (old != unsigned(sw.splits - 1)) return;
    // the last of the tile's workgroups: every other split's partial is complete
    // (all kMaxSplits loads issued at once; those past the resource's splits * 1 KiB read
    // zero, and adding zero after the last split leaves the sum as it is)
    float4 v[kMaxSplits];
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k) v[k] = coherent_load16(pr, uint32_t(k * 64 + w.lane) * 16u);
    s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k) {
      s.x += v[k].x; s.y += v[k].y; s.z += v[k].z; s.w += v[k].w;
    }
    if (w.lane == 0) atomicExch(sw.cnt + tile, 0u);
  }
  const int row = w.wg_r0 + w.rg * 16 + 4 * w.q;
  if (w.li >= tokens || row >= rows) return;
  uint16_t* out = Y + size_t(w.li) * unsigned(rows);
  const float e[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (row + k < rows) out[row + k] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(e[k]));
}

// ---- 2:4 (DIRECT) and 4:8 / 8:16 (SPLIT): whole 128-byte lines per load.
// The instruction's A layout puts 16 rows on the lanes of every 16-lane row (lane l: row
// l % 16), so a load shaped like the operand covers 16 rows x 64 bytes: half of each row's
// 128-byte line, whose other half the next step's load requests later. Measured on MI355X
// this holds the weight stream well below the SpMV's (14336 x 4096 at 8 vectors: 20.3 us
// with such loads against 16.7 us when every load covers whole lines). So each load here
// covers 8 rows x one whole line (128 columns, two 64-column products): load h (0, 1) gives
// lane l row 8h + l % 8 and 16-byte chunk 2 (l / 16) + (l / 8) % 2 of the line. One row_ror:8
// DPP move and a select per dword then give, for j = 0, 1, the operand T_j in which lane l
// holds row l % 16, chunk 2 (l / 16) + j:
//   T_0 = (l % 16 < 8) ? load0 : ror8(load1),   T_1 = (l % 16 < 8) ? ror8(load0) : load1.
// Product j takes T_j, so its logical K index k (A lane q holds k = 16q .. 16q+15) sits at
// line column 32 (k / 16) + 16 j + k % 16: the X fragment of lane q (K = 8q .. 8q+7 and
// 32+8q .. 32+8q+7) is the line's 8-column chunks 4 (q / 2) + q % 2 + 2 j and that plus 8,
// and the mask bits of lane q are half j of the line's word q.
__device__ __forceinline__ uint4 ror8_rows(uint4 v) {   // row_ror:8 inside every 16-lane row
  return make_uint4(uint32_t(__builtin_amdgcn_mov_dpp(int(v.x), 0x128, 0xF, 0xF, false)),
                    uint32_t(__builtin_amdgcn_mov_dpp(int(v.y), 0x128, 0xF, 0xF, false)),
                    uint32_t(__builtin_amdgcn_mov_dpp(int(v.z), 0x128, 0xF, 0xF, false)),
                    uint32_t(__builtin_amdgcn_mov_dpp(int(v.w), 0x128, 0xF, 0xF, false)));
}

__device__ __forceinline__ uint4 sel4(bool c, uint4 a, uint4 b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

constexpr int kLineDepth = 2;   // lines (two loads each) in flight per wave
constexpr int kMaskLines = 2;   // lines per mask block (8 words of each row)

// COLS: the column-split form (skinny_colsplit_kernel); without it the split bookkeeping is
// compiled out, so that the unsplit kernel is the same code as before the split existed.
template <int MODE, bool COLS>
__device__ __forceinline__ void skinny_line_body(const uint16_t* __restrict__ values,
                                                 const uint32_t* __restrict__ masks,
                                                 const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                 int rows, int cols, int tokens, int rg_count, int cs_count,
                                                 int phase_cols, const SplitWs& sw) {
  constexpr bool SPLIT = MODE == kModeSplit;
  static_assert(MODE == kModeDirect || MODE == kModeSplit, "whole-line loads: 2:4 and the split patterns");
  extern __shared__ __attribute__((aligned(16))) char lds_base[];
  char* const lds = lds_base + lead_bytes<MODE>();   // SPLIT: the split tables first, X after them
  const int tid = threadIdx.x;
  const Tile w(values, masks, X, rows, cols, tokens, rg_count, cs_count, COLS ? sw.splits : 1);
  const int q = w.q, li = w.li;
  // this workgroup's columns: lines [L s / S, L (s + 1) / S) of the row's L for split s of S
  // (lines <= 2^14 and splits <= 8: 32-bit products); without a split the whole row
  int c_beg = 0, c_end = cols;
  if constexpr (COLS) {
    const unsigned lines = unsigned(cols + 127) >> 7;
    c_beg = 128 * int(lines * unsigned(w.split) / unsigned(sw.splits));
    c_end = min(cols, 128 * int(lines * unsigned(w.split + 1) / unsigned(sw.splits)));
  }
  // value loads: lane l of load h reads row 8h + l % 8 of the row group, chunk kc of the line
  const int kc = 2 * q + ((w.lane >> 3) & 1);
  const uint32_t voff0 = uint32_t(w.rg * 16 + (w.lane & 7)) * uint32_t(cols) + 16u * uint32_t(kc);
  const uint32_t voff1 = voff0 + 8u * uint32_t(cols);
  // mask blocks: lane (q, li) holds words 2q, 2q+1 of the block for row li
  const uint32_t moff = uint32_t(w.rg * 16 + li) * uint32_t(w.words) * 4u + 8u * uint32_t(q);
  const bool lo8 = (w.lane & 8) == 0;
  const int xq = 4 * (q >> 1) + (q & 1);   // X chunk of lane q in product 0 of a line
  // token rows past the batch read the last token's X: their products are never stored
  const int xt = min(li, tokens - 1);

  f4_t acc = f4_t{0.f, 0.f, 0.f, 0.f};
  uint4 va[kLineDepth], vb[kLineDepth];
  uint2 mcur, mnext;
  // SPLIT: this thread's 16-byte chunks of the split tables (1024 + 64 chunks), loaded
  // before anything else so that the waits for X below cover them
  uint4 lut_a{}, lut_b{};
  if constexpr (SPLIT) {
    const uint4* tab = reinterpret_cast<const uint4*>(&kSplitTable);
    lut_a = tab[tid];
    lut_b = tab[2 * kSplitEntries + (tid & 63)];
  }
  for (int p0 = c_beg; p0 < c_end; p0 += phase_cols) {
    const int pc = min(phase_cols, c_end - p0);      // columns in this phase (multiple of 32)
    const uint32_t rb = uint32_t(2 * phase_cols);    // LDS bytes per token row
    // this wave's lines of the phase (phase_cols is a multiple of 128)
    const int plines = (pc + 127) / 128;
    const int l_lo = int((int64_t(plines) * w.cs) / cs_count);
    const int l_hi = int((int64_t(plines) * (w.cs + 1)) / cs_count);
    const int n = w.active ? l_hi - l_lo : 0;
    const int last = max(n - 1, 0);
    const int c_lo = p0 + 128 * l_lo;                // first column of the wave's range
    // line p of the range holds this lane's chunk iff p < p_lim; lines past it (the last
    // block's padding, a tail of 32 to 96 columns) load zeros, which add exactly zero
    const int p_lim = min(n, (cols - c_lo - 16 * kc + 127) / 128);
    const uint32_t vb0 = voff0 + uint32_t(c_lo), vb1 = voff1 + uint32_t(c_lo);
    auto load_line = [&](uint4& f0, uint4& f1, int p) {
      const bool ok = p < p_lim;
      f0 = buf_load16(w.vr, ok ? vb0 + 128u * uint32_t(p) : kOutOfRange);
      f1 = buf_load16(w.vr, ok ? vb1 + 128u * uint32_t(p) : kOutOfRange);
    };
    auto load_m = [&](int p) {   // mask block starting at line p of the range (clamped into it)
      const uint32_t cm = uint32_t(c_lo + 128 * min(p, last)) >> 3;
      mnext = buf_load8(w.mr, n > 0 ? moff + cm : kOutOfRange);
    };
    XStage xst;
    xst.load(w.xr, tokens, cols, p0, plines * 16, rb);
    // then the first weight loads, in flight while X is written to LDS (the X loads were
    // issued first, so waiting for them does not wait for these; mask block first, as in
    // the loop, so that the loop's waits are the same on every pass)
    load_m(0);
#pragma unroll
    for (int d = 0; d < kLineDepth; ++d) load_line(va[d], vb[d], d);
    __syncthreads();                                 // the previous phase's LDS reads are done
    if constexpr (SPLIT) {
      if (p0 == c_beg) {
        reinterpret_cast<uint4*>(lds_base)[tid] = lut_a;
        if (tid < 64) reinterpret_cast<uint4*>(lds_base)[2 * kSplitEntries + tid] = lut_b;
      }
    }
    xst.store(lds);
    __syncthreads();
    if (n > 0) {
      // X fragment addresses of products 0 and 1 of the phase's first line
      const uint32_t b_lo0 = xoff(xt, xq, rb), b_hi0 = xoff(xt, xq + 8, rb);
      const uint32_t b_lo1 = xoff(xt, xq + 2, rb), b_hi1 = xoff(xt, xq + 10, rb);
      for (int pb = 0; pb < n; pb += kMaskLines) {
        // 2:4: the position codes of the block's words, once per block
        mcur = SPLIT ? mnext : make_uint2(pair_codes32(mnext.x), pair_codes32(mnext.y));
        load_m(pb + kMaskLines);
#pragma unroll
        for (int j = 0; j < kMaskLines; ++j) {
          const int p = pb + j;
          const int d = j % kLineDepth;
          // word q of line j of the block is word 4j + q, held by lane (li, 2j + q / 2) as
          // component q % 2
          const int src = 4 * (li + 16 * (2 * j + (q >> 1)));
          const uint32_t wx = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(mcur.x)));
          const uint32_t wy = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(mcur.y)));
          const uint32_t word = (q & 1) ? wy : wx;
          // the line's two operands in the instruction's layout
          const uint4 t0 = sel4(lo8, va[d], ror8_rows(vb[d]));
          const uint4 t1 = sel4(lo8, ror8_rows(va[d]), vb[d]);
          // X of the line's two products; zero past the range (a wave-uniform test)
          uint4 x0l = make_uint4(0, 0, 0, 0), x0h = x0l, x1l = x0l, x1h = x0l;
          if (p < n) {
            const uint32_t cb = uint32_t(l_lo + p) * 256u;
            x0l = *reinterpret_cast<const uint4*>(lds + b_lo0 + cb);
            x0h = *reinterpret_cast<const uint4*>(lds + b_hi0 + cb);
            x1l = *reinterpret_cast<const uint4*>(lds + b_lo1 + cb);
            x1h = *reinterpret_cast<const uint4*>(lds + b_hi1 + cb);
          }
          // the loaded registers are free once the operands are formed: the line after the
          // next one is requested now, while the products run
          load_line(va[d], vb[d], p + kLineDepth);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint4 cur = h ? t1 : t0;
            const uint4 lo = h ? x1l : x0l, hi = h ? x1h : x0h;
            const u8_t xv = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const h16_t bf = __builtin_bit_cast(h16_t, xv);
            const uint32_t m16 = __builtin_amdgcn_ubfe(word, 16u * uint32_t(h), 16);
            if constexpr (SPLIT) {
              const uint32_t e0 = 32u * (m16 & 0xFFu), e1 = 32u * (256u + (m16 >> 8));
              const uint4 s0 = *reinterpret_cast<const uint4*>(lds_base + e0);
              const uint4 s1 = *reinterpret_cast<const uint4*>(lds_base + e0 + 16);
              const uint4 s2 = *reinterpret_cast<const uint4*>(lds_base + e1);
              const uint4 s3 = *reinterpret_cast<const uint4*>(lds_base + e1 + 16);
              const uint16_t* codes = reinterpret_cast<const uint16_t*>(lds_base + kSplitSelBytes);
              const uint32_t i0 = codes[m16 & 0xFFu], i1 = codes[256u + (m16 >> 8)];
              auto pick = [&](uint32_t lo_sel, uint32_t hi_sel) {
                return __builtin_amdgcn_perm(cur.y, cur.x, lo_sel) | __builtin_amdgcn_perm(cur.w, cur.z, hi_sel);
              };
              const uint4 opa = make_uint4(pick(s0.x, s0.y), pick(s1.x, s1.y), pick(s2.x, s2.y), pick(s3.x, s3.y));
              const uint4 opb = make_uint4(pick(s0.z, s0.w), pick(s1.z, s1.w), pick(s2.z, s2.w), pick(s3.z, s3.w));
              const int ia = int(__builtin_amdgcn_perm(i1, i0, 0x0C0C0400u));   // A codes of groups 0..3
              const int ib = int(__builtin_amdgcn_perm(i1, i0, 0x0C0C0501u));   // B codes
              acc = __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(h8_t, opa), bf, acc, ia, 0, 0);
              acc = __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(h8_t, opb), bf, acc, ib, 0, 0);
            } else {
              // m16 holds the position codes of the lane's 4 groups
              acc = __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(h8_t, cur), bf, acc, int(m16), 0, 0);
            }
          }
        }
      }
    }
  }
  if constexpr (COLS)
    reduce_store(w, acc, cs_count, rows, tokens, Y, lds_base, sw);
  else
    reduce_store(w, acc, cs_count, rows, tokens, Y, lds_base);
}

// ---- 16:32 (EXPAND): 64-column steps, each wave's values of a step through its own LDS area.
constexpr int kMaskSteps = 4;   // 64-column steps per mask block
constexpr int kDepth = 4;       // value loads in flight per wave

__device__ __forceinline__ void skinny_expand_body(const uint16_t* __restrict__ values,
                                                   const uint32_t* __restrict__ masks,
                                                   const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                   int rows, int cols, int tokens, int rg_count, int cs_count,
                                                   int phase_cols) {
  extern __shared__ __attribute__((aligned(16))) char lds_base[];
  // the expansion table and the waves' value areas, then X
  char* const lds = lds_base + lead_bytes<kModeExpand>();
  const int tid = threadIdx.x;
  const Tile w(values, masks, X, rows, cols, tokens, rg_count, cs_count);
  const int q = w.q, li = w.li;
  // lane (q, li) loads values 8q .. 8q+7 of a 64-column step for row li, and words 2q, 2q+1
  // of a mask block
  const uint32_t rl = uint32_t(w.rg * 16 + li);   // row within the workgroup
  const uint32_t voff = rl * uint32_t(cols) + 16u * uint32_t(q);
  const uint32_t moff = rl * uint32_t(w.words) * 4u + 8u * uint32_t(q);
  const int qcol = 32 * (q >> 1);
  // token rows past the batch read the last token's X: their products are never stored
  const int xt = min(li, tokens - 1);
  char* const area = lds_base + kExpandBytes + uint32_t(w.wave) * kExpandWaveBytes;

  f4_t acc = f4_t{0.f, 0.f, 0.f, 0.f};
  uint4 vbuf[kDepth];
  uint2 mcur, mnext;
  // the expansion table: 2 * kExpandEntries chunks of 16 bytes, loaded first so that the
  // waits for X cover it
  const uint4 lut = reinterpret_cast<const uint4*>(&kExpandTable)[tid & (2 * kExpandEntries - 1)];
  for (int p0 = 0; p0 < cols; p0 += phase_cols) {
    const int pc = min(phase_cols, cols - p0);       // columns in this phase (multiple of 32)
    const uint32_t rb = uint32_t(2 * phase_cols);    // LDS bytes per token row
    // this wave's steps of the phase
    const int psteps = (pc + 63) / 64;
    const int s_lo = int((int64_t(psteps) * w.cs) / cs_count), s_hi = int((int64_t(psteps) * (w.cs + 1)) / cs_count);
    const int n = w.active ? s_hi - s_lo : 0;
    const int last = max(n - 1, 0);
    const int c_lo = p0 + 64 * s_lo;                 // first column of the wave's range
    // value loads: step s of the range is inside the row for this lane iff s < s_lim; steps
    // past it (the last block's padding, a 32-column tail) load zeros, so they add exactly
    // zero and every slot of a block runs the same code
    const int s_lim = min(n, (cols - c_lo - qcol + 63) / 64);
    const uint32_t vbase = voff + uint32_t(c_lo);
    auto load_v = [&](uint4& f, int s) { f = buf_load16(w.vr, s < s_lim ? vbase + 64u * uint32_t(s) : kOutOfRange); };
    auto load_m = [&](int s) {   // mask block starting at step s of the range (clamped into it)
      const uint32_t cm = uint32_t(c_lo + 64 * min(s, last)) >> 3;
      mnext = buf_load8(w.mr, n > 0 ? moff + cm : kOutOfRange);
    };
    XStage xst;
    xst.load(w.xr, tokens, cols, p0, psteps * 8, rb);
    load_m(0);
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load_v(vbuf[d], d);
    __syncthreads();                                 // the previous phase's LDS reads are done
    if (p0 == 0 && tid < 2 * kExpandEntries) reinterpret_cast<uint4*>(lds_base)[tid] = lut;
    xst.store(lds);
    __syncthreads();
    if (n > 0) {
      const uint32_t b_lo = xoff(xt, q, rb), b_hi = xoff(xt, 4 + q, rb);
      for (int s0 = 0; s0 < n; s0 += kMaskSteps) {
        mcur = mnext;
        load_m(s0 + kMaskSteps);
#pragma unroll
        for (int j = 0; j < kMaskSteps; ++j) {
          const int s = s0 + j;
          // the products read vbuf[j] in place; its next load is issued after them, so the
          // registers are never copied (a copy would wait for every load in flight)
          const uint4 cur = vbuf[j % kDepth];
          const int src = 4 * (li + 16 * j);
          // X of the step (chunks 8 (s_lo + s) ..); zero past the range (a wave-uniform test)
          uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
          if (s < n) {
            const uint32_t cb = uint32_t(s_lo + s) * 128u;
            lo = *reinterpret_cast<const uint4*>(lds + b_lo + cb);
            hi = *reinterpret_cast<const uint4*>(lds + b_hi + cb);
          }
          const uint32_t w0 = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(mcur.x)));
          const uint32_t w1 = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(mcur.y)));
          // the step's values to this wave's area (row li at 64 li, lane q's 16 bytes at
          // 16 q), visible to the other lanes of the wave before they are read back
          *reinterpret_cast<uint4*>(area + 64 * li + 16 * q) = cur;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
          for (int i = 0; i < 2; ++i) {   // word i of the step: one dense 16 x 16 x 32 product
            const uint32_t wi = i ? w1 : w0;
            const uint32_t byte = __builtin_amdgcn_ubfe(wi, 8u * uint32_t(q), 8);
            // first kept value of the lane's byte among the word's 16 (at most 16 for a
            // valid mask; clamped so that any mask keeps the window inside the area)
            const uint32_t first = min(uint32_t(__builtin_popcount(wi & ((1u << (8 * q)) - 1u))), 16u);
            const uint32_t off = 64u * uint32_t(li) + 32u * uint32_t(i) + 2u * first;   // window, bytes
            const uint32_t* wd = reinterpret_cast<const uint32_t*>(area + (off & ~3u));
            const uint32_t sh = (off & 2u) * 8u;   // 16 when the window starts mid-dword
            const uint32_t r0 = wd[0], r1 = wd[1], r2 = wd[2], r3 = wd[3], r4 = wd[4];
            const uint32_t v0 = __builtin_amdgcn_alignbit(r1, r0, sh), v1 = __builtin_amdgcn_alignbit(r2, r1, sh);
            const uint32_t v2 = __builtin_amdgcn_alignbit(r3, r2, sh), v3 = __builtin_amdgcn_alignbit(r4, r3, sh);
            const uint4 s0 = *reinterpret_cast<const uint4*>(lds_base + 32u * byte);
            const uint4 s1 = *reinterpret_cast<const uint4*>(lds_base + 32u * byte + 16u);
            auto pick = [&](uint32_t lo_sel, uint32_t hi_sel) {
              return __builtin_amdgcn_perm(v1, v0, lo_sel) | __builtin_amdgcn_perm(v3, v2, hi_sel);
            };
            const uint4 dense = make_uint4(pick(s0.x, s0.y), pick(s0.z, s0.w), pick(s1.x, s1.y), pick(s1.z, s1.w));
            const uint4 xf = i ? hi : lo;   // X of the word's columns 8q .. 8q+7, every token
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, dense),
                                                         __builtin_bit_cast(h8_t, xf), acc, 0, 0, 0);
          }
          // every lane has read the area before the next step writes it
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          load_v(vbuf[j % kDepth], s + kDepth);
        }
      }
    }
  }
  reduce_store(w, acc, cs_count, rows, tokens, Y, lds_base);
}

// TR (row tiles per wave) is 1: one 16-row tile per wave; the parameter stays in the kernel
// names that profiles and tests refer to.
template <int TR, bool SPLIT>
__global__ __launch_bounds__(kThreadsFixed) void skinny_spmm_kernel(const uint16_t* __restrict__ values,
                                                                     const uint32_t* __restrict__ masks,
                                                                     const uint16_t* __restrict__ X,
                                                                     uint16_t* __restrict__ Y, int rows, int cols,
                                                                     int tokens, int rg_count, int cs_count,
                                                                     int phase_cols) {
  static_assert(TR == 1, "one row tile per wave");
  skinny_line_body<SPLIT ? kModeSplit : kModeDirect, false>(values, masks, X, Y, rows, cols, tokens, rg_count,
                                                            cs_count, phase_cols, SplitWs{nullptr, nullptr, 1});
}

// The same products with the columns of each 16-row tile split over `splits` (2, 4 or 8)
// consecutive workgroups, one tile per workgroup (SplitWs: partials and counters).
template <bool SPLIT>
__global__ __launch_bounds__(kThreadsFixed) void skinny_colsplit_kernel(const uint16_t* __restrict__ values,
                                                                         const uint32_t* __restrict__ masks,
                                                                         const uint16_t* __restrict__ X,
                                                                         uint16_t* __restrict__ Y, int rows, int cols,
                                                                         int tokens, int cs_count, int phase_cols,
                                                                         int splits, float4* part, unsigned* cnt) {
  skinny_line_body<SPLIT ? kModeSplit : kModeDirect, true>(values, masks, X, Y, rows, cols, tokens, 1, cs_count,
                                                           phase_cols, SplitWs{part, cnt, splits});
}

template <int TR>
__global__ __launch_bounds__(kThreadsFixed) void skinny_expand_kernel(const uint16_t* __restrict__ values,
                                                                       const uint32_t* __restrict__ masks,
                                                                       const uint16_t* __restrict__ X,
                                                                       uint16_t* __restrict__ Y, int rows, int cols,
                                                                       int tokens, int rg_count, int cs_count,
                                                                       int phase_cols) {
  static_assert(TR == 1, "one row tile per wave");
  skinny_expand_body(values, masks, X, Y, rows, cols, tokens, rg_count, cs_count, phase_cols);
}

}  // namespace skinny_detail
}  // namespace nm
