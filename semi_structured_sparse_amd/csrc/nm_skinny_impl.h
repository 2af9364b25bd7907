// Small-batch 2:4 product on the gfx950 sparse matrix instruction: Y [tokens][rows] =
// X [tokens][cols] W'^T for 1 <= tokens <= 16, W' given as the packed 2:4 values and
// bitmask (the batch side of the SpMV / SpMM split the news.bitwarelabs.com page draws in
// "What's new"; bitmask format of the aimodeling.com page, "The Kernel Is the Other Half of
// the Answer").
//
// With at most 16 tokens the product is bound by reading the packed weights once, like the
// batch-one SpMV, so the kernel is laid out like the SpMV: a workgroup holds RG row groups
// of 16 * TR rows, each split over CS waves along the columns (RG * CS <= 16; the other
// waves only help stage X); X of all tokens sits in LDS
// (in column phases when it does not fit); each wave streams its rows' values and masks
// with no barrier in its loop and multiplies them on the sparse matrix instruction (one
// 16 x 16 x 64 instruction per 16 rows and 64 columns covers every token), and the CS
// partial tiles of a row group are summed through LDS at the end.
//
// Operand layouts, the K permutation that makes a lane's 8 values contiguous in the packed
// row, the position codes and the mask-block permute are those of the prefill kernel
// (nm_prefill_impl.h), with mask blocks of 4 steps here (a wave may own only 4 steps):
// lane (q = l / 16, li = l % 16) holds values 8q .. 8q+7 of a 64-column step for row li,
// and the X fragment of token li at column chunks q and 4 + q of the step.
//
// 4:8 and 8:16 (SPLIT): each 4-column group is split into two 2:4 operands (its first two
// kept values, and the rest) by the split tables of nm_prefill_impl.h, which this kernel
// keeps in LDS; both operands go through the sparse instruction with the same X fragment.
//
// 16:32 (EXPAND, skinny_expand_kernel): a word's 16 kept values may sit anywhere in its 32
// columns, so the dense 16 x 16 x 32 instruction takes each word, with the lanes' fragments
// expanded to dense columns: each wave writes the step's loaded values (16 rows x 64 bytes)
// to its own LDS area, and lane (row, q) reads the 8 halves from its mask byte's first kept
// value on and places them with the expansion table (nm_prefill_impl.h). The X fragments,
// loads, mask blocks and reduction are those of the 2:4 kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nm_prefill_impl.h"

namespace nm {
namespace skinny_detail {

using namespace prefill_detail;

constexpr int kMaxWaves = 16;
constexpr int kMaxTokens = 16;
constexpr int kMaskSteps = 4;   // 64-column steps per mask block
constexpr int kDepth = 4;       // value loads in flight per row tile
constexpr int kThreadsFixed = 64 * kMaxWaves;           // every launch uses 16 waves
constexpr int kXChunksPerThread = 8;                    // X staged per phase: <= 8 x 16 B per thread
constexpr size_t kMaxXBytes = size_t(kThreadsFixed) * kXChunksPerThread * 16;   // 128 KiB

// LDS bytes of the X buffer for `tokens` rows of `phase_cols` columns, and of the reduction
// area for `waves` waves of TR tiles (one float4 per lane per tile).
__host__ __device__ inline size_t x_bytes(int tokens, int phase_cols) { return size_t(tokens) * phase_cols * 2; }
__host__ __device__ inline size_t red_bytes(int waves, int tr) { return size_t(waves) * tr * 64 * 16; }

// LDS byte offset of 16-byte chunk c of token t, rows of rb bytes: the low 3 bits of the
// chunk index are XORed with the token's (8 tokens read at a time land on 8 bank groups).
__device__ __forceinline__ uint32_t xoff(int t, int c, uint32_t rb) {
  return uint32_t(t) * rb + (uint32_t(c ^ (t & 7)) << 4);
}


// What the kernel does with the packed operand: 2:4 directly, 4:8 / 8:16 split, 16:32
// expanded.
constexpr int kModeDirect = 0, kModeSplit = 1, kModeExpand = 2;
// EXPAND: LDS bytes of one wave's area per row tile: the step's values of 16 rows (64 bytes
// each) and room for a window read past the last row's second word
constexpr uint32_t kExpandWaveBytes = 16 * 64 + 64;

// LDS bytes ahead of X: the split tables, or the expansion table and the waves' value areas.
template <int TR, int MODE>
__host__ __device__ constexpr uint32_t lead_bytes() {
  return MODE == kModeSplit ? kSplitLutBytes
       : MODE == kModeExpand ? kExpandBytes + uint32_t(kMaxWaves) * TR * kExpandWaveBytes
                             : 0u;
}

template <int TR, int MODE>
__device__ __forceinline__ void skinny_body(const uint16_t* __restrict__ values, const uint32_t* __restrict__ masks,
                                            const uint16_t* __restrict__ X, uint16_t* __restrict__ Y, int rows,
                                            int cols, int tokens, int rg_count, int cs_count, int phase_cols) {
  constexpr bool SPLIT = MODE == kModeSplit;
  constexpr bool EXPAND = MODE == kModeExpand;
  extern __shared__ __attribute__((aligned(16))) char lds_base[];
  // SPLIT: the split tables first, X after them; EXPAND: the expansion table and the waves'
  // value areas, then X
  char* const lds = lds_base + lead_bytes<TR, MODE>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index and everything derived from it are wave-uniform (scalar registers): the
  // loop bounds, the step offsets and the checks on them cost no vector instructions
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, li = lane & 15;
  const int rg = wave / cs_count, cs = wave - rg * cs_count;
  // waves past rg_count * cs_count (when 16 is not a multiple of cs_count) stage X and meet
  // the barriers but own no rows
  const bool active = rg < rg_count;
  const int wg_rows_max = rg_count * 16 * TR;
  const int wg_r0 = int(blockIdx.x) * wg_rows_max;
  const int wg_rows = min(wg_rows_max, rows - wg_r0);
  const int words = cols >> 5;

  const __amdgpu_buffer_rsrc_t vr = make_rsrc(values + size_t(wg_r0) * unsigned(cols >> 1), int64_t(wg_rows) * cols);
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(masks + size_t(wg_r0) * unsigned(words), int64_t(wg_rows) * words * 4);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, int64_t(tokens) * cols * 2);
  uint32_t voff[TR], moff[TR];
#pragma unroll
  for (int a = 0; a < TR; ++a) {
    const uint32_t rl = uint32_t(rg * 16 * TR + 16 * a + li);   // row within the workgroup
    voff[a] = rl * uint32_t(cols) + 16u * uint32_t(q);
    moff[a] = rl * uint32_t(words) * 4u + 8u * uint32_t(q);
  }
  const int qcol = 32 * (q >> 1);
  const uint32_t mshift = 16u * uint32_t(q & 1);
  const bool tok_live = li < tokens;
  // token rows past the batch read the last token's X: their products are never stored
  const int xt = min(li, tokens - 1);

  f4_t acc[TR];
#pragma unroll
  for (int a = 0; a < TR; ++a) acc[a] = f4_t{0.f, 0.f, 0.f, 0.f};

  uint4 vb[kDepth][TR];
  uint2 mcur[TR], mnext[TR];
  // SPLIT: this thread's 16-byte chunks of the split tables (1024 + 64 chunks), loaded
  // before anything else so that the waits for X below cover them
  uint4 lut_a{}, lut_b{};
  if constexpr (SPLIT) {
    const uint4* tab = reinterpret_cast<const uint4*>(&kSplitTable);
    lut_a = tab[tid];
    lut_b = tab[2 * kSplitEntries + (tid & 63)];
  }
  if constexpr (EXPAND) {   // the expansion table: 2 * kExpandEntries chunks of 16 bytes
    const uint4* tab = reinterpret_cast<const uint4*>(&kExpandTable);
    lut_a = tab[tid & (2 * kExpandEntries - 1)];
  }
  for (int p0 = 0; p0 < cols; p0 += phase_cols) {
    const int pc = min(phase_cols, cols - p0);       // columns in this phase (multiple of 32)
    const uint32_t rb = uint32_t(2 * phase_cols);    // LDS bytes per token row
    // this wave's steps of the phase
    const int psteps = (pc + 63) / 64;
    const int s_lo = int((int64_t(psteps) * cs) / cs_count), s_hi = int((int64_t(psteps) * (cs + 1)) / cs_count);
    const int n = active ? s_hi - s_lo : 0;
    const int last = max(n - 1, 0);
    const int c_lo = p0 + 64 * s_lo;                 // first column of the wave's range
    // value loads: step s of the range is inside the row for this lane iff s < s_lim; steps
    // past it (the last block's padding, a 32-column tail) load zeros, so they add exactly
    // zero and every slot of a block runs the same code
    const int s_lim = min(n, (cols - c_lo - qcol + 63) / 64);
    uint32_t vbase[TR];
#pragma unroll
    for (int a = 0; a < TR; ++a) vbase[a] = voff[a] + uint32_t(c_lo);
    auto load_v = [&](uint4 (&f)[TR], int s) {
      const bool ok = s < s_lim;
#pragma unroll
      for (int a = 0; a < TR; ++a) f[a] = buf_load16(vr, ok ? vbase[a] + 64u * uint32_t(s) : kOutOfRange);
    };
    auto load_m = [&](int s) {   // mask block starting at step s of the range (clamped into it)
      const uint32_t cm = uint32_t(c_lo + 64 * min(s, last)) >> 3;
#pragma unroll
      for (int a = 0; a < TR; ++a) mnext[a] = buf_load8(mr, n > 0 ? moff[a] + cm : kOutOfRange);
    };
    // ---- X[0 .. tokens)[p0 .. p0 + pc) into registers (columns past the row read as zero):
    // flat chunk k = tid + kThreadsFixed * j of token t = k / chunks, chunk c = k % chunks
    // (one division, then steps of kThreadsFixed); chunks past the end load out of range
    // (zero) and are not written
    const int chunks = psteps * 8;                   // 16-byte chunks per token row, whole steps
    const int nchunks = tokens * chunks;
    const int dt = kThreadsFixed / chunks, dc = kThreadsFixed - dt * chunks;
    uint4 xs[kXChunksPerThread];
    uint32_t xdst[kXChunksPerThread];
    {
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
    // then the first weight loads: they are in flight while X is written to LDS (the X
    // loads were issued first, so waiting for them does not wait for these). The mask
    // block goes first, as in the loop (mask block, then the block's value loads), so the
    // waits the loop needs are the same on its first pass as on later ones.
    load_m(0);
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load_v(vb[d], d);
    __syncthreads();                                 // the previous phase's LDS reads are done
    if constexpr (SPLIT) {
      if (p0 == 0) {
        reinterpret_cast<uint4*>(lds_base)[tid] = lut_a;
        if (tid < 64) reinterpret_cast<uint4*>(lds_base)[2 * kSplitEntries + tid] = lut_b;
      }
    }
    if constexpr (EXPAND) {
      if (p0 == 0 && tid < 2 * kExpandEntries) reinterpret_cast<uint4*>(lds_base)[tid] = lut_a;
    }
#pragma unroll
    for (int j = 0; j < kXChunksPerThread; ++j)
      if (xdst[j] != 0xFFFFFFFFu) *reinterpret_cast<uint4*>(lds + xdst[j]) = xs[j];
    __syncthreads();
    if (n > 0) {
      const uint32_t b_lo = xoff(xt, q, rb), b_hi = xoff(xt, 4 + q, rb);
      for (int s0 = 0; s0 < n; s0 += kMaskSteps) {
        // 2:4: the position codes of the block's words, once per block; the steps then
        // only fetch and shift them
#pragma unroll
        for (int a = 0; a < TR; ++a)
          mcur[a] = (SPLIT || EXPAND) ? mnext[a] : make_uint2(pair_codes32(mnext[a].x), pair_codes32(mnext[a].y));
        load_m(s0 + kMaskSteps);
#pragma unroll
        for (int j = 0; j < kMaskSteps; ++j) {
          const int s = s0 + j;
          // the products read vb[j] in place; its next load is issued after them, so the
          // registers are never copied (a copy would wait for every load in flight)
          const uint4 (&cur)[TR] = vb[j % kDepth];
          const int src = 4 * (li + 16 * j);
          // X of the step (chunks 8 (s_lo + s) ..); zero past the range (a wave-uniform test)
          uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
          if (s < n) {
            const uint32_t cb = uint32_t(s_lo + s) * 128u;
            lo = *reinterpret_cast<const uint4*>(lds + b_lo + cb);
            hi = *reinterpret_cast<const uint4*>(lds + b_hi + cb);
          }
          const u8_t xv = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          const h16_t bf = __builtin_bit_cast(h16_t, xv);
#pragma unroll
          for (int a = 0; a < TR; ++a) {
            const uint32_t w0 = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(mcur[a].x)));
            const uint32_t w1 = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(mcur[a].y)));
            if constexpr (EXPAND) {
              // the step's values to this wave's area (row li at 64 li, lane q's 16 bytes at
              // 16 q), visible to the other lanes of the wave before they are read back
              char* const va = lds_base + kExpandBytes + uint32_t(wave * TR + a) * kExpandWaveBytes;
              *reinterpret_cast<uint4*>(va + 64 * li + 16 * q) = cur[a];
              __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
              __builtin_amdgcn_wave_barrier();
              __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
              for (int i = 0; i < 2; ++i) {   // word i of the step: one dense 16 x 16 x 32 product
                const uint32_t w = i ? w1 : w0;
                const uint32_t byte = __builtin_amdgcn_ubfe(w, 8u * uint32_t(q), 8);
                // first kept value of the lane's byte among the word's 16 (at most 16 for a
                // valid mask; clamped so that any mask keeps the window inside the area)
                const uint32_t pc = min(uint32_t(__builtin_popcount(w & ((1u << (8 * q)) - 1u))), 16u);
                const uint32_t off = 64u * uint32_t(li) + 32u * uint32_t(i) + 2u * pc;   // window, bytes
                const uint32_t* wd = reinterpret_cast<const uint32_t*>(va + (off & ~3u));
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
                acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, dense),
                                                                __builtin_bit_cast(h8_t, xf), acc[a], 0, 0, 0);
              }
              // every lane has read the area before the next step writes it
              __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
              __builtin_amdgcn_wave_barrier();
              __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
              continue;
            }
            const uint32_t m16 = __builtin_amdgcn_ubfe((q >> 1) ? w1 : w0, mshift, 16);
            if constexpr (SPLIT) {
              const uint32_t e0 = 32u * (m16 & 0xFFu), e1 = 32u * (256u + (m16 >> 8));
              const uint4 s0 = *reinterpret_cast<const uint4*>(lds_base + e0);
              const uint4 s1 = *reinterpret_cast<const uint4*>(lds_base + e0 + 16);
              const uint4 s2 = *reinterpret_cast<const uint4*>(lds_base + e1);
              const uint4 s3 = *reinterpret_cast<const uint4*>(lds_base + e1 + 16);
              const uint16_t* codes = reinterpret_cast<const uint16_t*>(lds_base + kSplitSelBytes);
              const uint32_t i0 = codes[m16 & 0xFFu], i1 = codes[256u + (m16 >> 8)];
              const uint4 v = cur[a];
              auto pick = [&](uint32_t lo_sel, uint32_t hi_sel) {
                return __builtin_amdgcn_perm(v.y, v.x, lo_sel) | __builtin_amdgcn_perm(v.w, v.z, hi_sel);
              };
              const uint4 va = make_uint4(pick(s0.x, s0.y), pick(s1.x, s1.y), pick(s2.x, s2.y), pick(s3.x, s3.y));
              const uint4 vb2 = make_uint4(pick(s0.z, s0.w), pick(s1.z, s1.w), pick(s2.z, s2.w), pick(s3.z, s3.w));
              const int ia = int(__builtin_amdgcn_perm(i1, i0, 0x0C0C0400u));   // A codes of groups 0..3
              const int ib = int(__builtin_amdgcn_perm(i1, i0, 0x0C0C0501u));   // B codes
              acc[a] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(h8_t, va), bf, acc[a], ia, 0, 0);
              acc[a] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(h8_t, vb2), bf, acc[a], ib, 0, 0);
            } else {
              // m16 holds the position codes of the lane's 4 groups
              acc[a] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(h8_t, cur[a]), bf, acc[a],
                                                                int(m16), 0, 0);
            }
          }
          load_v(vb[j % kDepth], s + kDepth);
        }
      }
    }
  }
  // ---- sum the CS partial tiles of each row group; the first wave of the group stores
  __syncthreads();
  float4* red = reinterpret_cast<float4*>(lds_base);
#pragma unroll
  for (int a = 0; a < TR; ++a)
    red[(wave * TR + a) * 64 + lane] = make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
  __syncthreads();
  if (cs != 0 || !active) return;
#pragma unroll
  for (int a = 0; a < TR; ++a) {
    float4 s = red[(wave * TR + a) * 64 + lane];
    for (int w = 1; w < cs_count; ++w) {
      const float4 v = red[((wave + w) * TR + a) * 64 + lane];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const int row = wg_r0 + rg * 16 * TR + 16 * a + 4 * q;
    if (!tok_live || row >= rows) continue;
    uint16_t* out = Y + size_t(li) * unsigned(rows);
    const float e[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (row + k < rows) out[row + k] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(e[k]));
  }
}

template <int TR, bool SPLIT>
__global__ __launch_bounds__(kThreadsFixed) void skinny_spmm_kernel(const uint16_t* __restrict__ values,
                                                                     const uint32_t* __restrict__ masks,
                                                                     const uint16_t* __restrict__ X,
                                                                     uint16_t* __restrict__ Y, int rows, int cols,
                                                                     int tokens, int rg_count, int cs_count,
                                                                     int phase_cols) {
  skinny_body<TR, SPLIT ? kModeSplit : kModeDirect>(values, masks, X, Y, rows, cols, tokens, rg_count, cs_count,
                                                     phase_cols);
}

template <int TR>
__global__ __launch_bounds__(kThreadsFixed) void skinny_expand_kernel(const uint16_t* __restrict__ values,
                                                                       const uint32_t* __restrict__ masks,
                                                                       const uint16_t* __restrict__ X,
                                                                       uint16_t* __restrict__ Y, int rows, int cols,
                                                                       int tokens, int rg_count, int cs_count,
                                                                       int phase_cols) {
  skinny_body<TR, kModeExpand>(values, masks, X, Y, rows, cols, tokens, rg_count, cs_count, phase_cols);
}

}  // namespace skinny_detail
}  // namespace nm
