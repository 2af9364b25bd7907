// Launchers of the prefill-sized products (many tokens per weight) on the matrix cores:
// the 50% sparse products (2:4 directly, 4:8 and 8:16 split into two 2:4 operands) and the
// dense product. The kernels are in nm_prefill_impl.h.
#include "nm_internal.h"
#include "nm_prefill_impl.h"

namespace nm {

using namespace prefill_detail;

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile shapes (TR x TT output tiles of 16 x 16 per wave, KS columns per step, loads D steps
// ahead). Dense: 128 rows x 256 tokens per workgroup (each weight fragment serves 16 token
// tiles) where the grid has a workgroup per CU, else 64 x 64. Sparse: the tile with the least
// modelled time (sparse_tile), from 64 x 64 up to 256 x 256.
using DenseLarge = Tile<2, 16, 64>;
using Small = Tile<1, 4, 64>;
using SparseLarge = Tile<4, 8, 64>;
constexpr int kDepth = 2;

template <typename T>
int64_t workgroups(int64_t rows, int64_t tokens) {
  return ceil_div(rows, T::kRows) * ceil_div(tokens, T::kTokens);
}

template <typename T>
bool use_large(int64_t rows, int64_t tokens, const DeviceInfo& dev) {
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  return workgroups<T>(rows, tokens) >= cus;
}

// Sparse tile choice. A workgroup's time is its 64-column steps times the time of a step,
// which grows with the workgroups n = ceil(grid / CUs) that share a CU: t1 + (n - 1) * tn
// (us; where fewer of them fit a CU at once the later ones wait, so tn >= t1 there). Fitted
// per tile to sweeps on MI355X (256 .. 4096 tokens, 1024 .. 14336 rows and columns; the model
// is within about 15% of every measured time and picks the fastest tile or one within 7% of
// it): 14336 x 4096 x 512, 2:4, 58.6 us on 256 x 128 against 119.2 on 64 x 64; 4096 x 14336 x
// 1024, 125.6 on 128 x 128 against 219.7; 4:8 at 4096 x 4096 x 2048, 96.3 on 128 x 256
// against 116.4 on 256 x 128; 64 x 128 tiles (three or more workgroups per CU) at 512 tokens:
// 4:8 at 4096 x 14336, 136 against 156 us on 128 x 64; 16:32 at 4096 x 4096, 64 against 83
// on 64 x 64. The split patterns' steps cost more (two instructions and the table lookups per
// fragment), so their wide token tiles pay off sooner.
struct TileCost {
  int tr, tt;
  double t1, tn;
};
constexpr TileCost kDirectTiles[] = {{1, 4, 0.266, 0.210}, {1, 8, 0.428, 0.310}, {2, 4, 0.378, 0.328},
                                     {2, 8, 0.537, 0.475}, {4, 8, 0.717, 0.825}, {4, 16, 1.27, 1.38}};
constexpr TileCost kSplitTiles[] = {{1, 4, 0.45, 0.273}, {1, 8, 0.625, 0.435}, {2, 4, 0.68, 0.443},
                                    {2, 8, 0.91, 0.693}, {4, 8, 1.57, 1.57},   {2, 16, 1.40, 1.42},
                                    {4, 16, 2.28, 2.37}};
// 16:32's steps expand each word's fragments through LDS first (about twice the split
// patterns' step time). It has no 256-row tiles: 256 x 128 (2.62 us a step) lost to
// 128 x 256 at every measured size, and 256 x 256 would spill its expansion registers.
constexpr TileCost kExpandTiles[] = {{1, 4, 0.80, 0.51},  {1, 8, 0.963, 0.627}, {1, 16, 1.37, 0.944},
                                     {2, 4, 1.28, 0.93},  {2, 8, 1.46, 1.09},   {2, 16, 1.85, 1.83}};

// the kernel family of a 50% pattern: 2:4 direct, 4:8 / 8:16 split, 16:32 expanded
int pf_mode(int n) { return n == 2 ? kPfDirect : n == 16 ? kPfExpand : kPfSplit; }

TileCost sparse_tile(int64_t rows, int64_t tokens, int mode, const DeviceInfo& dev) {
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const TileCost* c = mode == kPfDirect ? kDirectTiles : mode == kPfSplit ? kSplitTiles : kExpandTiles;
  const int n = mode == kPfDirect ? int(sizeof(kDirectTiles) / sizeof(TileCost))
              : mode == kPfSplit  ? int(sizeof(kSplitTiles) / sizeof(TileCost))
                                  : int(sizeof(kExpandTiles) / sizeof(TileCost));
  TileCost best = c[0];
  double best_t = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t grid = ceil_div(rows, 64 * c[i].tr) * ceil_div(tokens, 16 * c[i].tt);
    const double t = c[i].t1 + double(ceil_div(grid, cus) - 1) * c[i].tn;
    if (i == 0 || t < best_t) {
      best = c[i];
      best_t = t;
    }
  }
  return best;
}

template <int TR, int TT>
const void* sparse_kernel(int mode) {
  return mode == kPfDirect  ? reinterpret_cast<const void*>(&prefill_spmm_kernel<TR, TT, 64, kDepth>)
         : mode == kPfSplit ? reinterpret_cast<const void*>(&prefill_split_kernel<TR, TT, 64, kDepth>)
                            : reinterpret_cast<const void*>(&prefill_expand_kernel<TR, TT, 64, kDepth>);
}

// The kernel of a tile in the mode's table (64 x 256 for 16:32 only; 128 x 256 not for 2:4;
// 256-row tiles not for 16:32).
const void* sparse_kernel_of(const TileCost& t, int mode) {
  if (t.tr == 1) {
    if (t.tt == 4) return sparse_kernel<1, 4>(mode);
    if (t.tt == 8) return sparse_kernel<1, 8>(mode);
    return reinterpret_cast<const void*>(&prefill_expand_kernel<1, 16, 64, kDepth>);   // 16:32 only
  }
  if (t.tr == 2) {
    if (t.tt == 4) return sparse_kernel<2, 4>(mode);
    if (t.tt == 8) return sparse_kernel<2, 8>(mode);
    return mode == kPfSplit ? reinterpret_cast<const void*>(&prefill_split_kernel<2, 16, 64, kDepth>)
                            : reinterpret_cast<const void*>(&prefill_expand_kernel<2, 16, 64, kDepth>);
  }
  if (t.tt == 8)
    return mode == kPfSplit ? reinterpret_cast<const void*>(&prefill_split_kernel<4, 8, 64, kDepth>)
                            : reinterpret_cast<const void*>(&prefill_spmm_kernel<4, 8, 64, kDepth>);
  return mode == kPfSplit ? reinterpret_cast<const void*>(&prefill_split_kernel<4, 16, 64, kDepth>)
                          : reinterpret_cast<const void*>(&prefill_spmm_kernel<4, 16, 64, kDepth>);
}

}  // namespace

bool prefill_fits(int64_t rows, int64_t cols, int64_t tokens) {
  // byte offsets inside one workgroup's slices are 32-bit; workgroup counts fit an int
  return cols <= kPrefillMaxCols && tokens <= kPrefillMaxTokens && workgroups<Small>(rows, tokens) <= INT32_MAX;
}

bool prefill_pattern(int n, int m) { return 2 * n == m && (n == 2 || n == 4 || n == 8 || n == 16); }

namespace {

// Column splits where the small-tile grid leaves CUs idle: tiles of 64 rows x 32 tokens (up
// to 32 tokens) or x 64 tokens, and S = 2, 4, .. kMaxColSplits workgroups per tile while every
// split keeps at least one block of kColBlock columns and the grid stays within one
// workgroup per CU, or two where the CUs have at least 4 blocks each. Fitted to a sweep on
// MI355X (17..256 tokens, 1024..14336 rows and columns): one workgroup per CU costs about
// 7.6 us plus 0.31 us per 64-column step, two about 11.9 us plus 0.175 us per step of the CU
// (4096 x 4096 x 64, 2:4: 12.6 us at 4 splits against 14.7 at 8; 8192 x 8192 x 32: 23.1 us at
// 4 against 27.6 at 2). Where one workgroup per CU allows no split, 2 splits if two fit.
struct ColPlan {
  int splits = 1, blocks = 0, tt = 4;
  int64_t tiles = 0;
};

ColPlan colsplit_plan(int64_t rows, int64_t cols, int64_t tokens, const DeviceInfo& dev) {
  ColPlan p;
  if (use_large<SparseLarge>(rows, tokens, dev)) return p;
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  p.tt = tokens <= 32 ? 2 : 4;
  p.tiles = ceil_div(rows, Small::kRows) * ceil_div(tokens, 16 * p.tt);
  const int64_t nblk = ceil_div(cols, kColBlock);
  const int64_t cap = p.tiles * nblk >= 4 * cus ? 2 * cus : cus;   // workgroups in the grid
  int s = 1;
  while (s < kMaxColSplits && p.tiles * (2 * s) <= cap && 2 * s <= nblk) s *= 2;
  if (s == 1 && p.tiles * 2 <= 2 * cus && nblk >= 2) s = 2;
  if (s == 1) return p;
  p.blocks = int(ceil_div(nblk, s));
  p.splits = int(ceil_div(nblk, p.blocks));   // every split non-empty
  return p;
}

size_t colsplit_bytes(const ColPlan& p, const DeviceInfo& dev) {
  if (p.splits == 1) return 0;
  return counter_bytes(dev) + size_t(p.tiles) * size_t(p.splits) * size_t(kThreads) * size_t(p.tt) * 16u;
}

// Taller column splits for prompts of more than 128 tokens. There the 64-row tiles fill the
// CUs, but each walks every column (or half of them) with little reuse of its operands, while
// 128 x 128 and 256 x 128 tiles do more products per step but leave CUs idle unsplit. Their
// columns go to S = 2, 4 or 8 workgroups with at most one workgroup per CU (tiles * S <= CUs).
// Estimated time of a column split, fitted to sweeps on MI355X (256 .. 1024 tokens, 1024 ..
// 14336 rows and columns, 2:4 and 4:8, each split and tile; within about 15% on the large
// layers): kSplitFixedUs + kSplitRoundUs per further unit of partial loads in the hand-off
// (handoff_units) + kSplitStepScale * (the tile's modelled step time) per 64-column step of a
// split. The same form estimates what runs otherwise (the 64-row split, else the unsplit tile,
// one unit), and a taller split is taken below kTallMargin of that (the margin leaves out the
// shapes where the split measured no faster, e.g. 4096 x 4096 at 768 and 1024 tokens). The
// hand-off's cost follows the partial bytes the last workgroup loads (kSplitRoundUs per unit of
// 32 float4 per lane), not its round trips. Measured (µs, the
// split against what ran before, weights read from memory / resident in the last-level
// cache): 2:4 4096 x 14336 x 512 80 / 71 against 121 / 95 (256 x 128, 4 splits), x 256 51 / 48
// against 65 / 54 (128 x 128, 4 splits); 8192 x 28672 x 256 145 / 132 against 243 / 234;
// 5120 x 25600 x 256 114 / 94 against 210 / 164; 4096 x 4096 x 384 29 / 27 against 36 / 30;
// 4:8 4096 x 14336 x 384 114 / 107 against 135 / 131; 16:32 (128 x 128 only) 4096 x 14336 x 256
// 96 / 94 against 134 / 135, 8192 x 28672 x 256 329 / 320 against 404 / 404.
constexpr int64_t kTallMinTokens = 128;
constexpr double kSplitFixedUs = 7.6;
constexpr double kSplitRoundUs = 3.0;
constexpr double kSplitStepScale = 1.17;
constexpr double kTallMargin = 0.78;
constexpr int kStepsPerBlock = kColBlock / 64;

struct TallPlan {
  int tr = 0, tt = 0, splits = 1, blocks = 0;
  int64_t tiles = 0;   // 0: no taller split
};

const TileCost* mode_tile(int mode, int tr, int tt) {
  const TileCost* c = mode == kPfDirect ? kDirectTiles : mode == kPfSplit ? kSplitTiles : kExpandTiles;
  const int n = mode == kPfDirect ? int(sizeof(kDirectTiles) / sizeof(TileCost))
              : mode == kPfSplit  ? int(sizeof(kSplitTiles) / sizeof(TileCost))
                                  : int(sizeof(kExpandTiles) / sizeof(TileCost));
  for (int i = 0; i < n; ++i)
    if (c[i].tr == tr && c[i].tt == tt) return &c[i];
  return nullptr;
}

// steps: 64-column steps of one workgroup; n: workgroups per CU; units: hand-off load units
double split_estimate_us(int64_t steps, const TileCost& c, int64_t n, int units) {
  return kSplitFixedUs + kSplitRoundUs * double(units - 1) + kSplitStepScale * double(steps) * (c.t1 + double(n - 1) * c.tn);
}

// The partials the last workgroup of a tile loads in the hand-off, in units of 32 float4 per
// lane (a 64 x 64 tile's 8 splits make one unit, a 256 x 128 tile's S splits make S).
int handoff_units(int tr, int tt, int splits) { return (splits * tr * tt + 31) / 32; }

TallPlan tall_plan(int64_t rows, int64_t cols, int64_t tokens, int mode, const DeviceInfo& dev) {
  TallPlan best;
  if (tokens <= kTallMinTokens) return best;
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int64_t nblk = ceil_div(cols, kColBlock);
  double current;
  const ColPlan p = colsplit_plan(rows, cols, tokens, dev);
  const TileCost* small = mode_tile(mode, 1, p.tt);
  if (p.splits > 1 && small != nullptr) {
    current = split_estimate_us(int64_t(p.blocks) * kStepsPerBlock, *small, ceil_div(p.tiles * p.splits, cus),
                                handoff_units(1, p.tt, p.splits));
  } else {
    const TileCost u = sparse_tile(rows, tokens, mode, dev);
    const int64_t grid = ceil_div(rows, 64 * u.tr) * ceil_div(tokens, 16 * u.tt);
    current = split_estimate_us(ceil_div(cols, 64), u, ceil_div(grid, cus), 1);
  }
  double best_t = kTallMargin * current;
  static const int kTall[2][2] = {{2, 8}, {4, 8}};
  for (const auto& tl : kTall) {
    const int tr = tl[0], tt = tl[1];
    if (mode != kPfDirect && tr == 4) continue;   // 256-row tiles: 2:4 only
    const TileCost* c = mode_tile(mode, tr, tt);
    if (c == nullptr) continue;
    const int64_t tiles = ceil_div(rows, 64 * tr) * ceil_div(tokens, 16 * tt);
    for (int s = 2; s <= kMaxColSplits && s <= nblk && tiles * s <= cus; s *= 2) {
      const int blocks = int(ceil_div(nblk, s));
      const int splits = int(ceil_div(nblk, blocks));
      const double t = split_estimate_us(int64_t(blocks) * kStepsPerBlock, *c, 1, handoff_units(tr, tt, splits));
      if (t < best_t) {
        best_t = t;
        best.tr = tr;
        best.tt = tt;
        best.splits = splits;
        best.blocks = blocks;
        best.tiles = tiles;
      }
    }
  }
  return best;
}

size_t tall_bytes(const TallPlan& t, const DeviceInfo& dev) {
  if (t.tiles == 0) return 0;
  return counter_bytes(dev) + size_t(t.tiles) * size_t(t.splits) * size_t(kThreads) * size_t(t.tr) * size_t(t.tt) * 16u;
}

const void* tall_kernel(const TallPlan& t, int mode) {
  if (mode == kPfExpand) return reinterpret_cast<const void*>(&prefill_colsplit_expand_kernel<2, 8, 64, kDepth>);
  if (mode == kPfSplit) return reinterpret_cast<const void*>(&prefill_colsplit_kernel<2, 8, 64, kDepth, true>);
  return t.tr == 2 ? reinterpret_cast<const void*>(&prefill_colsplit_kernel<2, 8, 64, kDepth, false>)
                   : reinterpret_cast<const void*>(&prefill_colsplit_kernel<4, 8, 64, kDepth, false>);
}

const void* colsplit_kernel(int tt, int mode) {
  if (mode == kPfExpand)
    return tt == 2 ? reinterpret_cast<const void*>(&prefill_colsplit_expand_kernel<1, 2, 64, kDepth>)
                   : reinterpret_cast<const void*>(&prefill_colsplit_expand_kernel<1, 4, 64, kDepth>);
  if (mode == kPfSplit)
    return tt == 2 ? reinterpret_cast<const void*>(&prefill_colsplit_kernel<1, 2, 64, kDepth, true>)
                   : reinterpret_cast<const void*>(&prefill_colsplit_kernel<1, 4, 64, kDepth, true>);
  return tt == 2 ? reinterpret_cast<const void*>(&prefill_colsplit_kernel<1, 2, 64, kDepth, false>)
                 : reinterpret_cast<const void*>(&prefill_colsplit_kernel<1, 4, 64, kDepth, false>);
}

}  // namespace

size_t prefill_workspace_bytes(int64_t rows, int64_t cols, int64_t tokens, int n, const DeviceInfo& dev) {
  if (!prefill_fits(rows, cols, tokens)) return 0;
  const TallPlan t = tall_plan(rows, cols, tokens, pf_mode(n), dev);
  if (t.tiles > 0) return tall_bytes(t, dev);
  return colsplit_bytes(colsplit_plan(rows, cols, tokens, dev), dev);
}

hipError_t launch_prefill_spmm(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                               int64_t rows, int64_t cols, int64_t tokens, int n, int m, hipStream_t stream,
                               const DeviceInfo& dev, void* workspace, size_t workspace_bytes) {
  if (!prefill_fits(rows, cols, tokens) || !prefill_pattern(n, m)) return hipErrorInvalidValue;
  int r = int(rows), c = int(cols), t = int(tokens);
  const int mode = pf_mode(n);
  if (workspace != nullptr) {
    const TallPlan tp = tall_plan(rows, cols, tokens, mode, dev);
    if (tp.tiles > 0 && workspace_bytes >= tall_bytes(tp, dev)) {
      int sp = tp.splits, bl = tp.blocks;
      unsigned* cnt = static_cast<unsigned*>(workspace);
      float4* part = reinterpret_cast<float4*>(static_cast<char*>(workspace) + counter_bytes(dev));
      void* cargs[] = {&values, &masks, &X, &Y, &r, &c, &t, &sp, &bl, &part, &cnt};
      return launch(tall_kernel(tp, mode), dim3(unsigned(tp.tiles * tp.splits)), dim3(kThreads), cargs, 0, stream,
                    dev);
    }
  }
  const ColPlan p = colsplit_plan(rows, cols, tokens, dev);
  const size_t need = colsplit_bytes(p, dev);
  if (need > 0 && workspace != nullptr && workspace_bytes >= need) {
    int sp = p.splits, bl = p.blocks;
    unsigned* cnt = static_cast<unsigned*>(workspace);
    float4* part = reinterpret_cast<float4*>(static_cast<char*>(workspace) + counter_bytes(dev));
    void* cargs[] = {&values, &masks, &X, &Y, &r, &c, &t, &sp, &bl, &part, &cnt};
    return launch(colsplit_kernel(p.tt, mode), dim3(unsigned(p.tiles * p.splits)), dim3(kThreads), cargs, 0, stream,
                  dev);
  }
  void* args[] = {&values, &masks, &X, &Y, &r, &c, &t};
  const TileCost tc = sparse_tile(rows, tokens, mode, dev);
  const int64_t grid = ceil_div(rows, 64 * tc.tr) * ceil_div(tokens, 16 * tc.tt);
  return launch(sparse_kernel_of(tc, mode), dim3(unsigned(grid)), dim3(kThreads), args, 0, stream, dev);
}

hipError_t launch_prefill_gemm(const uint16_t* W, const uint16_t* X, uint16_t* Y, int64_t rows, int64_t cols,
                               int64_t tokens, hipStream_t stream, const DeviceInfo& dev) {
  if (!prefill_fits(rows, cols, tokens)) return hipErrorInvalidValue;
  int r = int(rows), c = int(cols), t = int(tokens);
  void* args[] = {&W, &X, &Y, &r, &c, &t};
  if (use_large<DenseLarge>(rows, tokens, dev))
    return launch(reinterpret_cast<const void*>(&prefill_gemm_kernel<2, 16, 64, kDepth>),
                  dim3(unsigned(workgroups<DenseLarge>(rows, tokens))), dim3(kThreads), args, 0, stream, dev);
  return launch(reinterpret_cast<const void*>(&prefill_gemm_kernel<1, 4, 64, kDepth>),
                dim3(unsigned(workgroups<Small>(rows, tokens))), dim3(kThreads), args, 0, stream, dev);
}

const char* prefill_colsplit_variant(int64_t rows, int64_t cols, int64_t tokens, const DeviceInfo& dev, int n) {
  const int mode = pf_mode(n);
  const TallPlan t = tall_plan(rows, cols, tokens, mode, dev);
  if (t.tiles > 0) {
    if (mode == kPfExpand) return "prefill_colsplit_expand_kernel<2, 8, 64, 2>";
    if (mode == kPfSplit) return "prefill_colsplit_kernel<2, 8, 64, 2, true>";
    return t.tr == 2 ? "prefill_colsplit_kernel<2, 8, 64, 2, false>" : "prefill_colsplit_kernel<4, 8, 64, 2, false>";
  }
  const ColPlan p = colsplit_plan(rows, cols, tokens, dev);
  if (p.splits == 1) return "";
  if (mode == kPfExpand)
    return p.tt == 2 ? "prefill_colsplit_expand_kernel<1, 2, 64, 2>" : "prefill_colsplit_expand_kernel<1, 4, 64, 2>";
  if (mode == kPfSplit)
    return p.tt == 2 ? "prefill_colsplit_kernel<1, 2, 64, 2, true>" : "prefill_colsplit_kernel<1, 4, 64, 2, true>";
  return p.tt == 2 ? "prefill_colsplit_kernel<1, 2, 64, 2, false>" : "prefill_colsplit_kernel<1, 4, 64, 2, false>";
}

const char* prefill_variant(int64_t rows, int64_t tokens, bool sparse, const DeviceInfo& dev, int n) {
  if (sparse) {
    static const char* const kNames[3][5][3] = {
        {{"prefill_spmm_kernel<1, 4, 64, 2>", "prefill_spmm_kernel<1, 8, 64, 2>", ""},
         {"prefill_spmm_kernel<2, 4, 64, 2>", "prefill_spmm_kernel<2, 8, 64, 2>", ""},
         {"", "", ""},
         {"prefill_spmm_kernel<4, 8, 64, 2>", "prefill_spmm_kernel<4, 16, 64, 2>", ""},
         {"", "", ""}},
        {{"prefill_split_kernel<1, 4, 64, 2>", "prefill_split_kernel<1, 8, 64, 2>", ""},
         {"prefill_split_kernel<2, 4, 64, 2>", "prefill_split_kernel<2, 8, 64, 2>", "prefill_split_kernel<2, 16, 64, 2>"},
         {"", "", ""},
         {"prefill_split_kernel<4, 8, 64, 2>", "prefill_split_kernel<4, 16, 64, 2>", ""},
         {"", "", ""}},
        {{"prefill_expand_kernel<1, 4, 64, 2>", "prefill_expand_kernel<1, 8, 64, 2>",
          "prefill_expand_kernel<1, 16, 64, 2>"},
         {"prefill_expand_kernel<2, 4, 64, 2>", "prefill_expand_kernel<2, 8, 64, 2>",
          "prefill_expand_kernel<2, 16, 64, 2>"},
         {"", "", ""},
         {"prefill_expand_kernel<4, 8, 64, 2>", "prefill_expand_kernel<4, 16, 64, 2>", ""},
         {"", "", ""}}};
    const int mode = pf_mode(n);
    const TileCost t = sparse_tile(rows, tokens, mode, dev);
    const int col = t.tr == 4 ? (t.tt == 8 ? 0 : 1) : t.tr == 1 ? (t.tt == 4 ? 0 : t.tt == 8 ? 1 : 2)
                                                  : (t.tt == 4 ? 0 : t.tt == 8 ? 1 : 2);
    return kNames[mode][t.tr - 1][col];
  }
  return use_large<DenseLarge>(rows, tokens, dev) ? "prefill_gemm_kernel<2, 16, 64, 2>"
                                                  : "prefill_gemm_kernel<1, 4, 64, 2>";
}

}  // namespace nm
