// Launcher of the small-batch 50% products on the matrix instructions (1..16 tokens): 2:4
// directly, 4:8 and 8:16 split into two 2:4 operands, 16:32 expanded to dense fragments. The
// kernels are in nm_skinny_impl.h.
#include <algorithm>

#include "nm_internal.h"
#include "nm_skinny_impl.h"

namespace nm {

using namespace skinny_detail;

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct SkinnyShape {
  int rg = 1, cs = 16, phase_cols = 128;
  int splits = 1;   // workgroups per row group's columns (with a workspace)
  int64_t grid = 0;
  size_t lds = 0;
};

// Workgroup shape: 16 waves, RG = ceil(tiles / CUs) row groups of 16 rows with CS =
// floor(16 / RG) waves splitting the columns (RG * CS <= 16 waves own rows), so that the
// grid is as close to one workgroup per CU as whole row groups allow: 17408 rows take 218
// workgroups of 5 x 3 waves, where a power-of-two RG (8 x 2) would leave 120 CUs idle. X is
// staged in column phases of at most 128 KiB (and the device's per-workgroup LDS, less the
// tables the pattern needs).
int mode_of(int n) { return n == 2 ? kModeDirect : n == 16 ? kModeExpand : kModeSplit; }

size_t lead_of(int mode) {
  return mode == kModeSplit ? lead_bytes<kModeSplit>() : mode == kModeExpand ? lead_bytes<kModeExpand>() : 0;
}

size_t x_budget(int mode, const DeviceInfo& dev) {
  const size_t lds = size_t(dev.max_lds_per_block > 0 ? dev.max_lds_per_block : 65536);
  const size_t lead = lead_of(mode);
  const size_t avail = lds > lead ? lds - lead : 0;
  return std::min<size_t>(kMaxXBytes, avail);
}

// Column splits: a layer of at most half as many 16-row tiles as CUs (1024 rows: 64 tiles)
// leaves most CUs idle, so with a workspace its columns can go to S = 2, 4 or 8 workgroups per
// tile (S * tiles <= CUs, at least 2 lines per split), whose partial tiles the last of them
// sums (SplitWs). The hand-off (partial store, count, the last workgroup's loads) costs about
// 1.3 us, so a split is taken where it measured faster on MI355X (1024 x 4096 at 16 vectors
// 2:4: 8.4 us unsplit, 8.7 split; 1024 x 8192: 13.3 against 9.3; 1024 x 14336: 22.3 against
// 10.8): rows of at least 64 lines; at least 40 lines from 8 vectors with S >= 4; the split
// patterns' slower lines from 9 vectors with S >= 4. Not for 16:32 (its expansion kernel
// has no split).
int splits_for(int64_t tiles, int64_t cols, int tokens, int mode, const DeviceInfo& dev) {
  if (mode == kModeExpand) return 1;
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int64_t lines = ceil_div(cols, 128);
  int s = 1;
  while (s < kMaxSplits && tiles * (2 * s) <= cus && lines >= int64_t(2) * (2 * s)) s *= 2;
  const bool pays = lines >= 64 || (s >= 4 && lines >= 40 && tokens >= 8) ||
                    (s >= 4 && mode == kModeSplit && tokens >= 9);
  return pays ? s : 1;
}

SkinnyShape skinny_shape(int64_t rows, int64_t cols, int tokens, int mode, const DeviceInfo& dev,
                         bool with_ws = false) {
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int64_t tiles = ceil_div(rows, 16);
  const int64_t want = std::min<int64_t>(kMaxWaves, std::max<int64_t>(1, ceil_div(tiles, cus)));
  SkinnyShape s;
  s.rg = int(want);
  s.cs = kMaxWaves / s.rg;
  s.splits = with_ws && s.rg == 1 ? splits_for(tiles, cols, tokens, mode, dev) : 1;
  s.grid = ceil_div(tiles, s.rg) * s.splits;
  // phases of whole 128-column lines (the loads of the 2:4 and split kernels cover lines)
  const int64_t pc_max = int64_t(x_budget(mode, dev) / (2 * size_t(tokens))) / 128 * 128;
  s.phase_cols = int(std::min<int64_t>(pc_max, ceil_div(cols, 128) * 128));
  s.lds = std::max(lead_of(mode) + x_bytes(tokens, s.phase_cols), red_bytes(kMaxWaves));
  return s;
}

}  // namespace

bool skinny_pattern(int n, int m) { return 2 * n == m && (n == 2 || n == 4 || n == 8 || n == 16); }

bool skinny_fits(int64_t rows, int64_t cols, int64_t tokens, int n, int m, const DeviceInfo& dev) {
  // byte offsets inside a workgroup's slices are 32-bit; X of one phase must fit LDS
  if (!skinny_pattern(n, m) || tokens < 1 || tokens > kMaxTokens || cols > kPrefillMaxCols) return false;
  return x_budget(mode_of(n), dev) >= 2 * size_t(tokens) * 128 && ceil_div(rows, 16) <= INT32_MAX;
}

bool use_skinny(int64_t rows, int64_t cols, int64_t batch, int n, int m, const DeviceInfo& dev) {
  if (batch < kSkinnyMinBatch || batch > kSkinnyBatch)   // per launch of at most 16 vectors
    return false;
  if (rows < kSkinnySmallMinRows || !skinny_fits(rows, cols, kSkinnyBatch, n, m, dev)) return false;
  if (n == 16) return false;   // routed per launch (skinny_expand_chunk)
  if (rows >= kSkinnyMinRows || n == 2) return true;
  return batch >= 12 || (batch >= 9 && cols <= 5120);   // the split patterns on smaller layers
}

// From a sweep at 12..31 vectors on MI355X (16:32, µs per product): a launch of 14..16
// vectors takes about as long as one of 12, and as one of 5, while the small-batch kernel pays
// per 8 vectors: at 16 vectors 4096 x 14336 runs in 42.4 against 53.3 µs, 4096 x 8192 24.9
// against 32.8, 8192 x 8192 38.2 against 48.7, 2048 x 4096 14.7 against 15.9; at 12 vectors
// the expansion wins only with X in one phase (<= 4096 columns) on >= 4096 rows (4096 x 4096:
// 15.4 against 18.9), and on 1024-row layers, or 2048 rows of more than 4096 columns, it
// loses or ties at every count.
bool skinny_expand_chunk(int64_t rows, int64_t cols, int64_t tokens, const DeviceInfo& dev) {
  if (rows < kSkinnySmallMinRows || !skinny_fits(rows, cols, kSkinnyBatch, 16, 32, dev)) return false;
  if (tokens >= kSkinnyExpandFullChunk && rows >= kSkinnyExpandFullMinRows &&
      (rows >= kSkinnyExpandMinRows || cols <= kSkinnyExpandMaxCols))
    return true;
  return tokens >= kSkinnyExpandMinBatch && rows >= kSkinnyExpandMinRows && cols <= kSkinnyExpandMaxCols;
}

const char* skinny_variant(int n) {
  return n == 2 ? "skinny_spmm_kernel<1, false>" : n == 16 ? "skinny_expand_kernel<1>" : "skinny_spmm_kernel<1, true>";
}

// The workspace: one counter per tile in a region of fixed size on a device (4 bytes per
// CU, rounded up to 256: a split layer has fewer tiles than CUs), so that every shape finds
// its counters where the previous calls left zeros; then one 1 KiB fp32 partial per tile
// and split.
size_t counter_bytes(const DeviceInfo& dev) {
  return size_t(ceil_div(4 * int64_t(dev.cu_count > 0 ? dev.cu_count : 256), 256) * 256);
}

size_t skinny_workspace_bytes(int64_t rows, int64_t cols, int tokens, int n, const DeviceInfo& dev) {
  const int64_t tiles = ceil_div(rows, 16);
  if (ceil_div(tiles, dev.cu_count > 0 ? dev.cu_count : 256) > 1) return 0;
  const int splits = splits_for(tiles, cols, tokens, mode_of(n), dev);
  if (splits == 1) return 0;
  return counter_bytes(dev) + size_t(tiles) * size_t(splits) * 1024u;
}

hipError_t launch_skinny_spmm(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                              int64_t rows, int64_t cols, int tokens, int n, int m, hipStream_t stream,
                              const DeviceInfo& dev, void* workspace, size_t workspace_bytes) {
  if (!skinny_fits(rows, cols, tokens, n, m, dev)) return hipErrorInvalidValue;
  const int mode = mode_of(n);
  const size_t need = skinny_workspace_bytes(rows, cols, tokens, n, dev);
  const bool split = need > 0 && workspace != nullptr && workspace_bytes >= need;
  const SkinnyShape s = skinny_shape(rows, cols, tokens, mode, dev, split);
  int r = int(rows), c = int(cols), t = tokens, rg = s.rg, cs = s.cs, pc = s.phase_cols, sp = s.splits;
  unsigned* cnt = split ? static_cast<unsigned*>(workspace) : nullptr;
  float4* part = split ? reinterpret_cast<float4*>(static_cast<char*>(workspace) + counter_bytes(dev)) : nullptr;
  if (mode == kModeExpand) {
    void* args[] = {&values, &masks, &X, &Y, &r, &c, &t, &rg, &cs, &pc};
    return launch(reinterpret_cast<const void*>(&skinny_expand_kernel<1>), dim3(unsigned(s.grid)),
                  dim3(kThreadsFixed), args, s.lds, stream, dev);
  }
  if (s.splits > 1) {
    void* args[] = {&values, &masks, &X, &Y, &r, &c, &t, &cs, &pc, &sp, &part, &cnt};
    const void* k = mode == kModeSplit ? reinterpret_cast<const void*>(&skinny_colsplit_kernel<true>)
                                       : reinterpret_cast<const void*>(&skinny_colsplit_kernel<false>);
    return launch(k, dim3(unsigned(s.grid)), dim3(kThreadsFixed), args, s.lds, stream, dev);
  }
  void* args[] = {&values, &masks, &X, &Y, &r, &c, &t, &rg, &cs, &pc};
  const void* k = mode == kModeSplit ? reinterpret_cast<const void*>(&skinny_spmm_kernel<1, true>)
                                     : reinterpret_cast<const void*>(&skinny_spmm_kernel<1, false>);
  return launch(k, dim3(unsigned(s.grid)), dim3(kThreadsFixed), args, s.lds, stream, dev);
}

}  // namespace nm
