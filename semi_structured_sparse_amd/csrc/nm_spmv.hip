// nm_spmv launcher: picks the decoder and the workgroup shape for the shape of W and
// launches spmv_kernel (nm_spmv_impl.h holds the kernel and the description of the
// method and of the work mapping).
#include <algorithm>

#include "nm_spmv_impl.h"

namespace nm {
namespace {

using namespace spmv_detail;

constexpr bool kNTV = true;  // values stream once, a whole 128-byte line per instruction
constexpr int kBatch = 4;    // steps whose loads are issued together

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Decoder for the pattern: the table-driven one when its LDS image fits one workgroup,
// else the bit walk (2 bytes of LDS per column).
int pick_decoder(int N, int64_t cols, const DeviceInfo& dev) {
  const size_t cap = size_t(dev.max_lds_per_block);
  const int c = int(cols);
  switch (N) {
    case 2: return lds_bytes<kPairTable>(c) <= cap ? kPairTable : kBitWalk;
    case 4:
    case 8: return lds_bytes<kByteLut>(c) <= cap ? kByteLut : kBitWalk;
    default: return lds_bytes<kRevWalk>(c) <= cap ? kRevWalk : kBitWalk;
  }
}

// Workgroup shape from the row count and the row length in steps (128 columns = 128
// bytes of packed values), measured on MI355X over the Llama / Qwen projection shapes
// (1024..28672 rows, 4096..28672 columns, all four patterns; rows per workgroup 1..56,
// 2..16 waves per row group): within 1.0% of the best shape per layer on average, 7% at
// worst. Every rule keeps the grid a near-multiple of the CU count, so that each CU
// streams the same number of rows.
//   * long rows (more than 64 steps): one workgroup of at most 40 rows per CU in each pass over the CUs,
//     about 12 waves (3..12 per row group). Each workgroup stages all of x, so fewer,
//     taller workgroups spend less on staging, and the long rows give every wave many
//     steps;
//   * narrow layers (at most 8 rows per CU): a few rows per workgroup and about 4 steps per
//     wave, to spread the little work over all CUs;
//   * otherwise: about 8 rows per workgroup (balanced over the CUs) and 8 waves per row.
WorkgroupShape workgroup_shape(int64_t rows, int64_t steps, const DeviceInfo& dev) {
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  WorkgroupShape s;
  if (steps > 64) {
    const int64_t rounds = ceil_div(rows, cus * 40);
    s.rpb = int(ceil_div(rows, cus * rounds));
    const int rg = int(ceil_div(s.rpb, 8));
    s.cs = rg >= 4 ? 3 : 12 / rg;
    if (rg * s.cs > kMaxWaves) s.cs = kMaxWaves / rg;
  } else if (rows <= 8 * cus) {
    s.rpb = int(std::min<int64_t>(8, ceil_div(rows, cus)));
    s.cs = int(std::min<int64_t>(16, ceil_div(steps, 4)));
  } else {
    s.rpb = int(ceil_div(rows, cus * ceil_div(rows, 8 * cus)));
    s.cs = steps < 32 ? int(ceil_div(steps, 4)) : 8;
  }
  s.row_groups = int(ceil_div(s.rpb, 8));
  s.grid = ceil_div(rows, s.rpb);
  return s;
}

// The kernel for a shape's column ranges per wave: the narrow kernel serves the 16:32
// reversed walk only (the bit walk, which narrow layers never need on this GPU, and the
// other patterns take spmv_kernel, which suits any wave count).
template <int N, int DEC>
const void* kernel_for(int ci) {
  if constexpr (DEC != kRevWalk) {
    (void)ci;
    return reinterpret_cast<const void*>(&spmv_kernel<N, kBatch, kNTV, DEC>);
  } else {
    switch (ci) {
      case 2: return reinterpret_cast<const void*>(&spmv_narrow_kernel<N, kBatch, kNTV, DEC, 2>);
      case 4: return reinterpret_cast<const void*>(&spmv_narrow_kernel<N, kBatch, kNTV, DEC, 4>);
      case 8: return reinterpret_cast<const void*>(&spmv_narrow_kernel<N, kBatch, kNTV, DEC, 8>);
      default: return reinterpret_cast<const void*>(&spmv_kernel<N, kBatch, kNTV, DEC>);
    }
  }
}

template <int N, int DEC>
hipError_t launch_kernel(const uint16_t* values, const uint32_t* masks, const uint16_t* x, uint16_t* y,
                         int rows, int cols, const WorkgroupShape& s, hipStream_t stream, const DeviceInfo& dev) {
  const uint4* v4 = reinterpret_cast<const uint4*>(values);
  const uint4* x4 = reinterpret_cast<const uint4*>(x);
  int rpb = s.rpb, cs = s.cs;
  void* args[] = {&v4, &masks, &x4, &y, &rows, &cols, &rpb, &cs};
  return launch(kernel_for<N, DEC>(s.ci), dim3(unsigned(s.grid)), dim3(unsigned(64 * s.row_groups * s.cs)), args,
                lds_bytes<DEC>(cols), stream, dev);
}

}  // namespace

int64_t max_cols_for(const DeviceInfo& dev) {
  // the bit-walk kernel (2 bytes of LDS per column) bounds the accepted width
  const int64_t avail = int64_t(dev.max_lds_per_block) - int64_t(lds_bytes<kBitWalk>(0));
  if (avail <= 0) return 0;
  return (avail / 2) / 32 * 32;
}

// 50% patterns: 128 columns = 128 bytes of values per step. Narrow 16:32 layers (at most 8
// rows per CU, at most 64 steps per row) whose workgroups hold 1, 2 or 4 rows take the narrow
// kernel when every lane can get exactly one batch: CI = 8 / rows column ranges per wave of
// 4 whole steps each, steps / (4 CI) waves. Measured on MI355X on the 1024-row Llama and Qwen
// layers: 4-8% faster for 16:32, whose decoder does the most vector work per value; within
// +-3% (run-to-run spread) for the table decoders of 2:4, 4:8 and 8:16, which keep the
// kernel whose spare lanes repeat the last row.
WorkgroupShape spmv_shape(int64_t rows, int64_t cols, int N, const DeviceInfo& dev) {
  const int64_t steps = ceil_div(cols, 128);
  WorkgroupShape s = workgroup_shape(rows, steps, dev);
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const bool narrow = steps <= 64 && rows <= 8 * cus;  // the rule's narrow-layer class
  if (N == 16 && narrow && s.rpb < 8 && 8 % s.rpb == 0 && cols % 128 == 0) {
    const int ci = 8 / s.rpb;
    if (steps % (int64_t(kBatch) * ci) == 0) {
      s.ci = ci;
      s.cs = int(steps / (int64_t(kBatch) * ci));
    }
  }
  return s;
}

// 25% density: 256 columns = 128 bytes of values per step.
WorkgroupShape spmv_quarter_shape(int64_t rows, int64_t cols, const DeviceInfo& dev) {
  return workgroup_shape(rows, ceil_div(cols, 256), dev);
}

const char* spmv_variant(int64_t rows, int64_t cols, int N, int M, const DeviceInfo& dev) {
  if (M == 4 * N) return "spmv_quarter_kernel<4, true>";
  const int pi = N == 2 ? 0 : N == 4 ? 1 : N == 8 ? 2 : 3;
  const int dec = pick_decoder(N, cols, dev);
  const int ci = spmv_shape(rows, cols, N, dev).ci;
  if (ci > 1 && dec == kRevWalk) {
    // spmv_narrow_kernel<16, BATCH, NTV, kRevWalk, CI>
    static const char* const narrow[3] = {"spmv_narrow_kernel<16, 4, true, 3, 2>",
                                          "spmv_narrow_kernel<16, 4, true, 3, 4>",
                                          "spmv_narrow_kernel<16, 4, true, 3, 8>"};
    return narrow[ci == 2 ? 0 : ci == 4 ? 1 : 2];
  }
  // one string per (pattern, decoder): the template arguments of
  // spmv_kernel<N, BATCH, NTV, DEC> as profilers print them
  static const char* const names[4][4] = {
      {"spmv_kernel<2, 4, true, 0>", "spmv_kernel<2, 4, true, 1>", "", ""},
      {"spmv_kernel<4, 4, true, 0>", "", "spmv_kernel<4, 4, true, 2>", ""},
      {"spmv_kernel<8, 4, true, 0>", "", "spmv_kernel<8, 4, true, 2>", ""},
      {"spmv_kernel<16, 4, true, 0>", "", "", "spmv_kernel<16, 4, true, 3>"},
  };
  static_assert(kBatch == 4 && kNTV, "variant names spell BATCH = 4 and NTV = true");
  return names[pi][dec];
}

hipError_t launch_spmv(const uint16_t* values, const uint32_t* masks, const uint16_t* x,
                       uint16_t* y, int64_t rows, int64_t cols, int N, int M, hipStream_t stream,
                       const DeviceInfo& dev) {
  const int r = int(rows), c = int(cols);
  if (M == 4 * N) {  // 25% density: one kernel for 1:4, 2:8, 4:16 and 8:32
    const WorkgroupShape q = spmv_quarter_shape(rows, cols, dev);
    const uint4* v4 = reinterpret_cast<const uint4*>(values);
    const uint4* x4 = reinterpret_cast<const uint4*>(x);
    int rr = r, cc = c, rpb = q.rpb, cs = q.cs;
    void* args[] = {&v4, &masks, &x4, &y, &rr, &cc, &rpb, &cs};
    return launch(reinterpret_cast<const void*>(&spmv_quarter_kernel<kBatch, kNTV>), dim3(unsigned(q.grid)),
                  dim3(unsigned(64 * q.row_groups * q.cs)), args, lds_bytes<kBitWalk>(c), stream, dev);
  }
  const WorkgroupShape s = spmv_shape(rows, cols, N, dev);
  const int dec = pick_decoder(N, cols, dev);
  switch (N) {
    case 2:
      if (dec == kPairTable) return launch_kernel<2, kPairTable>(values, masks, x, y, r, c, s, stream, dev);
      return launch_kernel<2, kBitWalk>(values, masks, x, y, r, c, s, stream, dev);
    case 4:
      if (dec == kByteLut) return launch_kernel<4, kByteLut>(values, masks, x, y, r, c, s, stream, dev);
      return launch_kernel<4, kBitWalk>(values, masks, x, y, r, c, s, stream, dev);
    case 8:
      if (dec == kByteLut) return launch_kernel<8, kByteLut>(values, masks, x, y, r, c, s, stream, dev);
      return launch_kernel<8, kBitWalk>(values, masks, x, y, r, c, s, stream, dev);
    case 16:
      if (dec == kRevWalk) return launch_kernel<16, kRevWalk>(values, masks, x, y, r, c, s, stream, dev);
      return launch_kernel<16, kBitWalk>(values, masks, x, y, r, c, s, stream, dev);
    default: return hipErrorInvalidValue;
  }
}

// Products sharing x in one launch of spmv_group_kernel when the columns are at most 64
// steps (every workgroup one row group), the pattern is a 50% one with its table decoder,
// and there are at most kMaxGroup products: all take the workgroup shape the rule gives
// their rows together (as if their rows were concatenated), so that small products do not
// run workgroups whose lanes repeat rows. A row's summation order depends on the wave count
// only, not on the rows per workgroup, so a product's y is bit-identical to a separate
// launch of spmv_kernel whenever the rule gives that product alone the same wave count (for
// example every product of 4096 columns: 8 waves). Otherwise one nm_spmv launch per product.
static_assert(kMaxGroup == kMaxSpmvGroup, "one group size for the kernel and the ABI");

hipError_t launch_spmv_group(int count, const uint16_t* const* values, const uint32_t* const* masks,
                             const uint16_t* x, uint16_t* const* y, const int64_t* rows, int64_t cols, int N,
                             int M, hipStream_t stream, const DeviceInfo& dev) {
  if (count == 1) return launch_spmv(values[0], masks[0], x, y[0], rows[0], cols, N, M, stream, dev);
  const int64_t steps = ceil_div(cols, 128);
  const int dec = pick_decoder(N, cols, dev);
  bool one = M == 2 * N && steps <= 64 && count <= kMaxGroup && dec != kBitWalk;
  GroupArgs a{};
  int64_t grid = 0;
  if (one) {
    int64_t total = 0;
    for (int k = 0; k < count; ++k) total += rows[k];
    const WorkgroupShape s = workgroup_shape(total, steps, dev);
    if (s.row_groups != 1) one = false;
    a.cs = s.cs;
    a.rpb = s.rpb;
    for (int k = 0; k < count && one; ++k) {
      a.block0[k] = int(grid);
      grid += ceil_div(rows[k], s.rpb);
      a.values[k] = reinterpret_cast<const uint4*>(values[k]);
      a.masks[k] = masks[k];
      a.y[k] = y[k];
      a.rows[k] = int(rows[k]);
    }
    if (grid > (int64_t(1) << 31) - 1) one = false;
  }
  if (!one) {
    for (int k = 0; k < count; ++k) {
      const hipError_t e = launch_spmv(values[k], masks[k], x, y[k], rows[k], cols, N, M, stream, dev);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  a.block0[count] = int(grid);
  a.x = reinterpret_cast<const uint4*>(x);
  a.cols = int(cols);
  a.count = count;
  void* args[] = {&a};
  const void* fn = nullptr;
  size_t lds = 0;
  switch (N) {
    case 2: fn = reinterpret_cast<const void*>(&spmv_group_kernel<2, kBatch, kNTV, kPairTable>);
            lds = lds_bytes<kPairTable>(int(cols)); break;
    case 4: fn = reinterpret_cast<const void*>(&spmv_group_kernel<4, kBatch, kNTV, kByteLut>);
            lds = lds_bytes<kByteLut>(int(cols)); break;
    case 8: fn = reinterpret_cast<const void*>(&spmv_group_kernel<8, kBatch, kNTV, kByteLut>);
            lds = lds_bytes<kByteLut>(int(cols)); break;
    case 16: fn = reinterpret_cast<const void*>(&spmv_group_kernel<16, kBatch, kNTV, kRevWalk>);
             lds = lds_bytes<kRevWalk>(int(cols)); break;
    default: return hipErrorInvalidValue;
  }
  return launch(fn, dim3(unsigned(grid)), dim3(unsigned(64 * a.cs)), args, lds, stream, dev);
}

}  // namespace nm
