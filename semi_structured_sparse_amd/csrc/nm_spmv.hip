// nm_spmv launcher: picks the kernel configuration for the shape and launches it.
// The kernels themselves (and the description of the method and the work mapping)
// are in nm_spmv_impl.h.
#include "nm_spmv_impl.h"

namespace nm {
namespace {

using namespace spmv_detail;

constexpr bool kNTV = true;  // values stream once, a whole 128-byte line per instruction
constexpr int kBatch = 4;    // steps whose loads are issued together

// Workgroup shape: RG row groups of 8 rows x CS waves splitting the columns. Narrow
// layers (few rows) use 8-row workgroups so that more CUs get work.
template <int N, int DEC, int RG, int CS>
hipError_t launch_cfg(const uint16_t* values, const uint32_t* masks, const uint16_t* x, uint16_t* y,
                      int rows, int cols, hipStream_t stream, const DeviceInfo& dev) {
  const uint4* v4 = reinterpret_cast<const uint4*>(values);
  const uint4* x4 = reinterpret_cast<const uint4*>(x);
  void* args[] = {&v4, &masks, &x4, &y, &rows, &cols};
  const dim3 grid((rows + 8 * RG - 1) / (8 * RG));
  return launch(reinterpret_cast<const void*>(&spmv_line_kernel<N, RG, CS, kBatch, kNTV, DEC>), grid,
                dim3(64 * RG * CS), args, line_lds_bytes<DEC>(cols, RG * CS), stream, dev);
}

// Narrow layers (at most this many rows) use 8-row workgroups, the others 16-row ones.
constexpr int kNarrowRows = 2048;

template <int N, int DEC>
hipError_t launch_shape(const uint16_t* values, const uint32_t* masks, const uint16_t* x, uint16_t* y,
                        int rows, int cols, hipStream_t stream, const DeviceInfo& dev) {
  if (rows <= kNarrowRows) return launch_cfg<N, DEC, 1, 8>(values, masks, x, y, rows, cols, stream, dev);
  return launch_cfg<N, DEC, 2, 8>(values, masks, x, y, rows, cols, stream, dev);
}

constexpr int kMaxWaves = 16;  // largest workgroup the launcher uses (2 x 8 waves)

bool use_pair_table(int N, int64_t cols, const DeviceInfo& dev) {
  return N == 2 && line_lds_bytes<kPairTable>(int(cols), kMaxWaves) <= size_t(dev.max_lds_per_block);
}

bool use_rev_walk(int64_t cols, const DeviceInfo& dev) {
  return line_lds_bytes<kRevWalk>(int(cols), kMaxWaves) <= size_t(dev.max_lds_per_block);
}

bool use_byte_lut(int64_t cols, const DeviceInfo& dev) {
  return line_lds_bytes<kByteLut>(int(cols), kMaxWaves) <= size_t(dev.max_lds_per_block);
}

}  // namespace

int64_t max_cols_for(const DeviceInfo& dev) {
  // the bit-walk kernel (2 bytes of LDS per column) bounds the accepted width
  const int64_t avail = int64_t(dev.max_lds_per_block) - int64_t(line_lds_bytes<kBitWalk>(0, kMaxWaves));
  if (avail <= 0) return 0;
  return (avail / 2) / 32 * 32;
}

const char* spmv_variant(int64_t rows, int64_t cols, int N, const DeviceInfo& dev) {
  // one string per (pattern, decoder, workgroup shape); they spell the template arguments
  // of spmv_line_kernel<N, RG, CS, BATCH, NTV, DEC> as profilers print them
  static const char* const names[4][3][2] = {
      {{"spmv_line_kernel<2, 1, 8, 4, true, 0>", "spmv_line_kernel<2, 2, 8, 4, true, 0>"},
       {"spmv_line_kernel<2, 1, 8, 4, true, 1>", "spmv_line_kernel<2, 2, 8, 4, true, 1>"}, {"", ""}},
      {{"spmv_line_kernel<4, 1, 8, 4, true, 0>", "spmv_line_kernel<4, 2, 8, 4, true, 0>"}, {"", ""},
       {"spmv_line_kernel<4, 1, 8, 4, true, 2>", "spmv_line_kernel<4, 2, 8, 4, true, 2>"}},
      {{"spmv_line_kernel<8, 1, 8, 4, true, 0>", "spmv_line_kernel<8, 2, 8, 4, true, 0>"}, {"", ""},
       {"spmv_line_kernel<8, 1, 8, 4, true, 2>", "spmv_line_kernel<8, 2, 8, 4, true, 2>"}},
      {{"spmv_line_kernel<16, 1, 8, 4, true, 0>", "spmv_line_kernel<16, 2, 8, 4, true, 0>"}, {"", ""},
       {"spmv_line_kernel<16, 1, 8, 4, true, 3>", "spmv_line_kernel<16, 2, 8, 4, true, 3>"}},
  };
  static_assert(kBatch == 4 && kNTV, "variant names spell BATCH = 4 and NTV = true");
  const int pi = N == 2 ? 0 : N == 4 ? 1 : N == 8 ? 2 : 3;
  const int di = N == 2 ? (use_pair_table(N, cols, dev) ? 1 : 0)
               : (N == 4 || N == 8) ? (use_byte_lut(cols, dev) ? 2 : 0)
                                    : (use_rev_walk(cols, dev) ? 2 : 0);
  return names[pi][di][rows <= kNarrowRows ? 0 : 1];
}

hipError_t launch_spmv(const uint16_t* values, const uint32_t* masks, const uint16_t* x,
                       uint16_t* y, int64_t rows, int64_t cols, int N, int M, hipStream_t stream,
                       const DeviceInfo& dev) {
  (void)M;  // validated together with N: M == 2 * N
  const int r = int(rows), c = int(cols);
  switch (N) {
    case 2:
      // 2:4 uses the x pair table (6 bytes of LDS per column) whenever it fits
      if (use_pair_table(N, cols, dev)) return launch_shape<2, kPairTable>(values, masks, x, y, r, c, stream, dev);
      return launch_shape<2, kBitWalk>(values, masks, x, y, r, c, stream, dev);
    case 4:
      if (use_byte_lut(cols, dev)) return launch_shape<4, kByteLut>(values, masks, x, y, r, c, stream, dev);
      return launch_shape<4, kBitWalk>(values, masks, x, y, r, c, stream, dev);
    case 8:
      if (use_byte_lut(cols, dev)) return launch_shape<8, kByteLut>(values, masks, x, y, r, c, stream, dev);
      return launch_shape<8, kBitWalk>(values, masks, x, y, r, c, stream, dev);
    case 16:
      if (use_rev_walk(cols, dev)) return launch_shape<16, kRevWalk>(values, masks, x, y, r, c, stream, dev);
      return launch_shape<16, kBitWalk>(values, masks, x, y, r, c, stream, dev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nm
