// Batch-one N:M sparse matrix-vector product y = W x on gfx950.
//
// Method (pages: news.bitwarelabs.com "SparseDecoding: decoding-aware pruning for
// accurate and fast LLM generation", "What's new"; aimodeling.com SparseDecoding
// article, "The Kernel Is the Other Half of the Answer"): the weights are read once
// per product, so the kernel is bound by HBM bandwidth; a 32-bit mask word indexes 32
// input columns and carries exactly 16 kept values at 50% density, so the values of
// word w start at a fixed offset 16*w and the traversal of a word is a fixed number
// of find-lowest-set-bit steps with no prefix scan.
//
// Work mapping (one workgroup = 16 rows x all columns, KS waves):
//   * A "step" covers 64 columns (2 mask words) of every row of the tile. In one step
//     each row's 64 bytes of packed values are split over 4 lanes: lane u of the row
//     loads one 16-byte dwordx4 holding 8 values, the half h = u & 1 of word
//     2*step + (u >> 1). The 16 rows x 4 lanes fill the 64 lanes of a wave, and a
//     wave's consecutive steps walk each row 64 bytes at a time.
//   * The KS waves split the steps of the row range evenly (contiguous ranges) and
//     their partial sums are combined in LDS in a fixed order.
//   * x is staged once per workgroup in LDS; each kept value gathers its x with one
//     16-bit LDS read. In one wave instruction the 32 lanes of a half-wave touch at
//     most two adjacent mask words, i.e. 32 consecutive dwords of x, so the gathers
//     hit 32 distinct banks or broadcast: no bank conflicts.
//   * For 2:4, 4:8 and 8:16 each 16-column half of a word holds exactly 8 kept
//     columns, so the lane owning half h walks the set bits of (mask & half h). For
//     16:32 the lane with the low 8 values walks the lowest 8 set bits and the lane
//     with the high 8 values first clears the lowest 8 set bits.
//   * Products are fp16 x fp16 (exact in fp32) accumulated in fp32 by v_dot2_f32_f16
//     on pairs, reduced across the row's 4 lanes with DPP, then across waves in LDS,
//     and rounded once to fp16.
#include "nm_internal.h"

namespace nm {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;   // waves per workgroup (column split)
constexpr int kBatch = 8;   // steps whose loads are issued together

__device__ __forceinline__ float dpp_quad_sum(float v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of a quad ends with the quad's sum.
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  return v;
}

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

// Gathers the x values of this lane's 8 kept columns: `bits` holds the columns as set
// bits relative to xw, the x window of the mask word, and xp[k] receives the pair for
// values 2k and 2k+1. Bit 31 is kept set as a sentinel so that a malformed (short)
// mask still reads inside the window.
__device__ __forceinline__ void gather_x(uint32_t bits, const _Float16* __restrict__ xw,
                                         half2_t (&xp)[4]) {
  bits |= 0x80000000u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t p0 = __builtin_ctz(bits);
    bits = (bits & (bits - 1)) | 0x80000000u;
    const uint32_t p1 = __builtin_ctz(bits);
    bits = (bits & (bits - 1)) | 0x80000000u;
    xp[k].x = xw[p0];
    xp[k].y = xw[p1];
  }
}

// acc += the 8 products of the lane's values (4 fp16 pairs in v) with their x pairs.
__device__ __forceinline__ float dot_half_word(uint4 v, const half2_t (&xp)[4], float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.x), xp[0], acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.y), xp[1], acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.z), xp[2], acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.w), xp[3], acc, false);
  return acc;
}

__device__ __forceinline__ float half_word(uint4 v, uint32_t bits, const _Float16* __restrict__ xw,
                                           float acc) {
  half2_t xp[4];
  gather_x(bits, xw, xp);
  return dot_half_word(v, xp, acc);
}

template <int N, int M>
__global__ __launch_bounds__(64 * kWaves) void nm_spmv_kernel(
    const uint4* __restrict__ values, const uint32_t* __restrict__ masks,
    const uint4* __restrict__ x, uint16_t* __restrict__ y, int rows, int cols) {
  extern __shared__ uint4 lds[];
  _Float16* xs = reinterpret_cast<_Float16*>(lds);
  float* red = reinterpret_cast<float*>(lds + (cols >> 3));

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
  const int s_beg = int((int64_t(steps) * wave) / kWaves);
  const int s_end = int((int64_t(steps) * (wave + 1)) / kWaves);
  const int s_main = min(s_end, full_steps);

  const uint4* __restrict__ vrow = values + size_t(r) * unsigned(cols >> 4);
  const uint32_t* __restrict__ mrow = masks + size_t(r) * unsigned(words);
  const uint32_t keep_high = half ? 0xFFFF0000u : 0xFFFFFFFFu;

  // Stage x in LDS.
  const int n16 = cols >> 3;
  for (int i = tid; i < n16; i += 64 * kWaves) lds[i] = x[i];
  __syncthreads();

  float part[4] = {0.f, 0.f, 0.f, 0.f};
  // Per step the lane's values advance 64 bytes (4 x uint4), its mask 2 words and its
  // x window 64 columns.
  const uint4* __restrict__ vp = vrow + 4 * unsigned(s_beg) + unsigned(u);
  const uint32_t* __restrict__ mp = mrow + 2 * unsigned(s_beg) + unsigned(wsel);
  const _Float16* xw = xs + 64 * unsigned(s_beg) + 32 * unsigned(wsel);
  int n = s_main - s_beg;
  for (; n >= kBatch; n -= kBatch) {
    uint4 v[kBatch];
    uint32_t m[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      v[i] = vp[4 * i];
      m[i] = mp[2 * i];
    }
    // Gather phase for the whole batch first, so that many LDS reads are in flight,
    // then the products into independent partial sums.
    half2_t xp[kBatch][4];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) gather_x(lane_bits<N>(m[i], half, keep_high), xw + 64 * i, xp[i]);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) part[i & 3] = dot_half_word(v[i], xp[i], part[i & 3]);
    vp += 4 * kBatch;
    mp += 2 * kBatch;
    xw += 64 * kBatch;
  }
  float acc = (part[0] + part[1]) + (part[2] + part[3]);
  if (n > 0) {  // fewer than kBatch full steps left (n is wave-uniform)
    uint4 v[kBatch];
    uint32_t m[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (i < n) {
        v[i] = vp[4 * i];
        m[i] = mp[2 * i];
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (i < n) acc = half_word(v[i], lane_bits<N>(m[i], half, keep_high), xw + 64 * i, acc);
  }
  // Odd word count: the last step holds a single word, owned by the lanes with wsel == 0.
  if (s_end > full_steps && wsel == 0) {
    const unsigned w = 2 * unsigned(full_steps);
    const uint4 v = vrow[2 * w + unsigned(u)];
    const uint32_t m = mrow[w];
    acc = half_word(v, lane_bits<N>(m, half, keep_high), xs + 32 * w, acc);
  }

  acc = dpp_quad_sum(acc);
  if (u == 0) red[wave * kRowsPerBlock + (lane >> 2)] = acc;
  __syncthreads();
  if (tid < kRowsPerBlock) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) t += red[k * kRowsPerBlock + tid];
    const int rr = row0 + tid;
    if (rr < rows) y[rr] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(t));
  }
}

template <int N, int M>
hipError_t launch_spmv_t(const uint16_t* values, const uint32_t* masks, const uint16_t* x,
                         uint16_t* y, int rows, int cols, hipStream_t stream) {
  const uint4* v4 = reinterpret_cast<const uint4*>(values);
  const uint4* x4 = reinterpret_cast<const uint4*>(x);
  void* args[] = {&v4, &masks, &x4, &y, &rows, &cols};
  const dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  const size_t lds = size_t(cols) * 2 + reduction_lds_bytes(kWaves);
  return launch(reinterpret_cast<const void*>(&nm_spmv_kernel<N, M>), grid, dim3(64 * kWaves), args,
                lds, stream);
}

}  // namespace

int64_t max_cols_for(const DeviceInfo& dev) {
  const int64_t avail = int64_t(dev.max_lds_per_block) - int64_t(reduction_lds_bytes(kWaves));
  if (avail <= 0) return 0;
  return (avail / 2) / 32 * 32;
}

hipError_t launch_spmv(const uint16_t* values, const uint32_t* masks, const uint16_t* x,
                       uint16_t* y, int64_t rows, int64_t cols, int N, int M, hipStream_t stream,
                       const DeviceInfo& dev) {
  (void)dev;
  (void)M;  // validated together with N: M == 2 * N
  const int r = int(rows), c = int(cols);
  switch (N) {
    case 2: return launch_spmv_t<2, 4>(values, masks, x, y, r, c, stream);
    case 4: return launch_spmv_t<4, 8>(values, masks, x, y, r, c, stream);
    case 8: return launch_spmv_t<8, 16>(values, masks, x, y, r, c, stream);
    case 16: return launch_spmv_t<16, 32>(values, masks, x, y, r, c, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nm
