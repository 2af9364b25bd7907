// Dense fp16 matrix-vector product y = W x on gfx950: the same-GPU baseline the
// sparse product is measured against (aimodeling.com SparseDecoding article, "The
// Kernel Is the Other Half of the Answer", quotes every speedup against dense).
//
// It is tuned the same way as the sparse kernel so that the ratio is fair: one
// workgroup = 16 rows x all columns with kWaves waves splitting the columns; per
// step each row's 64 bytes (32 columns) are loaded by 4 lanes as dwordx4; x is
// staged once in LDS and read back as 16-byte vectors (4 distinct addresses per
// wave instruction, broadcast); fp16 pairs are multiplied and summed in fp32 by
// v_dot2_f32_f16; rows are reduced with DPP inside the quad and in LDS across
// waves, in a fixed order, and rounded once to fp16.
#include "nm_internal.h"

namespace nm {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kBatch = 8;

__device__ __forceinline__ float dpp_quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  return v;
}

__device__ __forceinline__ float dot8(uint4 w, uint4 xv, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.x), __builtin_bit_cast(half2_t, xv.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.y), __builtin_bit_cast(half2_t, xv.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.z), __builtin_bit_cast(half2_t, xv.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.w), __builtin_bit_cast(half2_t, xv.w), acc, false);
  return acc;
}

__global__ __launch_bounds__(64 * kWaves) void nm_gemv_kernel(const uint4* __restrict__ W,
                                                              const uint4* __restrict__ x,
                                                              uint16_t* __restrict__ y, int rows,
                                                              int cols) {
  extern __shared__ uint4 lds[];
  float* red = reinterpret_cast<float*>(lds + (cols >> 3));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int u = lane & 3;
  const int row0 = blockIdx.x * kRowsPerBlock;
  const int r = min(row0 + (lane >> 2), rows - 1);

  const int steps = cols >> 5;  // 32 columns of every row per step
  const int s_beg = int((int64_t(steps) * wave) / kWaves);
  const int s_end = int((int64_t(steps) * (wave + 1)) / kWaves);
  const uint4* __restrict__ wrow = W + size_t(r) * size_t(cols >> 3);

  const int n16 = cols >> 3;
  for (int i = tid; i < n16; i += 64 * kWaves) lds[i] = x[i];
  __syncthreads();

  float acc = 0.f;
  for (int s = s_beg; s < s_end; s += kBatch) {
    uint4 wv[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (s + i < s_end) wv[i] = wrow[4 * (s + i) + u];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (s + i < s_end) acc = dot8(wv[i], lds[4 * (s + i) + u], acc);
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

}  // namespace

hipError_t launch_gemv(const uint16_t* W, const uint16_t* x, uint16_t* y, int64_t rows,
                       int64_t cols, hipStream_t stream, const DeviceInfo& dev) {
  (void)dev;
  const uint4* w4 = reinterpret_cast<const uint4*>(W);
  const uint4* x4 = reinterpret_cast<const uint4*>(x);
  int r = int(rows), c = int(cols);
  void* args[] = {&w4, &x4, &y, &r, &c};
  const dim3 grid((r + kRowsPerBlock - 1) / kRowsPerBlock);
  const size_t lds = size_t(c) * 2 + reduction_lds_bytes(kWaves);
  return launch(reinterpret_cast<const void*>(&nm_gemv_kernel), grid, dim3(64 * kWaves), args, lds,
                stream);
}

}  // namespace nm
