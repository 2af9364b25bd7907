// N:M encoder on gfx950: dense fp16 W -> (values, masks).
//
// Format (news.bitwarelabs.com "SparseDecoding: decoding-aware pruning for accurate
// and fast LLM generation", "What's new": N of every M consecutive weights are kept;
// aimodeling.com SparseDecoding article, "The Kernel Is the Other Half of the
// Answer": one 32-bit mask word per 32 input columns, 16 set bits at 50%).
// Selection: in each aligned group of M columns keep the N largest magnitudes, the
// magnitude being the fp16 bit pattern with the sign cleared; equal magnitudes go
// to the lower column.
//
// One thread encodes one mask word. Because W is row-major with 32 fp16 per word,
// word t (row-major over rows x words) is exactly W[32t, 32t+32), its values are
// values[V t, V t + V) with V = 32 N / M kept values per word (16 at 50% density, 8 at
// 25%) and its mask is masks[t], so the encoder is a flat map over words. Each weight gets the integer key (magnitude << 5) | (31 - column in group):
// keys are distinct inside a group and larger means "wins", so an element is kept
// iff fewer than N members of its group have a larger key. The kept fp16 bits are
// then compacted in ascending column order through a private LDS slot.
#include "nm_internal.h"

namespace nm {
namespace {

constexpr int kPackThreads = 256;
constexpr int kSlot = 17;  // dwords per thread in LDS (16 + 1 to spread banks)

template <int N, int M>
__global__ __launch_bounds__(kPackThreads) void nm_pack_kernel(const uint4* __restrict__ W,
                                                               uint4* __restrict__ values,
                                                               uint32_t* __restrict__ masks,
                                                               int64_t total_words) {
  __shared__ uint32_t slot_all[kPackThreads * kSlot];
  uint32_t* slot = slot_all + threadIdx.x * kSlot;
  const int64_t stride = int64_t(gridDim.x) * kPackThreads;
  for (int64_t t = int64_t(blockIdx.x) * kPackThreads + threadIdx.x; t < total_words; t += stride) {
    uint32_t d[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 a = W[4 * t + q];
      d[4 * q + 0] = a.x;
      d[4 * q + 1] = a.y;
      d[4 * q + 2] = a.z;
      d[4 * q + 3] = a.w;
    }
    uint32_t key[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t bits = (d[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      key[i] = ((bits & 0x7FFFu) << 5) | uint32_t(31 - (i % M));
    }
    uint32_t mask = 0;
#pragma unroll
    for (int g = 0; g < 32 / M; ++g) {
#pragma unroll
      for (int i = 0; i < M; ++i) {
        int larger = 0;
#pragma unroll
        for (int k = 0; k < M; ++k) larger += (key[g * M + k] > key[g * M + i]) ? 1 : 0;
        if (larger < N) mask |= 1u << (g * M + i);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) slot[i] = d[i];
    constexpr int V = 32 * N / M;  // kept values per word
    uint32_t out[V / 2];
    uint32_t rest = mask;
#pragma unroll
    for (int k = 0; k < V / 2; ++k) {
      const uint32_t p0 = __builtin_ctz(rest | 0x80000000u);
      rest &= rest - 1;
      const uint32_t p1 = __builtin_ctz(rest | 0x80000000u);
      rest &= rest - 1;
      const uint32_t lo = (slot[p0 >> 1] >> (16 * (p0 & 1))) & 0xFFFFu;
      const uint32_t hi = (slot[p1 >> 1] >> (16 * (p1 & 1))) & 0xFFFFu;
      out[k] = lo | (hi << 16);
    }
#pragma unroll
    for (int q = 0; q < V / 8; ++q)
      values[(V / 8) * t + q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
    masks[t] = mask;
  }
}

// Decoder, the inverse of the encoder: one thread writes the 32 dense fp16 of one mask
// word, taking the kept values in ascending column order (the value of set bit j is the
// one after all set bits below j) and +0 for dropped columns. The word's V values go
// through a private LDS slot so that the running index can address them; a mask with
// more than V set bits reuses the last value (unspecified result, no access outside the
// slot).
template <int V>
__global__ __launch_bounds__(kPackThreads) void nm_unpack_kernel(const uint4* __restrict__ values,
                                                                 const uint32_t* __restrict__ masks,
                                                                 uint4* __restrict__ W, int64_t total_words) {
  constexpr int kSlotU = V / 2 + 1;
  __shared__ uint32_t slot_all[kPackThreads * kSlotU];
  uint32_t* slot = slot_all + threadIdx.x * kSlotU;
  const int64_t stride = int64_t(gridDim.x) * kPackThreads;
  for (int64_t t = int64_t(blockIdx.x) * kPackThreads + threadIdx.x; t < total_words; t += stride) {
#pragma unroll
    for (int q = 0; q < V / 8; ++q) {
      const uint4 a = values[(V / 8) * t + q];
      slot[4 * q + 0] = a.x;
      slot[4 * q + 1] = a.y;
      slot[4 * q + 2] = a.z;
      slot[4 * q + 3] = a.w;
    }
    const uint32_t m = masks[t];
    uint32_t out[16];
    uint32_t k = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t b = (m >> j) & 1u;
      const uint32_t kk = k < uint32_t(V - 1) ? k : uint32_t(V - 1);
      const uint32_t h = b ? (slot[kk >> 1] >> (16 * (kk & 1))) & 0xFFFFu : 0u;
      k += b;
      if (j & 1)
        out[j >> 1] |= h << 16;
      else
        out[j >> 1] = h;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) W[4 * t + q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
  }
}

template <int V>
hipError_t launch_unpack_t(const uint16_t* values, const uint32_t* masks, uint16_t* W, int64_t words,
                           hipStream_t stream, const DeviceInfo& dev) {
  const uint4* v4 = reinterpret_cast<const uint4*>(values);
  uint4* w4 = reinterpret_cast<uint4*>(W);
  void* args[] = {&v4, &masks, &w4, &words};
  int64_t blocks = (words + kPackThreads - 1) / kPackThreads;
  const int64_t cap = int64_t(dev.cu_count > 0 ? dev.cu_count : 256) * 32;
  if (blocks > cap) blocks = cap;
  return launch(reinterpret_cast<const void*>(&nm_unpack_kernel<V>), dim3(unsigned(blocks)), dim3(kPackThreads),
                args, 0, stream, dev);
}

template <int N, int M>
hipError_t launch_pack_t(const uint16_t* W, uint16_t* values, uint32_t* masks, int64_t words,
                         hipStream_t stream, const DeviceInfo& dev) {
  const uint4* w4 = reinterpret_cast<const uint4*>(W);
  uint4* v4 = reinterpret_cast<uint4*>(values);
  void* args[] = {&w4, &v4, &masks, &words};
  int64_t blocks = (words + kPackThreads - 1) / kPackThreads;
  const int64_t cap = int64_t(dev.cu_count > 0 ? dev.cu_count : 256) * 32;
  if (blocks > cap) blocks = cap;
  return launch(reinterpret_cast<const void*>(&nm_pack_kernel<N, M>), dim3(unsigned(blocks)),
                dim3(kPackThreads), args, 0, stream, dev);
}

}  // namespace

hipError_t launch_unpack(const uint16_t* values, const uint32_t* masks, uint16_t* W, int64_t rows, int64_t cols,
                         int N, int M, hipStream_t stream, const DeviceInfo& dev) {
  const int64_t words = rows * (cols / 32);
  return M == 2 * N ? launch_unpack_t<16>(values, masks, W, words, stream, dev)
                    : launch_unpack_t<8>(values, masks, W, words, stream, dev);
}

hipError_t launch_pack(const uint16_t* W, uint16_t* values, uint32_t* masks, int64_t rows,
                       int64_t cols, int N, int M, hipStream_t stream, const DeviceInfo& dev) {
  const int64_t words = rows * (cols / 32);
  if (M == 2 * N) {  // 50%
    switch (N) {
      case 2: return launch_pack_t<2, 4>(W, values, masks, words, stream, dev);
      case 4: return launch_pack_t<4, 8>(W, values, masks, words, stream, dev);
      case 8: return launch_pack_t<8, 16>(W, values, masks, words, stream, dev);
      case 16: return launch_pack_t<16, 32>(W, values, masks, words, stream, dev);
      default: return hipErrorInvalidValue;
    }
  }
  switch (N) {  // 25%: M == 4 * N
    case 1: return launch_pack_t<1, 4>(W, values, masks, words, stream, dev);
    case 2: return launch_pack_t<2, 8>(W, values, masks, words, stream, dev);
    case 4: return launch_pack_t<4, 16>(W, values, masks, words, stream, dev);
    case 8: return launch_pack_t<8, 32>(W, values, masks, words, stream, dev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nm
