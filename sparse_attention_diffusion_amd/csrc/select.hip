// Block selector: mean-pooled Q/K per 64-token block, pooled logits, and a
// per-query-block top-k with always-kept (forced) blocks.
//
// Method: the Re-ttention project page keeps only a small subset of the tokens
// (Abstract: as few as 3.1%).  How the subset is chosen is not spelled out
// there; this library scores 64-token blocks by the scaled dot product of
// their mean query and mean key and keeps, per query block, the forced blocks
// plus the best remaining ones (ties to the lower block index).
//
// Kernels
//   pool_kernel   : one wave per (tensor, bh, block); float32 sums in token order.
//   select_kernel : one wave per (bh, query block); float32 scores, then a
//                   bitonic sort of (score, index) keys in LDS and an ascending
//                   compaction of the winners with wave ballots.
#include "internal.h"

namespace rettn {
namespace {

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

// grid.x: (bh, block) pairs laid out per XCD; grid.y: 0 = q, 1 = k.
template <typename T, int D>
__global__ void __launch_bounds__(64) pool_kernel(SelectArgs a, XcdGrid grid) {
  const uint32_t lin = grid.linear(blockIdx.x);
  if (lin >= grid.total) return;
  const int Nb = a.Nb, N = a.N;
  const int bh = lin / Nb, i = lin % Nb;
  const T* x = (const T*)(blockIdx.y == 0 ? a.q : a.k) + (size_t)bh * N * D;
  float* out = (blockIdx.y == 0 ? a.qb : a.kb) + ((size_t)bh * Nb + i) * D;
  const int r0 = i * kBlock, r1 = min(N, r0 + kBlock);
  for (int d = threadIdx.x; d < D; d += 64) {
    float acc = 0.f;
    for (int r = r0; r < r1; ++r) acc += to_f32<T>(x[(size_t)r * D + d]);
    out[d] = acc / (float)(r1 - r0);
  }
}

// Order-preserving map of a float32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int D>
__global__ void __launch_bounds__(64) select_kernel(SelectArgs a, XcdGrid grid) {
  __shared__ unsigned long long keys[kMaxBlocks];
  __shared__ float qrow[D];
  __shared__ unsigned char flags[kMaxBlocks];

  const uint32_t lin = grid.linear(blockIdx.x);
  if (lin >= grid.total) return;
  const int Nb = a.Nb, keep = a.keep;
  const int bh = lin / Nb, i = lin % Nb;
  const int lane = threadIdx.x;
  const float* kb = a.kb + (size_t)bh * Nb * D;
  for (int d = lane; d < D; d += 64) qrow[d] = a.qb[((size_t)bh * Nb + i) * D + d];
  int P = 64;
  while (P < Nb) P <<= 1;
  __syncthreads();

  float* srow = a.scores ? a.scores + ((size_t)bh * Nb + i) * Nb : nullptr;
  for (int j = lane; j < P; j += 64) {
    unsigned long long key = 0ull;  // padding sorts last
    if (j < Nb) {
      float acc = 0.f;
      const float* kr = kb + (size_t)j * D;
#pragma unroll 8
      for (int d = 0; d < D; ++d) acc = fmaf(qrow[d], kr[d], acc);
      float s = acc * a.alpha + 0.0f;  // + 0 turns -0 into +0: equal scores compare equal
      if (srow) srow[j] = s;
      const bool forced = (a.forced[j >> 5] >> (j & 31)) & 1u;
      const uint32_t hi = forced ? 0xFFFFFFFFu : order_key(s);
      key = ((unsigned long long)hi << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)j);
    }
    keys[j] = key;
  }
  __syncthreads();

  // Bitonic sort of P keys, descending.
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = lane; t < (P >> 1); t += 64) {
        const int lo = (t / j) * 2 * j + (t % j);
        const int hi = lo + j;
        const unsigned long long x = keys[lo], y = keys[hi];
        const bool desc = (lo & k) == 0;
        if ((x < y) == desc) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  for (int j = lane; j < Nb; j += 64) flags[j] = 0;
  __syncthreads();
  for (int t = lane; t < keep; t += 64) flags[0xFFFFFFFFu - (uint32_t)(keys[t] & 0xFFFFFFFFull)] = 1;
  __syncthreads();
  int32_t* out = a.idx + ((size_t)bh * Nb + i) * keep;
  int cnt = 0;
  for (int base = 0; base < Nb; base += 64) {
    const int j = base + lane;
    const bool f = j < Nb && flags[j];
    const unsigned long long mk = __ballot(f);
    if (f) out[cnt + __popcll(mk & ((1ull << lane) - 1ull))] = j;
    cnt += __popcll(mk);
  }
}

template <typename T, int D>
hipError_t launch_typed(const SelectArgs& a, hipStream_t s) {
  XcdGrid grid = make_xcd_grid((uint32_t)a.BH * (uint32_t)a.Nb);
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3(grid.grid(), 2), dim3(64), 0, s, a, grid);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((select_kernel<D>), dim3(grid.grid()), dim3(64), 0, s, a, grid);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(bool bf16, int D, const SelectArgs& a, hipStream_t s) {
  if (D == 64) return bf16 ? launch_typed<__bf16, 64>(a, s) : launch_typed<float, 64>(a, s);
  if (D == 80) return bf16 ? launch_typed<__bf16, 80>(a, s) : launch_typed<float, 80>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace rettn
