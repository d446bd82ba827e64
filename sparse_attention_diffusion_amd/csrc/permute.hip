// Row reorder of [BH, N, row] tensors: gather (dst row i = src row perm[i])
// or its inverse scatter (dst row perm[i] = src row i).  Used to put Q, K and
// V into a locality-preserving token order before 64-token blocking, and the
// output back (HilbertA blog page, section "Introducing HilbertA": the reorder
// happens once before and once after the denoising steps).
//
// HBM-bound copy: one lane per 16-byte chunk, a row's chunks in consecutive
// lanes, so every gathered row is read as whole cache lines and every store is
// coalesced.  perm entries are clamped to [0, N) (a list that is not a
// permutation gives an unspecified result but stays in bounds).
#include "internal.h"

namespace rettn {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) permute_kernel(PermuteArgs a) {
  const uint64_t t = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  const uint64_t rows = (uint64_t)a.BH * (uint32_t)a.N;
  if (t >= rows * (uint32_t)a.cpr) return;
  const uint64_t row = t / (uint32_t)a.cpr;
  const int c = (int)(t - row * (uint32_t)a.cpr);
  const uint64_t bh = row / (uint32_t)a.N;
  const int i = (int)(row - bh * (uint32_t)a.N);
  const int j = min(max(a.perm[i], 0), a.N - 1);
  const uint64_t from = a.inverse ? row : bh * (uint32_t)a.N + (uint32_t)j;
  const uint64_t to = a.inverse ? bh * (uint32_t)a.N + (uint32_t)j : row;
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)a.src + from * (uint32_t)a.cpr + c);
  __builtin_nontemporal_store(v, (u32x4*)a.dst + to * (uint32_t)a.cpr + c);
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const uint64_t total = (uint64_t)a.BH * (uint32_t)a.N * (uint32_t)a.cpr;
  const uint64_t blocks = (total + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(permute_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rettn
