// Float32 calibration and sparse-reshape attention on the vector ALUs.
//
// Same method and the same statistics as the bf16 MFMA kernels (Re-ttention
// project page, teaser and core-mechanism paragraphs), for float32 workloads.
// One workgroup (one wave) per 64-row query block; each lane owns one query
// row; the K and V rows of the current key block sit in LDS and are read by
// broadcast.  Meant for small float32 problems where exactness matters more
// than speed.
#include "internal.h"

namespace rettn {
namespace {

constexpr int kThreads = 64;

template <int D, AttnMode MODE>
__global__ void __launch_bounds__(kThreads) attn_f32_kernel(AttnArgs a, XcdGrid grid) {
  __shared__ float lk[kBlock][D];
  __shared__ float lv[kBlock][D];
  __shared__ int seq[kMaxBlocks];
  __shared__ unsigned char flags[kMaxBlocks];

  const uint32_t lin = grid.linear(blockIdx.x);
  if (lin >= grid.total) return;
  const int Nb = a.Nb, N = a.N, keep = a.keep;
  const int bh = lin / Nb, qi = lin % Nb;
  const int lane = threadIdx.x;
  const size_t head = (size_t)bh * N * D;
  const float* qh = (const float*)a.q + head;
  const float* kh = (const float*)a.k + head;
  const float* vh = (const float*)a.v + head;
  const int32_t* list = a.idx + ((size_t)bh * Nb + qi) * keep;

  // The row is read as a set: blocks are walked from a flag row, kept ones
  // first (ascending), then (calibration) the masked ones, so a repeated or
  // unordered entry counts once, as in every other kernel.
  for (int n = lane; n < Nb; n += kThreads) flags[n] = 0;
  __syncthreads();
  for (int n = lane; n < keep; n += kThreads) flags[min(max(list[n], 0), Nb - 1)] = 1;
  __syncthreads();
  int nkept = 0;
  for (int base = 0; base < Nb; base += 64) {
    const int j = base + lane;
    const bool f = j < Nb && flags[j];
    const unsigned long long mk = __ballot(f);
    if (f) seq[nkept + __popcll(mk & ((1ull << lane) - 1ull))] = j;
    nkept += __popcll(mk);
  }
  int nseq = nkept;
  if (MODE == AttnMode::kCalibrate) {
    for (int base = 0; base < Nb; base += 64) {
      const int j = base + lane;
      const bool f = j < Nb && !flags[j];
      const unsigned long long mk = __ballot(f);
      if (f) seq[nseq + __popcll(mk & ((1ull << lane) - 1ull))] = j;
      nseq += __popcll(mk);
    }
    if (a.idx_cache != nullptr) {
      int32_t* dst = a.idx_cache + ((size_t)bh * Nb + qi) * keep;
      for (int n = lane; n < keep; n += kThreads) dst[n] = list[n];
    }
  }
  __syncthreads();

  const int row = qi * kBlock + lane;
  const bool row_ok = row < N;
  float q[D], o[D], ok[MODE == AttnMode::kCalibrate ? D : 1];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = row_ok ? qh[(size_t)row * D + d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, z = 0.f, m_kept = 0.f, z_kept = 0.f;
  const float alpha = a.alpha;

  for (int n = 0; n < nseq; ++n) {
    const int j = __builtin_amdgcn_readfirstlane(seq[n]);
    __syncthreads();
    {
      const int key = min(j * kBlock + lane, N - 1);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        lk[lane][d] = kh[(size_t)key * D + d];
        lv[lane][d] = vh[(size_t)key * D + d];
      }
    }
    __syncthreads();
    if (MODE == AttnMode::kCalibrate && n == nkept) {
#pragma unroll
      for (int d = 0; d < D; ++d) { ok[d] = o[d]; o[d] = 0.f; }
      m_kept = m;
      z_kept = z;
      z = 0.f;
    }
    const int nvalid = min(kBlock, N - j * kBlock);
    for (int t = 0; t < nvalid; ++t) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], lk[t][d], acc);
      const float sc = acc * alpha;
      if (sc > m) {  // new running max: rescale what has been accumulated
        const float corr = m == -INFINITY ? 0.f : expf(m - sc);
        z *= corr;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= corr;
        m = sc;
      }
      const float p = expf(sc - m);
      z += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, lv[t][d], o[d]);
    }
  }

  if (!row_ok) return;
  const size_t srow = (size_t)bh * N + row;
  float* orow = (float*)a.o + srow * D;
  if (MODE == AttnMode::kCalibrate) {
    if (nseq == nkept) {
#pragma unroll
      for (int d = 0; d < D; ++d) { ok[d] = o[d]; o[d] = 0.f; }
      m_kept = m;
      z_kept = z;
      z = 0.f;
    }
    const float corr = expf(m_kept - m);
    const float zs = z_kept * corr;
    const float zf = zs + z;
    a.m[srow] = m;
    a.z_full[srow] = zf;
    a.z_sparse[srow] = zs;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      a.R[residual_index(bh, a.Nb, D, row, d)] = o[d];
      orow[d] = (ok[d] * corr + o[d]) / zf;
    }
  } else if (a.variant == 1) {  // R2: r * O_sparse + R / Z_full
    const float zf_c = a.z_full[srow], zs_c = a.z_sparse[srow];
    const float w = zs_c / (zf_c * z);
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = fmaf(o[d], w, a.R[residual_index(bh, a.Nb, D, row, d)] / zf_c);
  } else {
    const float m_c = a.m[srow], zf_c = a.z_full[srow], zs_c = a.z_sparse[srow];
    const float big = fmaxf(m, m_c);
    const float e1 = expf(m - big), e2 = expf(m_c - big);
    const float den = z * e1 * zf_c / zs_c;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = (o[d] * e1 + a.R[residual_index(bh, a.Nb, D, row, d)] * e2) / den;
  }
}

template <int D, AttnMode MODE>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  XcdGrid grid = make_xcd_grid((uint32_t)a.BH * (uint32_t)a.Nb);
  hipLaunchKernelGGL((attn_f32_kernel<D, MODE>), dim3(grid.grid()), dim3(kThreads), 0, s, a, grid);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(AttnMode mode, int D, const AttnArgs& a, hipStream_t s) {
  if (D == 64) return mode == AttnMode::kCalibrate ? launch_one<64, AttnMode::kCalibrate>(a, s)
                                                   : launch_one<64, AttnMode::kSparse>(a, s);
  if (D == 80) return mode == AttnMode::kCalibrate ? launch_one<80, AttnMode::kCalibrate>(a, s)
                                                   : launch_one<80, AttnMode::kSparse>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace rettn
