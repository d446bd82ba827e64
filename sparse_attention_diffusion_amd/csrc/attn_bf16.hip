// Flash attention on bf16 MFMA (gfx950) for the calibration step and for the
// sparse step with the statistical reshape epilogue.
//
// Method: Re-ttention project page ("Re-ttention: Ultra Sparse Visual
// Generation via Attention Statistical Reshape").  The calibration step runs
// full attention and records, per query row, the softmax max m, the full and
// sparse denominators and the residual of the masked-out keys (core-mechanism
// paragraph); the sparse step attends to the kept key blocks only and rescales
// its result with those cached statistics (teaser paragraph).
//
// Work decomposition.  One workgroup = one 64-row query block of one (b, h);
// two waves of 32 rows each.  Per key block (64 keys) a wave computes
//   S^T (64 keys x 32 rows) = K . Q^T   with v_mfma_f32_32x32x16_bf16, and
//   O^T (D x 32 rows)      += V^T . P^T  with the same instruction,
// so that every lane owns one query row (lane % 32) in both results and the
// row statistics never leave the lane (only lanes l and l^32 exchange the max).
// K and V tiles are staged in LDS (XOR-swizzled 16-byte units); V^T operands
// are read with ds_read_b64_tr_b16.  Calibration processes the kept blocks
// first, snapshots that partial result, then accumulates the masked blocks:
// one pass, one running max, no second accumulator inside the loop.
#include "internal.h"

namespace rettn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 128;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Shape {
  static constexpr int KS = D / 16;             // k-steps of the d contraction
  static constexpr int NT = (D + 31) / 32;      // 32-wide d tiles of O^T
  static constexpr int UNITS = D / 8;           // 16-byte units per row in HBM
  static constexpr int RSU = D == 64 ? 8 : 12;  // LDS row stride in units (80: 2 zero units)
  static constexpr int TILE = kBlock * RSU * 16;
  static constexpr int PER_THREAD = kBlock * UNITS / kThreads;
  static_assert(D == 64 || D == 80, "head dim");
  static_assert(kBlock * UNITS % kThreads == 0, "tile split");
};

// Physical 16-byte unit of logical unit u in LDS row r.  Units 0..7 are
// XOR-swizzled so that 16 consecutive rows read at one unit, and 4 consecutive
// rows read at 4 aligned units, fall in distinct bank groups.
__device__ __forceinline__ int phys_unit(int r, int u) {
  int f = (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  return u < 8 ? (u ^ f) : u;
}

template <int D>
__device__ __forceinline__ int lds_off(int r, int u) {
  return (r * Shape<D>::RSU + phys_unit(r, u)) * 16;
}

template <int D>
struct Tile {
  u32x4 k[Shape<D>::PER_THREAD];
  u32x4 v[Shape<D>::PER_THREAD];
};

// Global -> registers for key block j (rows past N are clamped to row N-1;
// their scores are masked later, so only finiteness matters).
template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& t, const char* kbase, const char* vbase, int j, int N) {
  constexpr int U = Shape<D>::UNITS;
#pragma unroll
  for (int n = 0; n < Shape<D>::PER_THREAD; ++n) {
    int e = threadIdx.x + n * kThreads;
    int r = e / U, u = e % U;
    int key = min(j * kBlock + r, N - 1);
    size_t off = ((size_t)key * D + u * 8) * 2;
    t.k[n] = *(const u32x4*)(kbase + off);
    t.v[n] = *(const u32x4*)(vbase + off);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const Tile<D>& t, char* lk, char* lv) {
  constexpr int U = Shape<D>::UNITS;
#pragma unroll
  for (int n = 0; n < Shape<D>::PER_THREAD; ++n) {
    int e = threadIdx.x + n * kThreads;
    int r = e / U, u = e % U;
    *(u32x4*)(lk + lds_off<D>(r, u)) = t.k[n];
    *(u32x4*)(lv + lds_off<D>(r, u)) = t.v[n];
  }
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

template <int D>
struct WaveState {
  bf16x8 q[Shape<D>::KS];      // Q^T operand: row lane%32, d = 16s + 8g + 0..7
  f32x16 o[Shape<D>::NT];      // O^T accumulator: row lane%32, d = 32t + 8(i/4) + 4g + i%4
  float m_raw;                 // running max of raw scores q.k (common to lanes l, l^32)
  float z;                     // this lane's partial denominator (its half of the keys)
};

// One key block for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
template <int D>
__device__ __forceinline__ void attend_block(WaveState<D>& st, const char* lk, const char* lv, int nvalid,
                                             float c) {
  constexpr int KS = Shape<D>::KS, NT = Shape<D>::NT;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5, l32 = lane & 31;
  f32x16 s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s[t] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 a = *(const bf16x8*)(lk + lds_off<D>(32 * t + l32, 2 * ks + g));
      s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.q[ks], s[t], 0, 0, 0);
    }
  }
  if (nvalid < kBlock) {  // ragged last key block: keys >= N do not exist
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        int key = 32 * t + (i >> 2) * 8 + 4 * g + (i & 3);
        if (key >= nvalid) s[t][i] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
  mx = fmaxf(mx, xor32(mx));
  const float m_new = fmaxf(st.m_raw, mx);
  if (__ballot(m_new > st.m_raw) != 0ull) {
    const float corr = st.m_raw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st.m_raw - m_new) * c);
    st.z *= corr;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[t][i] *= corr;
    st.m_raw = m_new;
  }
  const float mc = m_new * c;
  bf16x8 p[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float e = __builtin_amdgcn_exp2f(fmaf(s[t][i], c, -mc));
      st.z += e;
      p[t][i >> 3][i & 7] = (__bf16)e;
    }
  // O^T += V^T P^T.  k-step (t, hs) covers keys 32t + 16hs + 0..15; lane group g
  // holds slots j <-> key 32t + 16hs + 8(j/4) + 4g + j%4 in both operands.
  const int G = lane >> 4, i16 = lane & 15;
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        s16x4 h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          int key = 32 * t + 16 * hs + 8 * hh + 4 * g + (i16 >> 2);
          int doff = 32 * dt + 16 * (G & 1) + 4 * (i16 & 3);  // element offset in the row
          int off = lds_off<D>(key, doff >> 3) + (doff & 7) * 2;
          h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(lv + off));
        }
        const s16x8 both = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 a = __builtin_bit_cast(bf16x8, both);
        st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[t][hs], st.o[dt], 0, 0, 0);
      }
  }
}

template <int D, AttnMode MODE>
__global__ void __launch_bounds__(kThreads) attn_bf16_kernel(AttnArgs a, XcdGrid grid) {
  constexpr int NT = Shape<D>::NT, KS = Shape<D>::KS, TILE = Shape<D>::TILE;
  __shared__ __attribute__((aligned(16))) char lds_k[TILE + 64];
  __shared__ __attribute__((aligned(16))) char lds_v[TILE + 64];
  __shared__ int seq[kMaxBlocks];
  __shared__ unsigned char flags[kMaxBlocks];

  const uint32_t lin = grid.linear(blockIdx.x);
  if (lin >= grid.total) return;
  const int Nb = a.Nb, N = a.N, keep = a.keep;
  const int bh = lin / Nb, qi = lin % Nb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * N * D;
  const char* qbase = (const char*)a.q + head * 2;
  const char* kbase = (const char*)a.k + head * 2;
  const char* vbase = (const char*)a.v + head * 2;
  const int32_t* list = a.idx + ((size_t)bh * Nb + qi) * keep;

  // Processing order: the kept list, then (calibration only) every other block ascending.
  const int nseq = MODE == AttnMode::kCalibrate ? Nb : keep;
  for (int n = threadIdx.x; n < keep; n += kThreads) seq[n] = min(max(list[n], 0), Nb - 1);
  if (MODE == AttnMode::kCalibrate) {
    for (int n = threadIdx.x; n < Nb; n += kThreads) flags[n] = 0;
    __syncthreads();
    for (int n = threadIdx.x; n < keep; n += kThreads) flags[seq[n]] = 1;
    __syncthreads();
    if (wave == 0) {
      int cnt = keep;
      for (int base = 0; base < Nb; base += 64) {
        int j = base + lane;
        bool f = j < Nb && !flags[j];
        unsigned long long mk = __ballot(f);
        const int pos = cnt + __popcll(mk & ((1ull << lane) - 1ull));
        if (f && pos < kMaxBlocks) seq[pos] = j;  // bounded even for a list with repeats
        cnt += __popcll(mk);
      }
    }
    if (a.idx_cache != nullptr) {
      int32_t* dst = a.idx_cache + ((size_t)bh * Nb + qi) * keep;
      for (int n = threadIdx.x; n < keep; n += kThreads) dst[n] = list[n];
    }
  }
  // Zero the padding units of the V rows: the last O^T tile of D = 80 reads
  // them as channels 80..95 (those output rows are discarded; zeros keep them finite).
  if (Shape<D>::RSU > Shape<D>::UNITS) {
    for (int r = threadIdx.x; r < kBlock; r += kThreads)
      for (int u = Shape<D>::UNITS; u < Shape<D>::RSU; ++u) *(u32x4*)(lds_v + lds_off<D>(r, u)) = u32x4{};
  }
  __syncthreads();

  // Q^T operand for this wave's 32 rows (rows >= N read as zero).
  WaveState<D> st;
  const int row = qi * kBlock + wave * 32 + l32;
  const bool row_ok = row < N;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 raw = u32x4{};
    if (row_ok) raw = *(const u32x4*)(qbase + ((size_t)row * D + 16 * ks + 8 * g) * 2);
    st.q[ks] = __builtin_bit_cast(bf16x8, raw);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) st.o[t] = f32x16{};
  st.m_raw = -INFINITY;
  st.z = 0.f;
  const float c = a.alpha * kLog2e;

  f32x16 okept[MODE == AttnMode::kCalibrate ? NT : 1];
  float m_kept = 0.f, z_kept = 0.f;

  Tile<D> tile;
  int cur = __builtin_amdgcn_readfirstlane(seq[0]);
  load_tile<D>(tile, kbase, vbase, cur, N);
  for (int n = 0; n < nseq; ++n) {
    __syncthreads();
    store_tile<D>(tile, lds_k, lds_v);
    __syncthreads();
    int nxt = cur;
    if (n + 1 < nseq) {
      nxt = __builtin_amdgcn_readfirstlane(seq[n + 1]);
      load_tile<D>(tile, kbase, vbase, nxt, N);
    }
    if (MODE == AttnMode::kCalibrate && n == keep) {
#pragma unroll
      for (int t = 0; t < NT; ++t) { okept[t] = st.o[t]; st.o[t] = f32x16{}; }
      m_kept = st.m_raw;
      z_kept = st.z;
      st.z = 0.f;
    }
    attend_block<D>(st, lds_k, lds_v, min(kBlock, N - cur * kBlock), c);
    cur = nxt;
  }

  // Epilogue.  Every lane holds 16 * NT output values of row `row`:
  // d = 32t + 8(i/4) + 4g + (i%4).
  const size_t srow = (size_t)bh * N + row;
  if (MODE == AttnMode::kCalibrate) {
    if (nseq == keep) {  // nothing masked: everything so far is the kept part
#pragma unroll
      for (int t = 0; t < NT; ++t) { okept[t] = st.o[t]; st.o[t] = f32x16{}; }
      m_kept = st.m_raw;
      z_kept = st.z;
      st.z = 0.f;
    }
    const float corr = __builtin_amdgcn_exp2f((m_kept - st.m_raw) * c);
    float zs = z_kept * corr;
    zs += xor32(zs);
    float zm = st.z + xor32(st.z);
    const float zf = zs + zm;
    const float inv = 1.f / zf;
    if (row_ok) {
      if (g == 0) {
        a.m[srow] = st.m_raw * a.alpha;
        a.z_full[srow] = zf;
        a.z_sparse[srow] = zs;
      }
      float* rrow = a.R + srow * D;
      __bf16* orow = (__bf16*)a.o + srow * D;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          int d = 32 * t + 8 * i4 + 4 * g;
          if (d < D) {
            f32x4 r, o;
            __bf16 ob[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              r[e] = st.o[t][4 * i4 + e];
              o[e] = (okept[t][4 * i4 + e] * corr + r[e]) * inv;
              ob[e] = (__bf16)o[e];
            }
            *(f32x4*)(rrow + d) = r;
            *(u32x2*)(orow + d) = *(u32x2*)ob;
          }
        }
    }
  } else {
    float z = st.z + xor32(st.z);
    if (row_ok) {
      const float m_cur = st.m_raw * a.alpha;
      const float m_c = a.m[srow];
      const float zf_c = a.z_full[srow], zs_c = a.z_sparse[srow];
      const float big = fmaxf(m_cur, m_c);
      const float e1 = expf(m_cur - big), e2 = expf(m_c - big);
      const float inv = 1.f / (z * e1 * zf_c / zs_c);
      const float w1 = e1 * inv, w2 = e2 * inv;
      const float* rrow = a.R + srow * D;
      __bf16* orow = (__bf16*)a.o + srow * D;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          int d = 32 * t + 8 * i4 + 4 * g;
          if (d < D) {
            f32x4 r = *(const f32x4*)(rrow + d);
            __bf16 ob[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ob[e] = (__bf16)(st.o[t][4 * i4 + e] * w1 + r[e] * w2);
            *(u32x2*)(orow + d) = *(u32x2*)ob;
          }
        }
    }
  }
}

template <int D, AttnMode MODE>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  XcdGrid grid = make_xcd_grid((uint32_t)a.BH * (uint32_t)a.Nb);
  hipLaunchKernelGGL((attn_bf16_kernel<D, MODE>), dim3(grid.grid()), dim3(kThreads), 0, s, a, grid);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(AttnMode mode, int D, const AttnArgs& a, hipStream_t s) {
  if (D == 64) return mode == AttnMode::kCalibrate ? launch_one<64, AttnMode::kCalibrate>(a, s)
                                                   : launch_one<64, AttnMode::kSparse>(a, s);
  if (D == 80) return mode == AttnMode::kCalibrate ? launch_one<80, AttnMode::kCalibrate>(a, s)
                                                   : launch_one<80, AttnMode::kSparse>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace rettn
