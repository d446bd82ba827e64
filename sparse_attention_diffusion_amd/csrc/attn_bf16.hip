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
// Per wave: 32 query rows.  Per key block (64 keys) a wave computes
//   S^T (64 keys x 32 rows) = K . Q^T   with v_mfma_f32_32x32x16_bf16, and
//   O^T (D x 32 rows)      += V^T . P^T  with the same instruction,
// so every lane owns one query row (lane % 32) in both results and the row
// statistics never leave the lane pair (l, l^32).
//
// K and V tiles reach LDS by DMA (global_load_lds_dwordx4, no register
// staging) into a ring of NBUF slots, so NBUF-1 key blocks are in flight while
// one is consumed; one workgroup barrier per key block.  LDS rows are made of
// 16-byte units, XOR-swizzled.  All LDS reads of the ring are issued from
// inline asm that waits for them itself: the compiler would otherwise wait for
// every DMA in flight before each read (it cannot tell ring slots apart), which
// would undo the prefetch.  V^T operands come from ds_read_b64_tr_b16.  The
// softmax reference max is raised lazily (only when a block max exceeds it by
// more than a factor 2^8 in probability), which keeps the accumulator rescale
// off the common path.
//
// Sparse kernel: one workgroup (2 waves) per 64-row query block; the cached
// residual and statistics are prefetched into registers at entry.
// Calibration kernel: QB query blocks (2 waves each) share every K/V tile; key
// blocks are visited in ascending order and each wave adds a block either to
// its kept accumulator or to its residual accumulator (a wave-uniform choice).
#include "internal.h"

namespace rettn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;  // raise the reference max only past a factor 2^8

template <int D>
struct Shape {
  static constexpr int KS = D / 16;             // k-steps of the d contraction
  static constexpr int NT = (D + 31) / 32;      // 32-wide d tiles of O^T
  static constexpr int UNITS = D / 8;           // 16-byte units per row in HBM
  static constexpr int RSU = D == 64 ? 8 : 12;  // LDS row stride in units (80: 2 filler units)
  static constexpr int ROW = RSU * 16;          // LDS row stride in bytes
  static constexpr int TILE = kBlock * ROW;     // bytes of one K (or V) tile
  static constexpr int SLOT = 2 * TILE;         // K tile then V tile
  static_assert(D == 64 || D == 80, "head dim");
};

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Waits until the tile of this step has landed, allowing `younger` later tiles
// (IPT DMA instructions each) to stay in flight.  Any other memory operation
// issued after the tile only makes the wait longer, never too short.
template <int IPT>
__device__ __forceinline__ void wait_tile(int younger) {
  if (younger >= 2) wait_vmcnt<2 * IPT>();
  else if (younger == 1) wait_vmcnt<IPT>();
  else wait_vmcnt<0>();
}

// Physical 16-byte unit of logical unit u in LDS row r.  Units 0..7 are
// XOR-swizzled so that 16 consecutive rows read at one unit, and 4 consecutive
// rows read at 4 aligned units, fall in distinct bank groups.
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int phys_unit(int r, int u) { return u < 8 ? (u ^ swz(r)) : u; }

template <int D>
__device__ __forceinline__ int lds_off(int r, int u) {
  return r * Shape<D>::ROW + phys_unit(r, u) * 16;
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// ------------------------------------------------------------------ DMA of tiles
// A tile pair (K and V of one key block) is 2*RSU DMA instructions of 1 KB
// (64 lanes x 16 B).  Wave w of W takes the K instructions c = w, w+W, ... and
// the same c for V (W divides RSU).  Lane l of instruction c fills LDS unit
// 64c + l of the tile, i.e. (row, physical unit), and fetches the logical unit
// the swizzle puts there.  The per-lane source offsets are computed once.
template <int D, int W>
struct TileDma {
  static constexpr int RSU = Shape<D>::RSU;
  static_assert(RSU % W == 0, "waves must divide the row units");
  static constexpr int NI = RSU / W;  // K (and V) instructions per wave
  static constexpr int IPT = 2 * NI;  // DMA instructions per tile per wave
  uint32_t off[NI];
  int row[NI];
  int wave;

  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int L = 64 * (w + W * i) + lane;
      const int r = L / RSU, p = L % RSU;
      int u = p < 8 ? (p ^ swz(r)) : p;
      if (u >= Shape<D>::UNITS) u -= 2;  // filler units of d_pad = 80 rows: any finite data
      row[i] = r;
      off[i] = (uint32_t)((r * D + u * 8) * 2);
    }
  }
  // Key block j of the head at (kbase, vbase) into the slot at `slot`; keys
  // past N read row N-1 (finite data; their scores are masked).
  __device__ __forceinline__ void issue(char* slot, const char* kbase, const char* vbase, int j, int N) const {
    const size_t blk = (size_t)j * kBlock * D * 2;
    const char* kb = kbase + blk;
    const char* vb = vbase + blk;
    const int nvalid = N - j * kBlock;
    if (nvalid >= kBlock) {  // uniform: every block but a short last one
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        char* dst = slot + (wave + W * i) * 1024;
        __builtin_amdgcn_global_load_lds((const void*)(kb + off[i]), (lds_void*)dst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vb + off[i]), (lds_void*)(dst + Shape<D>::TILE), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t o = off[i] - (uint32_t)(max(0, row[i] - (nvalid - 1)) * D * 2);
        char* dst = slot + (wave + W * i) * 1024;
        __builtin_amdgcn_global_load_lds((const void*)(kb + o), (lds_void*)dst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vb + o), (lds_void*)(dst + Shape<D>::TILE), 16, 0, 0);
      }
    }
  }
};

// ------------------------------------------------------------------ LDS reads (asm)
// Per-lane LDS addresses of the MFMA operands in ring slot 0; other slots and
// the second 32-key half are compile-time offsets.
template <int D>
struct Frag {
  uint32_t k[Shape<D>::KS];     // K operand, key half t = 0, k-step ks
  uint32_t v[Shape<D>::NT][2];  // V^T operand, d tile dt, half hh, k-step (t, hs) = (0, 0)
  __device__ __forceinline__ void init(const char* ring) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 5, l32 = lane & 31, G = lane >> 4, i16 = lane & 15;
    const uint32_t base = lds_addr(ring);
#pragma unroll
    for (int ks = 0; ks < Shape<D>::KS; ++ks) k[ks] = base + lds_off<D>(l32, 2 * ks + g);
#pragma unroll
    for (int dt = 0; dt < Shape<D>::NT; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // ds_read_b64_tr_b16 transposes within 16-lane groups: lane i of a group
        // points at key kbase + i/4, columns 4(i%4)..+3, and receives column i of
        // keys kbase..kbase+3.  t and hs move whole 16-key groups (no swizzle change).
        const int key = 8 * hh + 4 * g + (i16 >> 2);
        const int doff = 32 * dt + 16 * (G & 1) + 4 * (i16 & 3);
        v[dt][hh] = base + Shape<D>::TILE + lds_off<D>(key, doff >> 3) + (doff & 7) * 2;
      }
  }
};

// K operands of one key block, both 32-key halves (offset OFF and OFF + H):
// 2*KS ds_read_b128 waited for in the same statement.  a[t*KS + ks].
template <int KS, int OFF, int H>
__device__ __forceinline__ void k_reads(u32x4 (&a)[2 * KS], const uint32_t (&ad)[KS]) {
  static_assert(OFF >= 0 && OFF + H < 65536, "ds offset");
  if constexpr (KS == 4) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%12\n\t"
        "ds_read_b128 %1, %9 offset:%12\n\t"
        "ds_read_b128 %2, %10 offset:%12\n\t"
        "ds_read_b128 %3, %11 offset:%12\n\t"
        "ds_read_b128 %4, %8 offset:%13\n\t"
        "ds_read_b128 %5, %9 offset:%13\n\t"
        "ds_read_b128 %6, %10 offset:%13\n\t"
        "ds_read_b128 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(OFF), "i"(OFF + H)
        : "memory");
  } else {
    static_assert(KS == 5, "k-steps");
    asm volatile(
        "ds_read_b128 %0, %10 offset:%15\n\t"
        "ds_read_b128 %1, %11 offset:%15\n\t"
        "ds_read_b128 %2, %12 offset:%15\n\t"
        "ds_read_b128 %3, %13 offset:%15\n\t"
        "ds_read_b128 %4, %14 offset:%15\n\t"
        "ds_read_b128 %5, %10 offset:%16\n\t"
        "ds_read_b128 %6, %11 offset:%16\n\t"
        "ds_read_b128 %7, %12 offset:%16\n\t"
        "ds_read_b128 %8, %13 offset:%16\n\t"
        "ds_read_b128 %9, %14 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7]),
          "=&v"(a[8]), "=&v"(a[9])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "i"(OFF), "i"(OFF + H)
        : "memory");
  }
}

// V^T operands of one d tile for the four k-steps (t, hs): eight
// ds_read_b64_tr_b16, waited for in the same statement.  h[t][hs][hh].
template <int OFF, int T, int HS>
__device__ __forceinline__ void tr_reads(u32x2 (&h)[2][2][2], uint32_t a0, uint32_t a1) {
  static_assert(OFF + T + HS < 65536, "ds offset");
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%10\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%10\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%11\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(h[0][0][0]), "=&v"(h[0][0][1]), "=&v"(h[0][1][0]), "=&v"(h[0][1][1]), "=&v"(h[1][0][0]),
        "=&v"(h[1][0][1]), "=&v"(h[1][1][0]), "=&v"(h[1][1][1])
      : "v"(a0), "v"(a1), "i"(OFF), "i"(OFF + HS), "i"(OFF + T), "i"(OFF + T + HS)
      : "memory");
}

// ------------------------------------------------------------------ per-block math
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct Rows {
  bf16x8 q[Shape<D>::KS];  // Q^T operand: row lane%32, d = 16s + 8g + 0..7
  float m_ref;             // reference max (raw q.k units) the exponentials are taken against
  float m_true;            // running max of raw scores
};

// S^T = K Q^T for the key block in the slot at byte offset SLOT_OFF; keys at
// or past nvalid are set to -inf.  s[t][i] is key 32t + 8(i/4) + 4g + i%4.
// S^T = K Q^T for the key block in the slot at byte offset SLOT_OFF; keys at
// or past nvalid are set to -inf.  s[t][i] is key 32t + 8(i/4) + 4g + i%4.
// The two 32-key halves are independent MFMA chains, issued alternately.
template <int D, int SLOT_OFF>
__device__ __forceinline__ void scores(f32x16 (&s)[2], const Rows<D>& st, const Frag<D>& fr, int nvalid) {
  constexpr int KS = Shape<D>::KS;
  u32x4 a[2 * KS];
  k_reads<KS, SLOT_OFF, 32 * Shape<D>::ROW>(a, fr.k);
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[ks]), st.q[ks], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[KS + ks]), st.q[ks], s[1], 0, 0, 0);
  }
  if (nvalid < kBlock) {
    const int g = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * t + (i >> 2) * 8 + 4 * g + (i & 3);
        if (key >= nvalid) s[t][i] = -INFINITY;
      }
  }
}

__device__ __forceinline__ float row_max(const f32x16 (&s)[2]) {
  float m0 = -INFINITY, m1 = -INFINITY;  // two independent chains
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m0 = fmaxf(m0, s[0][i]);
    m1 = fmaxf(m1, s[1][i]);
  }
  return pair_max(fmaxf(m0, m1));
}

// Raises the reference max when some row of the wave needs it; returns the
// factor the accumulators must be multiplied by, and whether any changed.
__device__ __forceinline__ float update_max(float& m_ref, float& m_true, float mx, float c, bool* any) {
  m_true = fmaxf(m_true, mx);
  const bool need = mx > m_ref + kLazyLog2 / c;
  *any = __ballot(need) != 0ull;
  float corr = 1.f;
  if (*any) {
    const float m_new = fmaxf(m_ref, mx);
    corr = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
    m_ref = m_new;
  }
  return corr;
}

// P = exp2(c s - c m_ref) as bf16 MFMA operands (p[t][hs] holds k-step (t, hs));
// returns this lane's float32 sum of P.
__device__ __forceinline__ float probs(bf16x8 (&p)[2][2], const f32x16 (&s)[2], float m_ref, float c) {
  const float mc = m_ref * c;
  float z = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(fmaf(s[t][i], c, -mc));
      z += e;
      p[t][i >> 3][i & 7] = (__bf16)e;
    }
  return z;
}

// This lane's sum of the bf16-rounded P (the values the numerator uses).
__device__ __forceinline__ float sum_rounded(const bf16x8 (&p)[2][2]) {
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  float z0 = 0.f, z1 = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x2 lo = {p[t][0][2 * k], p[t][0][2 * k + 1]};
      const bf16x2 hi = {p[t][1][2 * k], p[t][1][2 * k + 1]};
      z0 = __builtin_amdgcn_fdot2_f32_bf16(lo, ones, z0, false);
      z1 = __builtin_amdgcn_fdot2_f32_bf16(hi, ones, z1, false);
    }
  return z0 + z1;
}

// V^T operands of the key block in the slot at SLOT_OFF, all d tiles:
// h[dt][t][hs][hh].  Fetched before the softmax so that the LDS latency
// overlaps the exponentials.
template <int D, int SLOT_OFF>
__device__ __forceinline__ void v_fetch(u32x2 (&h)[Shape<D>::NT][2][2][2], const Frag<D>& fr) {
  constexpr int ROW = Shape<D>::ROW;
#pragma unroll
  for (int dt = 0; dt < Shape<D>::NT; ++dt) tr_reads<SLOT_OFF, 32 * ROW, 16 * ROW>(h[dt], fr.v[dt][0], fr.v[dt][1]);
}

// O^T += V^T P^T.  k-step (t, hs) covers keys 32t + 16hs + 0..15; lane group g
// holds slots j <-> key 32t + 16hs + 8(j/4) + 4g + j%4 in both operands.  The
// d tiles are independent MFMA chains, issued alternately.
template <int D>
__device__ __forceinline__ void pv_mfma(f32x16 (&o)[Shape<D>::NT], const bf16x8 (&p)[2][2],
                                        const u32x2 (&h)[Shape<D>::NT][2][2][2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
      for (int dt = 0; dt < Shape<D>::NT; ++dt) {
        const u32x4 both = __builtin_shufflevector(h[dt][t][hs][0], h[dt][t][hs][1], 0, 1, 2, 3);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), p[t][hs], o[dt], 0, 0, 0);
      }
}

template <int D, int SLOT_OFF>
__device__ __forceinline__ void pv(f32x16 (&o)[Shape<D>::NT], const bf16x8 (&p)[2][2], const Frag<D>& fr) {
  u32x2 h[Shape<D>::NT][2][2][2];
  v_fetch<D, SLOT_OFF>(h, fr);
  pv_mfma<D>(o, p, h);
}

// Q^T operand of this lane's row.  Rows >= N read row N-1 instead (every lane
// issues the same loads); their results are never stored.
template <int D>
__device__ __forceinline__ void load_q(Rows<D>& st, const char* qbase, int row, int N) {
  const int g = (threadIdx.x & 63) >> 5;
  const size_t r = (size_t)min(row, N - 1);
#pragma unroll
  for (int ks = 0; ks < Shape<D>::KS; ++ks)
    st.q[ks] = __builtin_bit_cast(
        bf16x8, __builtin_nontemporal_load((const u32x4*)(qbase + (r * D + 16 * ks + 8 * g) * 2)));
  st.m_ref = -INFINITY;
  st.m_true = -INFINITY;
}

// ---------------------------------------------------------------- sparse step
template <int D, int NBUF>
struct SparseCtx {
  static constexpr int NT = Shape<D>::NT;
  using Dma = TileDma<D, 2>;
  char* ring;
  const __attribute__((address_space(4))) int32_t* list;  // kept blocks, read with scalar loads
  const char* kbase;
  const char* vbase;
  int keep, N, Nb;
  float c;
  Dma dma;

  __device__ __forceinline__ int block_at(int n) const { return min(max(list[n], 0), Nb - 1); }
  Frag<D> fr;
  Rows<D> st;
  f32x16 o[NT];
  float z;

  // Key block n of the list, in ring slot SLOT = n % NBUF.
  template <int SLOT>
  __device__ __forceinline__ void step(int n) {
    wait_tile<Dma::IPT>(min(NBUF - 2, keep - 1 - n));
    __builtin_amdgcn_s_barrier();
    if (n + NBUF - 1 < keep) {
      constexpr int NEXT = (SLOT + NBUF - 1) % NBUF;
      dma.issue(ring + NEXT * Shape<D>::SLOT, kbase, vbase, block_at(n + NBUF - 1), N);
    }
    const int j = block_at(n);
    f32x16 s[2];
    scores<D, SLOT * Shape<D>::SLOT>(s, st, fr, min(kBlock, N - j * kBlock));
    bool any;
    const float corr = update_max(st.m_ref, st.m_true, row_max(s), c, &any);
    if (any) {
      z *= corr;
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] *= corr;
    }
    bf16x8 p[2][2];
    probs(p, s, st.m_ref, c);
    z += sum_rounded(p);
    pv<D, SLOT * Shape<D>::SLOT>(o, p, fr);
  }
};

template <int D, int NBUF>
__global__ void __launch_bounds__(128) sparse_kernel(AttnArgs a, XcdGrid grid) {
  constexpr int NT = Shape<D>::NT;
  static_assert(NBUF >= 2 && NBUF <= 3, "ring depth");
  __shared__ __attribute__((aligned(1024))) char ring[NBUF * Shape<D>::SLOT];

  const uint32_t lin = grid.linear(blockIdx.x);
  if (lin >= grid.total) return;
  const int Nb = a.Nb, N = a.N, keep = a.keep;
  const int bh = lin / Nb, qi = lin % Nb;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * N * D;
  const int row = qi * kBlock + wave * 32 + l32;
  const bool row_ok = row < N;
  const size_t srow = (size_t)bh * N + (row_ok ? row : N - 1);

  // Memory order: the first tiles (their block indices come from scalar loads
  // of the list), then Q, then the statistics and the residual (needed last).
  SparseCtx<D, NBUF> cx;
  cx.ring = ring;
  cx.list = (const __attribute__((address_space(4))) int32_t*)(a.idx + ((size_t)bh * Nb + qi) * keep);
  cx.kbase = (const char*)a.k + head * 2;
  cx.vbase = (const char*)a.v + head * 2;
  cx.keep = keep;
  cx.N = N;
  cx.Nb = Nb;
  cx.c = a.alpha * kLog2e;
  cx.dma.init(wave, lane);
  cx.fr.init(ring);
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < keep) cx.dma.issue(ring + t * Shape<D>::SLOT, cx.kbase, cx.vbase, cx.block_at(t), N);
  load_q<D>(cx.st, (const char*)a.q + head * 2, row, N);

  const float m_c = a.m[srow], zf_c = a.z_full[srow], zs_c = a.z_sparse[srow];
  f32x4 rc[NT][4];
  {
    const float* rrow = a.R + srow * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * t + 8 * i4 + 4 * g;
        rc[t][i4] = d < D ? __builtin_nontemporal_load((const f32x4*)(rrow + d)) : f32x4{};
      }
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) cx.o[t] = f32x16{};
  cx.z = 0.f;
  for (int n = 0; n < keep; n += NBUF) {
    cx.template step<0>(n);
    if (n + 1 < keep) cx.template step<1>(n + 1);
    if constexpr (NBUF > 2)
      if (n + 2 < keep) cx.template step<2>(n + 2);
  }

  // O = (N e^{m-M} + R_c e^{m_c-M}) / (Z e^{m-M} Z_full_c / Z_sparse_c), M = max(m, m_c);
  // N and Z are relative to m = the reference max (any reference gives the same O).
  const float z = pair_sum(cx.z);
  if (row_ok) {
    const float m_cur = cx.st.m_ref * a.alpha;
    const float big = fmaxf(m_cur, m_c);
    const float e1 = expf(m_cur - big), e2 = expf(m_c - big);
    const float inv = 1.f / (z * e1 * zf_c / zs_c);
    const float w1 = e1 * inv, w2 = e2 * inv;
    __bf16* orow = (__bf16*)a.o + srow * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * t + 8 * i4 + 4 * g;
        if (d < D) {
          __bf16 ob[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) ob[e] = (__bf16)(cx.o[t][4 * i4 + e] * w1 + rc[t][i4][e] * w2);
          *(u32x2*)(orow + d) = *(u32x2*)ob;
        }
      }
  }
}

// ---------------------------------------------------------------- sparse step, persistent
// A persistent variant of the sparse step: each workgroup walks a strided run
// of query blocks (all from its XCD's range) and feeds one continuous stream of
// key-block tiles through the ring, so the next query block's first tiles are
// already in flight while the current one finishes, and the per-block setup
// (list, Q, residual) overlaps with compute:
//   * Q of the next query block is loaded into a second register set one
//     block ahead;
//   * the residual and statistics of the current block are loaded right after
//     its first tile is consumed and waited for at its second tile;
//   * the block index of every tile comes from scalar loads of the list.
// Tiles are numbered T = k*keep + n over the workgroup's k-th query block.
struct PersistGrid {
  uint32_t total, per, g;  // query blocks, per XCD, workgroups per XCD
};

// Scalar context of one query block of the persistent walk.
template <int D>
struct ItemCtx {
  const __attribute__((address_space(4))) int32_t* list;  // its kept blocks (scalar loads)
  const char* kb;                                          // K, V, Q of its head
  const char* vb;
  const char* qb;
  uint32_t lin;
  int qi, bh;
  __device__ __forceinline__ void set(const AttnArgs& a, uint32_t l) {
    lin = l;
    bh = (int)(l / (uint32_t)a.Nb);
    qi = (int)(l - (uint32_t)bh * (uint32_t)a.Nb);
    const size_t head = (size_t)bh * a.N * D * 2;
    kb = (const char*)a.k + head;
    vb = (const char*)a.v + head;
    qb = (const char*)a.q + head;
    list = (const __attribute__((address_space(4))) int32_t*)(a.idx + (size_t)l * a.keep);
  }
  __device__ __forceinline__ int block(int n, int Nb) const { return min(max(list[n], 0), Nb - 1); }
};

template <int D, int NBUF>
__global__ void __launch_bounds__(128) sparse_persistent_kernel(AttnArgs a, PersistGrid pg) {
  constexpr int NT = Shape<D>::NT, KS = Shape<D>::KS, SLOT = Shape<D>::SLOT;
  using Dma = TileDma<D, 2>;
  static_assert(NBUF >= 2 && NBUF <= 3, "ring depth");
  __shared__ __attribute__((aligned(1024))) char ring[NBUF * SLOT];

  const uint32_t xcd = blockIdx.x % 8u, r = blockIdx.x / 8u;
  const uint32_t start = xcd * pg.per, end = min(pg.total, start + pg.per);
  if (start + r >= end) return;
  const int n_items = (int)((end - start - r + pg.g - 1) / pg.g);
  const int Nb = a.Nb, N = a.N, keep = a.keep;
  const int total_tiles = n_items * keep;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const float c = a.alpha * kLog2e;

  Dma dma;
  dma.init(wave, lane);
  Frag<D> fr;
  fr.init(ring);

  // DMA cursor: the next tile to request is block dn of query block dk.
  ItemCtx<D> dit;
  dit.set(a, start + r);
  int dk = 0, dn = 0, dslot = 0, issued = 0;
  auto issue_next = [&]() {
    dma.issue(ring + dslot * SLOT, dit.kb, dit.vb, dit.block(dn, Nb), N);
    ++issued;
    dslot = dslot + 1 == NBUF ? 0 : dslot + 1;
    if (++dn == keep) {
      dn = 0;
      if (++dk < n_items) dit.set(a, start + r + (uint32_t)dk * pg.g);
    }
  };
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < total_tiles) issue_next();

  ItemCtx<D> it;
  it.set(a, start + r);
  Rows<D> st, nx;  // current and next query block's Q operand
  load_q<D>(nx, it.qb, it.qi * kBlock + wave * 32 + l32, N);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(nx.q[ks]));  // Q of the first block in place

  int slot = 0, consumed = 0;
  for (int k = 0; k < n_items; ++k) {
    if (k > 0) it.set(a, start + r + (uint32_t)k * pg.g);
    const int row = it.qi * kBlock + wave * 32 + l32;
    const bool row_ok = row < N;
    const size_t srow = (size_t)it.bh * N + min(row, N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) st.q[ks] = nx.q[ks];
    f32x16 o[NT];
    float z = 0.f;
    float m_c = 0.f, zf_c = 1.f, zs_c = 1.f;
    f32x4 rc[NT][4];

    auto step = [&](int n, bool first) {
      wait_tile<Dma::IPT>(min(NBUF - 2, total_tiles - 1 - consumed));
      __builtin_amdgcn_s_barrier();
      if (issued < total_tiles) issue_next();
      if (first) {
        // residual and statistics of this block, and Q of the next one; waited for at the next tile
        m_c = a.m[srow];
        zf_c = a.z_full[srow];
        zs_c = a.z_sparse[srow];
        const float* rrow = a.R + srow * D;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d = 32 * t + 8 * i4 + 4 * g;
            rc[t][i4] = d < D ? __builtin_nontemporal_load((const f32x4*)(rrow + d)) : f32x4{};
          }
        if (k + 1 < n_items) {
          ItemCtx<D> nit;
          nit.set(a, start + r + (uint32_t)(k + 1) * pg.g);
          load_q<D>(nx, nit.qb, nit.qi * kBlock + wave * 32 + l32, N);
        }
      }
      const uint32_t soff = (uint32_t)slot * SLOT;
      slot = slot + 1 == NBUF ? 0 : slot + 1;
      ++consumed;
      Frag<D> f2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) f2.k[ks] = fr.k[ks] + soff;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        f2.v[dt][0] = fr.v[dt][0] + soff;
        f2.v[dt][1] = fr.v[dt][1] + soff;
      }
      const int j = it.block(n, Nb);
      f32x16 s[2];
      scores<D, 0>(s, st, f2, min(kBlock, N - j * kBlock));
      if (first) {  // nothing accumulated yet: start from this block's max
        const float mx = row_max(s);
        st.m_true = mx;
        st.m_ref = mx;
      } else {
        bool any;
        const float corr = update_max(st.m_ref, st.m_true, row_max(s), c, &any);
        if (any) {
          z *= corr;
#pragma unroll
          for (int t = 0; t < NT; ++t) o[t] *= corr;
        }
      }
      u32x2 vh[NT][2][2][2];
      v_fetch<D, 0>(vh, f2);
      bf16x8 p[2][2];
      probs(p, s, st.m_ref, c);
      z += sum_rounded(p);
      if (first) {
#pragma unroll
        for (int t = 0; t < NT; ++t) o[t] = f32x16{};
      }
      pv_mfma<D>(o, p, vh);
    };

    // keep >= 2 here (the launcher sends keep == 1 to the per-block kernel)
    step(0, true);
    step(1, false);
    // The loads issued at the first tile are complete here (the tile wait of
    // the second tile covered them); using them now keeps the compiler from
    // waiting for them later, when tile DMA would be in flight.
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) asm volatile("" ::"v"(rc[t][i4]));
    asm volatile("" ::"v"(m_c), "v"(zf_c), "v"(zs_c));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(nx.q[ks]));
    for (int n = 2; n < keep; ++n) step(n, false);

    const float zz = pair_sum(z);
    if (row_ok) {
      const float m_cur = st.m_ref * a.alpha;
      const float big = fmaxf(m_cur, m_c);
      const float e1 = expf(m_cur - big), e2 = expf(m_c - big);
      const float inv = 1.f / (zz * e1 * zf_c / zs_c);
      const float w1 = e1 * inv, w2 = e2 * inv;
      __bf16* orow = (__bf16*)a.o + srow * D;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = 32 * t + 8 * i4 + 4 * g;
          if (d < D) {
            __bf16 ob[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ob[e] = (__bf16)(o[t][4 * i4 + e] * w1 + rc[t][i4][e] * w2);
            *(u32x2*)(orow + d) = *(u32x2*)ob;
          }
        }
    }
  }
}

// ---------------------------------------------------------------- calibration step
template <int D, int NBUF, int QB>
struct CalibCtx {
  static constexpr int NT = Shape<D>::NT;
  using Dma = TileDma<D, 2 * QB>;
  char* ring;
  const unsigned char* flags;  // this wave's query block: 1 = kept key block
  const char* kbase;
  const char* vbase;
  int Nb, N;
  bool active;
  float c;
  Dma dma;
  Frag<D> fr;
  Rows<D> st;
  f32x16 okept[NT], ores[NT];
  float zk, zm;

  template <int SLOT>
  __device__ __forceinline__ void step(int j) {
    wait_tile<Dma::IPT>(min(NBUF - 2, Nb - 1 - j));
    __builtin_amdgcn_s_barrier();
    if (j + NBUF - 1 < Nb) {
      constexpr int NEXT = (SLOT + NBUF - 1) % NBUF;
      dma.issue(ring + NEXT * Shape<D>::SLOT, kbase, vbase, j + NBUF - 1, N);
    }
    if (!active) return;
    const bool kept = __builtin_amdgcn_readfirstlane(flags[j]) != 0;
    f32x16 s[2];
    scores<D, SLOT * Shape<D>::SLOT>(s, st, fr, min(kBlock, N - j * kBlock));
    bool any;
    const float corr = update_max(st.m_ref, st.m_true, row_max(s), c, &any);
    if (any) {
      zk *= corr;
      zm *= corr;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        okept[t] *= corr;
        ores[t] *= corr;
      }
    }
    bf16x8 p[2][2];
    const float zb = probs(p, s, st.m_ref, c);
    if (kept) {
      zk += zb;
      pv<D, SLOT * Shape<D>::SLOT>(okept, p, fr);
    } else {
      zm += zb;
      pv<D, SLOT * Shape<D>::SLOT>(ores, p, fr);
    }
  }
};

template <int D, int NBUF, int QB>
__global__ void __launch_bounds__(128 * QB) calib_kernel(AttnArgs a, XcdGrid grid) {
  constexpr int NT = Shape<D>::NT;
  static_assert(NBUF >= 2 && NBUF <= 3, "ring depth");
  __shared__ __attribute__((aligned(1024))) char ring[NBUF * Shape<D>::SLOT];
  __shared__ unsigned char flags[QB][kMaxBlocks];

  const uint32_t lin = grid.linear(blockIdx.x);
  if (lin >= grid.total) return;
  const int Nb = a.Nb, N = a.N, keep = a.keep;
  const int groups = (Nb + QB - 1) / QB;
  const int bh = lin / groups, q0 = (lin % groups) * QB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int qb = wave >> 1, qi = q0 + qb;
  const size_t head = (size_t)bh * N * D;

  for (int n = threadIdx.x; n < QB * kMaxBlocks; n += 128 * QB) (&flags[0][0])[n] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < QB * keep; e += 128 * QB) {
    const int b = e / keep, n = e % keep;
    if (q0 + b < Nb) {
      const size_t at = ((size_t)bh * Nb + q0 + b) * keep + n;
      const int j = a.idx[at];
      flags[b][min(max(j, 0), Nb - 1)] = 1;
      if (a.idx_cache != nullptr) a.idx_cache[at] = j;
    }
  }

  CalibCtx<D, NBUF, QB> cx;
  const int row = qi * kBlock + (wave & 1) * 32 + l32;
  const bool row_ok = qi < Nb && row < N;
  load_q<D>(cx.st, (const char*)a.q + head * 2, qi < Nb ? row : N, N);
  cx.ring = ring;
  cx.flags = flags[qb];
  cx.kbase = (const char*)a.k + head * 2;
  cx.vbase = (const char*)a.v + head * 2;
  cx.Nb = Nb;
  cx.N = N;
  cx.active = qi < Nb;
  cx.c = a.alpha * kLog2e;
  cx.dma.init(wave, lane);
  cx.fr.init(ring);
#pragma unroll
  for (int t = 0; t < NT; ++t) cx.okept[t] = cx.ores[t] = f32x16{};
  cx.zk = cx.zm = 0.f;
  __syncthreads();  // flags and Q in place

#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < Nb) cx.dma.issue(ring + t * Shape<D>::SLOT, cx.kbase, cx.vbase, t, N);

  for (int j = 0; j < Nb; j += NBUF) {
    cx.template step<0>(j);
    if (j + 1 < Nb) cx.template step<1>(j + 1);
    if constexpr (NBUF > 2)
      if (j + 2 < Nb) cx.template step<2>(j + 2);
  }

  // Statistics relative to the true row max m: factor e^{m_ref - m}.
  const float f = __builtin_amdgcn_exp2f((cx.st.m_ref - cx.st.m_true) * cx.c);
  const float zs = pair_sum(cx.zk) * f;
  const float zf = zs + pair_sum(cx.zm) * f;
  if (row_ok) {
    const size_t srow = (size_t)bh * N + row;
    if (g == 0) {
      a.m[srow] = cx.st.m_true * a.alpha;
      a.z_full[srow] = zf;
      a.z_sparse[srow] = zs;
    }
    const float inv = 1.f / zf;
    float* rrow = a.R + srow * D;
    __bf16* orow = (__bf16*)a.o + srow * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * t + 8 * i4 + 4 * g;
        if (d < D) {
          f32x4 r;
          __bf16 ob[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = cx.ores[t][4 * i4 + e] * f;
            ob[e] = (__bf16)((cx.okept[t][4 * i4 + e] * f + r[e]) * inv);
          }
          *(f32x4*)(rrow + d) = r;
          *(u32x2*)(orow + d) = *(u32x2*)ob;
        }
      }
  }
}

constexpr int kSparseRing = 2;
constexpr int kCalibRing = 3;
constexpr bool kPersistent = true;
constexpr int kPersistWgPerXcd = 32 * 4;  // 4 two-wave workgroups per CU

template <int D>
hipError_t launch_d(AttnMode mode, const AttnArgs& a, hipStream_t s) {
  if (mode == AttnMode::kSparse) {
    if (kPersistent && a.keep >= 2) {
      const uint32_t total = (uint32_t)a.BH * (uint32_t)a.Nb;
      PersistGrid pg{total, (total + 7u) / 8u, 0u};
      pg.g = min(pg.per, (uint32_t)kPersistWgPerXcd);
      hipLaunchKernelGGL((sparse_persistent_kernel<D, kSparseRing>), dim3(8u * pg.g), dim3(128), 0, s, a, pg);
    } else {
      XcdGrid grid = make_xcd_grid((uint32_t)a.BH * (uint32_t)a.Nb);
      hipLaunchKernelGGL((sparse_kernel<D, kSparseRing>), dim3(grid.grid()), dim3(128), 0, s, a, grid);
    }
  } else {
    constexpr int QB = D == 64 ? 4 : 2;  // 2*QB waves must divide the LDS row units
    const uint32_t groups = (uint32_t)(a.Nb + QB - 1) / QB;
    XcdGrid grid = make_xcd_grid((uint32_t)a.BH * groups);
    hipLaunchKernelGGL((calib_kernel<D, kCalibRing, QB>), dim3(grid.grid()), dim3(128 * QB), 0, s, a, grid);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(AttnMode mode, int D, const AttnArgs& a, hipStream_t s) {
  if (D == 64) return launch_d<64>(mode, a, s);
  if (D == 80) return launch_d<80>(mode, a, s);
  return hipErrorInvalidValue;
}

}  // namespace rettn
