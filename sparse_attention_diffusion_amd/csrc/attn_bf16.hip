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
// K and V tiles reach LDS by DMA (buffer/global_load ... lds, no register
// staging).  LDS rows are made of 16-byte units, XOR-swizzled.  All LDS reads
// of tiles are issued from inline asm that waits for them itself: the
// compiler would otherwise wait for every DMA in flight before each read (it
// cannot tell a slot being filled from one being read), which would undo the
// overlap.  V^T operands come from ds_read_b64_tr_b16.  At d_pad 64 both
// kernels first walk with a fixed softmax reference (the cached row max in the
// sparse step, key block 0's row max in the calibration) and walk a query
// block again where a row sum leaves the float32 range; that walk, and every
// walk at d_pad 80, raises the reference lazily (only when a block max exceeds
// it by more than a factor 2^8 in probability), which keeps the accumulator
// rescale off the common path.
//
// Sparse kernel: persistent, XCD-aware; one K slot and one V slot per
// two-wave workgroup and at most 128 VGPRs, so that many workgroups share a
// CU and hide each other's memory latency.  A query block's accumulator
// starts as its cached residual.
// Calibration kernel: QB query blocks (2 waves each) share every K/V tile; key
// blocks are visited in ascending order; each wave adds every block to an
// all-keys accumulator and its kept blocks also to a kept accumulator, and the
// residual is their difference.
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

// Workgroup barrier that the compiler also treats as a memory barrier: no
// load or store (LDS or global) moves across it, so the LDS a barrier guards
// (tiles, staged rows, flags) is read and written on the intended side.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// ---------------------------------------------------------------- buffer-resource helpers
// Global traffic of the sparse kernel goes through buffer resources: per-lane
// offsets are fixed, the base and the byte limit are scalar, and the limit
// zero-fills rows past N on loads and drops them on stores.
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format (descriptor word 3)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufFlags);
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
  int wave;

  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int L = 64 * (w + W * i) + lane;
      const int r = L / RSU, p = L % RSU;
      int u = p < 8 ? (p ^ swz(r)) : p;
      if (u >= Shape<D>::UNITS) u -= 2;  // filler units of d_pad = 80 rows: any finite data
      off[i] = (uint32_t)((r * D + u * 8) * 2);
    }
  }
  // Key block j of the head at (kbase, vbase) into the slot at `slot`,
  // through buffer resources (scalar base and byte limit, fixed per-lane
  // offsets): keys past N read as zeros (their scores are masked).
  __device__ __forceinline__ void issue(char* slot, const char* kbase, const char* vbase, int j, int N) const {
    const size_t blk = (size_t)j * kBlock * D * 2;
    const int bytes = min(N - j * kBlock, kBlock) * D * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + blk, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + blk, bytes);
    asm volatile("" ::: "memory");  // in program order with other memory operations (vmcnt counts)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      char* dst = slot + (wave + W * i) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)dst, 16, (int)off[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dst + Shape<D>::TILE), 16, (int)off[i], 0, 0, 0);
    }
    asm volatile("" ::: "memory");
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

// K operands of one 32-key half at byte offset `off` from the lane addresses:
// KS ds_read_b128 waited for in the same statement.
template <int KS>
__device__ __forceinline__ void k_half(u32x4 (&a)[KS], const uint32_t (&ad)[KS], uint32_t off) {
  if constexpr (KS == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
        : "v"(ad[0] + off), "v"(ad[1] + off), "v"(ad[2] + off), "v"(ad[3] + off)
        : "memory");
  } else {
    static_assert(KS == 5, "k-steps");
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %6\n\t"
        "ds_read_b128 %2, %7\n\t"
        "ds_read_b128 %3, %8\n\t"
        "ds_read_b128 %4, %9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4])
        : "v"(ad[0] + off), "v"(ad[1] + off), "v"(ad[2] + off), "v"(ad[3] + off), "v"(ad[4] + off)
        : "memory");
  }
}

// K operands of one 32-key half at the immediate LDS offset OFF: KS
// ds_read_b128 waited for in the same statement.
template <int KS, int OFF>
__device__ __forceinline__ void k_half_at(u32x4 (&a)[KS], const uint32_t (&ad)[KS]) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  if constexpr (KS == 4) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%8\n\t"
        "ds_read_b128 %1, %5 offset:%8\n\t"
        "ds_read_b128 %2, %6 offset:%8\n\t"
        "ds_read_b128 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(OFF)
        : "memory");
  } else {
    static_assert(KS == 5, "k-steps");
    asm volatile(
        "ds_read_b128 %0, %5 offset:%10\n\t"
        "ds_read_b128 %1, %6 offset:%10\n\t"
        "ds_read_b128 %2, %7 offset:%10\n\t"
        "ds_read_b128 %3, %8 offset:%10\n\t"
        "ds_read_b128 %4, %9 offset:%10\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "i"(OFF)
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

// The same two products with fewer operand registers live at once (K one
// 32-key half at a time, V^T one d tile at a time), for head dims whose
// accumulators leave little register room.
template <int D, int SLOT_OFF>
__device__ __forceinline__ void scores_lean(f32x16 (&s)[2], const Rows<D>& st, const Frag<D>& fr, int nvalid) {
  constexpr int KS = Shape<D>::KS;
  {
    u32x4 kk[KS];
    k_half_at<KS, SLOT_OFF>(kk, fr.k);
    s[0] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kk[ks]), st.q[ks], s[0], 0, 0, 0);
  }
  {
    u32x4 kk[KS];
    k_half_at<KS, SLOT_OFF + 32 * Shape<D>::ROW>(kk, fr.k);
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kk[ks]), st.q[ks], s[1], 0, 0, 0);
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

template <int D, int SLOT_OFF>
__device__ __forceinline__ void pv_lean(f32x16 (&o)[Shape<D>::NT], const bf16x8 (&p)[2][2], const Frag<D>& fr) {
  constexpr int ROW = Shape<D>::ROW;
#pragma unroll
  for (int dt = 0; dt < Shape<D>::NT; ++dt) {
    u32x2 h[2][2][2];
    tr_reads<SLOT_OFF, 32 * ROW, 16 * ROW>(h, fr.v[dt][0], fr.v[dt][1]);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const u32x4 both = __builtin_shufflevector(h[t][hs][0], h[t][hs][1], 0, 1, 2, 3);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), p[t][hs], o[dt], 0, 0, 0);
      }
  }
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

// Persistent grid: each of the 8 XCDs owns a contiguous range of `per` query
// blocks (blocks of a range share heads, hence K/V tiles in that XCD's L2);
// its `g` workgroups walk the range with stride g.
struct PersistGrid {
  uint32_t total, per, g;  // query blocks, per XCD, workgroups per XCD
};



// Cache policy of the streams read once per call (Q, the residual): non-temporal.
constexpr int kNT = 2;

// Tile DMA of one 64-row tile (K, V or Q), this wave's half (RSU/2
// instructions of 1 KB); same unit placement as TileDma.  Wave w fills tile
// rows 32w..32w+31 (LDS bytes [32w ROW, 32(w+1) ROW)), so a wave that
// overwrites only what it alone reads needs no barrier.
template <int D>
struct PipeDma {
  static constexpr int RSU = Shape<D>::RSU;
  static constexpr int NI = RSU / 2;
  uint32_t off[NI];
  int wave;
  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int L = 64 * (NI * w + i) + lane;
      const int r = L / RSU, p = L % RSU;
      int u = p < 8 ? (p ^ swz(r)) : p;
      if (u >= Shape<D>::UNITS) u -= 2;  // filler units of d_pad = 80 rows: any finite data
      off[i] = (uint32_t)((r * D + u * 8) * 2);
    }
  }
  // A 64-row tile at `tile`, `bytes` of it valid, into `slot`; rows past the
  // valid bytes are zero-filled by the buffer limit.  AUX is the cache policy
  // (0, or kNT for a tile read once).
  template <int AUX = 0>
  __device__ __forceinline__ void issue_at(char* slot, const char* tile, int bytes) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile, bytes);
    // The wave's first destination, kept opaque so that the compiler adds
    // the 1 KB steps at each call instead of holding (and spilling) one
    // scalar register per destination for the whole kernel.
    uint32_t dst = lds_addr(slot) + (uint32_t)(NI * wave * 1024);
    asm volatile("" : "+s"(dst));
    lds_void* const d0 = (lds_void*)(uintptr_t)dst;
    // The batch stays in program order with every other memory operation:
    // the vmcnt waits count instructions issued after it.
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)((__attribute__((address_space(3))) char*)d0 + i * 1024),
                                               16, off[i], 0, 0, AUX);
    asm volatile("" ::: "memory");
  }
};

// Scalar context of one query block: its kept list and its head.
template <int D>
struct PipeItem {
  const __attribute__((address_space(4))) int32_t* list;
  const char* kh;
  const char* vh;
  int bh, qi;
  __device__ __forceinline__ void set(const AttnArgs& a, uint32_t l) {
    bh = (int)(l / (uint32_t)a.Nb);
    qi = (int)(l - (uint32_t)bh * (uint32_t)a.Nb);
    const size_t head = (size_t)bh * a.N * D * 2;
    kh = (const char*)a.k + head;
    vh = (const char*)a.v + head;
    list = (const __attribute__((address_space(4))) int32_t*)(a.idx + (size_t)l * a.keep);
  }
  __device__ __forceinline__ int block(int n, int Nb) const { return min(max(list[n], 0), Nb - 1); }
  // The list entry as stored; clamped where it is used, so that the wait for
  // the scalar load falls there and not right after the load.
  __device__ __forceinline__ int raw(int n) const { return list[n]; }
};

// One query block's per-lane statistics (the cached row max only for the
// R1 epilogue, which needs the residual's reference).
template <int D>
struct PipeStats {
  float mc, zf, zs;
};

// Statistics of one query block: 3 loads (2 for R2).
template <int D, bool R2>
__device__ __forceinline__ void load_stats(PipeStats<D>& st, const AttnArgs& a, int bh, int qi, int rowq) {
  const size_t r0 = (size_t)bh * a.N + (size_t)qi * kBlock;  // first row of the block
  const int rows = min(a.N - qi * kBlock, kBlock);
  if (!R2)
    st.mc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.m + r0, rows * 4), rowq * 4, 0, 0));
  st.zf = __builtin_bit_cast(float,
                             __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.z_full + r0, rows * 4), rowq * 4, 0, 0));
  st.zs = __builtin_bit_cast(float,
                             __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.z_sparse + r0, rows * 4), rowq * 4, 0, 0));
}

// Cached residual of one query block in accumulator order: D/8 loads.  The
// cache holds it in that order (residual_index), padded to 64 rows, so every
// load is one contiguous run over the wave's lanes.
template <int D, bool RB>
__device__ __forceinline__ void load_residual(f32x4 (&r)[Shape<D>::NT][4], const AttnArgs& a, int bh, int qi, int rowq,
                                              int g) {
  // The wave's 32 rows: D/8 runs of 256 elements from this base.
  const size_t r0 = ((size_t)bh * a.Nb + (size_t)qi) * kBlock * D + (size_t)(rowq >> 5) * 32 * D;
  const __amdgpu_buffer_rsrc_t rr =
      RB ? make_rsrc((const __bf16*)a.R + r0, 32 * D * 2) : make_rsrc(a.R + r0, 32 * D * 4);
  // This lane's bytes into each run; kept opaque so that the compiler adds
  // the run offsets as constants instead of holding one register per run.
  int lo = (32 * g + (rowq & 31)) * 4 * (RB ? 2 : 4);
  asm volatile("" : "+v"(lo));
#pragma unroll
  for (int t = 0; t < Shape<D>::NT; ++t)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int run = (4 * t + i4) * 256 * (RB ? 2 : 4);  // bytes before this run
      if (32 * t + 8 * i4 >= D) {
        r[t][i4] = f32x4{};
      } else if (RB) {  // four bf16, widened exactly
        const u32x2 h = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rr, lo + run, 0, kNT));
        r[t][i4] = f32x4{__uint_as_float(h[0] << 16), __uint_as_float(h[0] & 0xFFFF0000u),
                         __uint_as_float(h[1] << 16), __uint_as_float(h[1] & 0xFFFF0000u)};
      } else {
        r[t][i4] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, lo + run, 0, kNT));
      }
    }
}

// O^T += V^T P^T with the V operands already fetched.
template <int D>
__device__ __forceinline__ void mask_keys(f32x16 (&s)[2], int nvalid) {
  const int g = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 32 * t + (i >> 2) * 8 + 4 * g + (i & 3);
      if (key >= nvalid) s[t][i] = -INFINITY;
    }
}

// P = exp2(c s - mr) as bf16 MFMA operands (mr: reference max times c).
__device__ __forceinline__ void probs_ref(bf16x8 (&p)[2][2], const f32x16 (&s)[2], float mr, float c) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) p[t][i >> 3][i & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[t][i], c, -mr));
}

// ---------------------------------------------------------------- sparse step, high occupancy
// The production sparse kernel.  One K slot and one V slot per workgroup
// (16 KB for d_pad 64) and at most 128 VGPRs per lane, so that 8 two-wave
// workgroups share a CU (4 waves per SIMD): the latency of tile DMA and of the
// per-query-block loads is hidden by the other workgroups instead of by a
// deep ring, which the LDS could not hold (each wave's vmcnt is one in-order
// counter, so any long-latency load a wave issues delays its next tile wait).
// Per key block n of a query block:
//   1. wait for K_n, barrier (V_{n-1} consumed by both waves), DMA V_n (at
//      n = 0 each wave first reads its Q rows, DMA'd into its half of the V
//      slot);
//   2. S^T = K_n Q^T in two 32-key halves and P against a reference max;
//   3. wait for V_n, barrier (K_n consumed), DMA K_{n+1} (which may belong to
//      the next query block);
//   4. O^T += V_n^T P^T.
// A query block's accumulator starts as its cached residual R with the
// reference max at the cached m (R is stored relative to m), so the reshape
// epilogue is O = acc * Z_sparse / (Z * Z_full) with Z the kept mass.  At
// d_pad 64 the first walk keeps that reference fixed (no per-tile maximum);
// a row sum that leaves the float32 range sends the block through a second
// walk with the lazy maximum, which rescales both parts together.  Variant R2
// (V2) instead blends the normalised sparse output with the cached masked
// output: the accumulator starts at zero, the reference is the first tile's
// row max, and the residual is fetched in the epilogue, which computes
// O = acc * Z_sparse / (Z * Z_full) + R / Z_full.  O leaves through the V
// slot as whole lines.  All global traffic goes through buffer resources
// whose byte limit zero-fills rows past N on loads and drops them on stores.
template <int D, bool RB, bool V2>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 3, 4)))
sparse_occ_kernel(AttnArgs a, PersistGrid pg) {
  constexpr int NT = Shape<D>::NT, KS = Shape<D>::KS, TILE = Shape<D>::TILE, ROW = Shape<D>::ROW;
  constexpr int NRL = D / 8;                  // residual loads per lane
  constexpr int NLD = V2 ? 2 : NRL + 3;       // loads issued after a query block's Q (statistics, R1: residual)
  __shared__ __attribute__((aligned(1024))) char ring[2 * TILE];  // K slot, V slot
  __shared__ int redo[2];  // per wave: a row of its 32 left the fixed reference's range
  char* const kslot = ring;
  char* const vslot = ring + TILE;

  const uint32_t xcd = blockIdx.x % 8u, rr = blockIdx.x / 8u;
  const uint32_t start = xcd * pg.per, end = min(pg.total, start + pg.per);
  if (start + rr >= end) return;
  const int n_items = (int)((end - start - rr + pg.g - 1) / pg.g);
  const int Nb = a.Nb, N = a.N, keep = a.keep;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31, G = lane >> 4, i16 = lane & 15;
  const int rowq = wave * 32 + l32;  // row within the query block
  const float c = a.alpha * kLog2e;
  auto item_at = [&](int k) { return start + rr + (uint32_t)k * pg.g; };
  // The arguments used once per query block (tensor and cache pointers) are
  // read again from the kernel-argument segment where they are used, with
  // scalar loads, instead of being held in scalar registers (and spilled) for
  // the whole kernel.
  auto args = [&]() {
    typedef const __attribute__((address_space(4))) AttnArgs* kptr;
    kptr p = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    static_assert(sizeof(AttnArgs) == 112, "the copy below names every field of AttnArgs");
    AttnArgs r;
    r.q = p->q; r.k = p->k; r.v = p->v; r.o = p->o;
    r.idx = p->idx; r.idx_cache = p->idx_cache;
    r.m = p->m; r.z_full = p->z_full; r.z_sparse = p->z_sparse; r.R = p->R;
    r.BH = p->BH; r.N = p->N; r.Nb = p->Nb; r.keep = p->keep;
    r.alpha = p->alpha; r.r_bf16 = p->r_bf16; r.variant = p->variant;
    return r;
  };

  // LDS that no DMA has written yet must still read as finite numbers.
  {
    const u32x4 zero = {};
#pragma unroll
    for (int i = 0; i < 2 * TILE / (16 * 128); ++i) *(u32x4*)(ring + (i * 128 + (int)threadIdx.x) * 16) = zero;
    __syncthreads();
  }

  PipeDma<D> dma;
  dma.init(wave, lane);
  uint32_t ka[KS], va[NT][2];  // LDS addresses of this lane's K and V^T operands
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ka[ks] = lds_addr(kslot) + lds_off<D>(l32, 2 * ks + g);
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      // ds_read_b64_tr_b16 transposes within 16-lane groups: lane i of a group
      // points at key kbase + i/4, columns 4(i%4)..+3, and receives column i of
      // keys kbase..kbase+3.
      const int key = 8 * hh + 4 * g + (i16 >> 2);
      const int doff = 32 * dt + 16 * (G & 1) + 4 * (i16 & 3);
      va[dt][hh] = lds_addr(vslot) + lds_off<D>(key, doff >> 3) + (doff & 7) * 2;
    }

  PipeItem<D> it, nit;  // query block being computed, and the next one
  it.set(a, item_at(0));
  nit.set(a, item_at(min(1, n_items - 1)));
  // Tile whose K went out last: its V tile and valid bytes.  The list entry
  // of the tile after it is read one tile ahead and clamped only when used.
  const size_t blk = (size_t)kBlock * D * 2;
  auto clampb = [&](int x) { return min(max(x, 0), Nb - 1); };
  int j = it.block(0, Nb);
  int jnext = keep > 1 ? it.raw(1) : nit.raw(0);
  int tbytes = min(N - j * kBlock, kBlock) * D * 2;
  const char* vtile = it.vh + (size_t)j * blk;
  dma.issue_at(kslot, it.kh + (size_t)j * blk, tbytes);  // K of the first tile

  bf16x8 q[KS];
  f32x16 o[NT];
  PipeStats<D> st;
  // Q of query block `it` into the V slot, each wave its own 32 rows (read
  // back at the block's first tile, before the wave's V DMA overwrites
  // them), then the statistics and (R1) the residual, straight into the
  // accumulator: NLD loads after the Q DMA.
  const size_t qblk = (size_t)kBlock * D * 2;
  // The accumulator's starting value: the cached residual (R1), or zero.
  auto init_acc = [&]() {
    if (V2) {
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] = f32x16{};
    } else {
      f32x4 r[NT][4];
      load_residual<D, RB>(r, args(), it.bh, it.qi, rowq, g);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] = r[t][i >> 2][i & 3];
    }
  };
  // S^T = K Q^T of the tile in the K slot, one 32-key half at a time.
  auto tile_scores = [&](f32x16 (&s)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 kk[KS];
      k_half<KS>(kk, ka, t * 32 * ROW);
      s[t] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kk[ks]), q[ks], s[t], 0, 0, 0);
    }
  };
  // O^T += V^T P^T with the tile in the V slot, one d tile at a time.
  auto tile_pv = [&](const bf16x8 (&p)[2][2]) {
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      u32x2 h[2][2][2];
      tr_reads<0, 32 * ROW, 16 * ROW>(h, va[dt][0], va[dt][1]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const u32x4 both = __builtin_shufflevector(h[t][hs][0], h[t][hs][1], 0, 1, 2, 3);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), p[t][hs], o[dt], 0, 0, 0);
        }
    }
  };
  auto load_rows = [&]() {
    const AttnArgs aa = args();
    dma.template issue_at<kNT>(vslot, (const char*)aa.q + ((size_t)it.bh * N * D * 2 + (size_t)it.qi * qblk),
                               min(N - it.qi * kBlock, kBlock) * D * 2);
    load_stats<D, V2>(st, aa, it.bh, it.qi, rowq);
    init_acc();
  };
  load_rows();

  for (int k = 0; k < n_items; ++k) {
    float mr, z;
    // The per-tile maximum: on the block's second walk, and always at d_pad 80
    // (whose calls are latency-bound and have no registers to spare for the
    // redo path).
    bool careful = D != 64;
    for (;;) {
    mr = V2 ? -INFINITY : st.mc * kLog2e;
    z = 0.f;
    int jprev = -1;  // a list entry equal to its predecessor is walked with every key masked
    for (int n = 0; n < keep; ++n) {
      // 1. K_n has landed (the loads issued after it may still be in flight).
      //    At n = 0 the wave's Q rows have landed too: read them before the
      //    wave's V DMA overwrites its half of the V slot.
      if (n == 0) {
        wait_vmcnt<NLD>();
        wg_barrier();
        u32x4 qq[KS];
        k_half<KS>(qq, ka, TILE + wave * 32 * ROW);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) q[ks] = __builtin_bit_cast(bf16x8, qq[ks]);
      } else {
        wait_vmcnt<0>();
        wg_barrier();
      }
      dma.issue_at(vslot, vtile, tbytes);
      const int nvalid = j == jprev ? 0 : tbytes / (D * 2);
      jprev = j;
      // 2. scores and P against the reference mr: the cached row max (R1) or,
      //    for R2, the row max of the block's first tile (it always holds a
      //    valid key).  The first walk takes no per-tile maximum; a row that
      //    leaves the float32 range there is caught after the block, and the
      //    block is walked again with the lazy maximum (raise the reference
      //    when a tile's row max passes it by a factor 2^8).
      f32x16 s[2];
      tile_scores(s);
      if (nvalid < kBlock) mask_keys<D>(s, nvalid);
      if (careful || (V2 && n == 0)) {
        const float mx = row_max(s) * c;
        if (__ballot(mx > mr + kLazyLog2) != 0ull) {
          const float mnew = fmaxf(mr, mx);
          const float corr = __builtin_amdgcn_exp2f(mr - mnew);
          mr = mnew;
          z *= corr;
#pragma unroll
          for (int t = 0; t < NT; ++t) o[t] *= corr;
        }
      }
      bf16x8 p[2][2];
      probs_ref(p, s, mr, c);
      z += sum_rounded(p);
      // 3. V_n has landed; K_n is consumed: K of the next tile goes out.
      wait_vmcnt<0>();
      wg_barrier();
      if (n + 1 < keep || k + 1 < n_items) {
        const bool same = n + 1 < keep;  // the next tile is in this query block
        j = clampb(jnext);
        tbytes = min(N - j * kBlock, kBlock) * D * 2;
        vtile = (same ? it.vh : nit.vh) + (size_t)j * blk;
        dma.issue_at(kslot, (same ? it.kh : nit.kh) + (size_t)j * blk, tbytes);
        // list entry of the tile after it
        if (n + 2 < keep) jnext = it.raw(n + 2);
        else if (n + 2 == keep) jnext = nit.raw(0);
        else if (keep > 1) jnext = nit.raw(1);
        else {  // one block per query block: the block after next
          PipeItem<D> t2;
          t2.set(args(), item_at(min(k + 2, n_items - 1)));
          jnext = t2.raw(0);
        }
      }
      // 4. P.V
      tile_pv(p);
    }
    // A row sum at 2^64 or more, or not finite, means a score rose far enough
    // above the reference for P or the accumulator to overflow: both waves
    // walk the block again with the per-tile maximum.
    if (careful) break;
    const bool bad = __ballot(!(pair_sum(z) < 0x1p64f)) != 0ull;  // every lane's row, all lanes active
    if (lane == 0) redo[wave] = bad;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    wg_barrier();
    if ((redo[0] | redo[1]) != 0) {
      // Back to this block's first tile: drain, its first K again, then its Q,
      // statistics and accumulator in the same order as for a new block.
      wait_vmcnt<0>();
      wg_barrier();
      j = it.block(0, Nb);
      jnext = keep > 1 ? it.raw(1) : nit.raw(0);
      tbytes = min(N - j * kBlock, kBlock) * D * 2;
      vtile = it.vh + (size_t)j * blk;
      dma.issue_at(kslot, it.kh + (size_t)j * blk, tbytes);
      load_rows();
      careful = true;
      continue;
    }
    break;
    }
    // O = acc * Z_sparse / (Z * Z_full) (+ R / Z_full for R2); rows past N
    // are dropped by the limit.
    {
      const float w = st.zs / (pair_sum(z) * st.zf);
      const float u = 1.f / st.zf;
      f32x4 rv[NT][4];  // R2: the residual, fetched now (no registers are free during the tiles)
      if (V2) {
        load_residual<D, RB>(rv, args(), it.bh, it.qi, rowq, g);
        wait_vmcnt<0>();
      }
      const size_t r0 = (size_t)it.bh * N + (size_t)it.qi * kBlock;
      const __amdgpu_buffer_rsrc_t ro =
          make_rsrc((const char*)args().o + r0 * D * 2, min(N - it.qi * kBlock, kBlock) * D * 2);
      // The output goes through the V slot (free once both waves are past
      // their last P.V): each wave writes its 32 rows there in the MFMA
      // layout, reads them back row-contiguous and stores whole 128-byte
      // lines, instead of 16 bytes of 32 different lines per store
      // instruction.  d = 64 rows (128 bytes) have their 16-byte units
      // XOR-swizzled by row & 7 against bank conflicts on the writes; the
      // 160-byte rows of d = 80 spread over the banks as they are.
      constexpr int RBYTES = D * 2;
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's V reads are done
      wg_barrier();
      char* const stage = vslot + wave * 32 * ROW;  // this wave's half of the slot
      // Offsets are made opaque per query block so that the compiler keeps
      // one register for them rather than hoisting every derived address
      // out of the loop.
      uint32_t woff = D == 64 ? l32 * 128 + (l32 & 7) * 16 : l32 * RBYTES;
      uint32_t roff = D == 64 ? (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) * 16) : lane * 16;
      asm volatile("" : "+v"(woff), "+v"(roff));
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          if (32 * t + 8 * i4 < D) {
            __bf16 ob[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              ob[e] = V2 ? (__bf16)fmaf(o[t][4 * i4 + e], w, rv[t][i4][e] * u) : (__bf16)(o[t][4 * i4 + e] * w);
            const uint32_t unit = 4 * t + i4;
            const uint32_t at = D == 64 ? (woff ^ (unit * 16)) : woff + unit * 16;
            *(u32x2*)(stage + at + 8 * g) = *(u32x2*)ob;
          }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // 16-byte unit c*64 + lane of the wave's 32 rows, row-major: the same
      // linear offset in the output.
#pragma unroll
      for (int cc = 0; cc < 32 * RBYTES / 1024; ++cc) {
        const u32x4 v = *(const u32x4*)(stage + roff + cc * 1024);
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, wave * 32 * RBYTES + (int)lane * 16 + cc * 1024, 0, 0);
      }
    }
    if (k + 1 < n_items) {
      it = nit;
      nit.set(args(), item_at(min(k + 2, n_items - 1)));
      load_rows();
    }
  }
}

// Every residual type and epilogue of the sparse kernel, instantiated
// explicitly (the host compiler otherwise emits the launch stub of only one).
template __global__ void sparse_occ_kernel<64, false, false>(AttnArgs, PersistGrid);
template __global__ void sparse_occ_kernel<64, true, false>(AttnArgs, PersistGrid);
template __global__ void sparse_occ_kernel<80, false, false>(AttnArgs, PersistGrid);
template __global__ void sparse_occ_kernel<80, true, false>(AttnArgs, PersistGrid);
template __global__ void sparse_occ_kernel<64, false, true>(AttnArgs, PersistGrid);
template __global__ void sparse_occ_kernel<64, true, true>(AttnArgs, PersistGrid);
template __global__ void sparse_occ_kernel<80, false, true>(AttnArgs, PersistGrid);
template __global__ void sparse_occ_kernel<80, true, true>(AttnArgs, PersistGrid);

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
  // Every key block is added to the all-keys accumulator (in place, the same
  // registers each step); kept blocks are also added to the kept accumulator.
  // The residual is the difference at the end: with every block kept the two
  // see identical operations, so R = 0 and Z_sparse = Z_full exactly.
  f32x16 oall[NT], okept[NT];
  float zall, zk;

  // lazy: the reference max follows the running row max (rescaling when it
  // rises past 2^8).  Otherwise it stays at block 0's row max and only the
  // running max of the raw scores is kept, per lane (no exchange per block);
  // a row sum that leaves the float32 range is caught after the walk.
  template <int SLOT>
  __device__ __forceinline__ void step(int j, bool lazy) {
    wait_tile<Dma::IPT>(min(NBUF - 2, Nb - 1 - j));
    wg_barrier();
    if (j + NBUF - 1 < Nb) {
      constexpr int NEXT = (SLOT + NBUF - 1) % NBUF;
      dma.issue(ring + NEXT * Shape<D>::SLOT, kbase, vbase, j + NBUF - 1, N);
    }
    if (!active) return;
    const bool kept = __builtin_amdgcn_readfirstlane(flags[j]) != 0;
    f32x16 s[2];
    if constexpr (D == 80) scores_lean<D, SLOT * Shape<D>::SLOT>(s, st, fr, min(kBlock, N - j * kBlock));
    else scores<D, SLOT * Shape<D>::SLOT>(s, st, fr, min(kBlock, N - j * kBlock));
    if (lazy) {
      bool any;
      const float corr = update_max(st.m_ref, st.m_true, row_max(s), c, &any);
      if (any) {
        zall *= corr;
        zk *= corr;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          oall[t] *= corr;
          okept[t] *= corr;
        }
      }
    } else {
      float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        m0 = fmaxf(m0, s[0][i]);
        m1 = fmaxf(m1, s[1][i]);
      }
      st.m_true = fmaxf(st.m_true, fmaxf(m0, m1));
      if (j == 0) st.m_ref = pair_max(st.m_true);
    }
    bf16x8 p[2][2];
    const float zb = probs(p, s, st.m_ref, c);  // float32 sums of the exact exponentials
    zall += zb;
    if constexpr (D == 80) {
      pv_lean<D, SLOT * Shape<D>::SLOT>(oall, p, fr);
      if (kept) {
        zk += zb;
        pv_lean<D, SLOT * Shape<D>::SLOT>(okept, p, fr);
      }
    } else {
      u32x2 h[NT][2][2][2];
      v_fetch<D, SLOT * Shape<D>::SLOT>(h, fr);
      pv_mfma<D>(oall, p, h);
      if (kept) {
        zk += zb;
        pv_mfma<D>(okept, p, h);
      }
    }
  }
};

template <int D, int NBUF, int QB, bool RB>
__global__ void __launch_bounds__(128 * QB) __attribute__((amdgpu_waves_per_eu(D == 80 ? 2 : 1, 4)))
calib_kernel(AttnArgs a, XcdGrid grid) {
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

  __shared__ int redo[2 * QB];
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
  for (int t = 0; t < NT; ++t) cx.oall[t] = cx.okept[t] = f32x16{};
  cx.zall = cx.zk = 0.f;
  __syncthreads();  // flags and Q in place

  // d_pad 64 walks first with the reference fixed at block 0's row max.  A
  // wave whose row sums reach 2^64 (or are not finite) walks again with the
  // lazy maximum; the other waves keep their results and only take part in
  // the tile loads and barriers of that walk.
  bool lazy = D != 64;
  for (;;) {
#pragma unroll
    for (int t = 0; t < NBUF - 1; ++t)
      if (t < Nb) cx.dma.issue(ring + t * Shape<D>::SLOT, cx.kbase, cx.vbase, t, N);
    for (int j = 0; j < Nb; j += NBUF) {
      cx.template step<0>(j, lazy);
      if (j + 1 < Nb) cx.template step<1>(j + 1, lazy);
      if constexpr (NBUF > 2)
        if (j + 2 < Nb) cx.template step<2>(j + 2, lazy);
    }
    if (lazy) break;
    const bool bad = cx.active && __ballot(!(pair_sum(cx.zall) < 0x1p64f)) != 0ull;  // every lane votes
    if (lane == 0) redo[wave] = bad;
    wg_barrier();  // also: every wave is done with the ring before it is refilled
    bool again = false;
#pragma unroll
    for (int w = 0; w < 2 * QB; ++w) again |= redo[w] != 0;
    if (!again) break;
    cx.active = bad;
    if (bad) {
#pragma unroll
      for (int t = 0; t < NT; ++t) cx.oall[t] = cx.okept[t] = f32x16{};
      cx.zall = cx.zk = 0.f;
      cx.st.m_ref = cx.st.m_true = -INFINITY;
    }
    lazy = true;
  }

  // Statistics relative to the true row max m: factor e^{m_ref - m}.
  cx.st.m_true = pair_max(cx.st.m_true);  // the fixed-reference walk keeps a per-lane max
  const float f = __builtin_amdgcn_exp2f((cx.st.m_ref - cx.st.m_true) * cx.c);
  const float zs = pair_sum(cx.zk) * f;
  const float zf = pair_sum(cx.zall) * f;
  const size_t srow = (size_t)bh * N + row;
  if (row_ok && g == 0) {
    a.m[srow] = cx.st.m_true * a.alpha;
    a.z_full[srow] = zf;
    a.z_sparse[srow] = zs;
  }
  // The residual goes out for every row of the block, the padding rows past N
  // included (they repeat query row N-1, so the values are finite), in
  // the cache's accumulator order: each store is one run over the wave's
  // lanes.  O only for the rows that exist.
  if (qi < Nb) {
    const float inv = 1.f / zf;
    __bf16* orow = (__bf16*)a.o + srow * D;
    const size_t rblock = ((size_t)bh * Nb + qi) * kBlock * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * t + 8 * i4 + 4 * g;
        if (d < D) {
          const size_t at = rblock + (size_t)(((wave & 1) * (D / 8) + 4 * t + i4) * 64 + lane) * 4;
          f32x4 r;
          __bf16 ob[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = (cx.oall[t][4 * i4 + e] - cx.okept[t][4 * i4 + e]) * f;
            ob[e] = (__bf16)(cx.oall[t][4 * i4 + e] * f * inv);
          }
          if (RB) {  // residual rounded to bf16 (nearest even)
            __bf16 rb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rb[e] = (__bf16)r[e];
            *(u32x2*)((__bf16*)a.R + at) = *(u32x2*)rb;
          } else {
            *(f32x4*)(a.R + at) = r;
          }
          if (row_ok) *(u32x2*)(orow + d) = *(u32x2*)ob;
        }
      }
  }
}

constexpr int kCalibRing = 2;
// Sparse kernel workgroups per XCD: 8 per CU for d_pad 64 (16 KB of LDS and
// <= 128 VGPRs each), 6 for d_pad 80 (24 KB, <= 168 VGPRs).
constexpr int kSparseWgPerXcd64 = 32 * 8;
constexpr int kSparseWgPerXcd80 = 32 * 6;

template <int D>
hipError_t launch_d(AttnMode mode, const AttnArgs& a, hipStream_t s) {
  if (mode == AttnMode::kSparse) {
    const uint32_t total = (uint32_t)a.BH * (uint32_t)a.Nb;
    PersistGrid pg{total, (total + 7u) / 8u, 0u};
    pg.g = min(pg.per, (uint32_t)(D == 64 ? kSparseWgPerXcd64 : kSparseWgPerXcd80));
    const dim3 grid(8u * pg.g), block(128);
    if (a.variant == 1) {
      if (a.r_bf16)
        hipLaunchKernelGGL((sparse_occ_kernel<D, true, true>), grid, block, 0, s, a, pg);
      else
        hipLaunchKernelGGL((sparse_occ_kernel<D, false, true>), grid, block, 0, s, a, pg);
    } else {
      if (a.r_bf16)
        hipLaunchKernelGGL((sparse_occ_kernel<D, true, false>), grid, block, 0, s, a, pg);
      else
        hipLaunchKernelGGL((sparse_occ_kernel<D, false, false>), grid, block, 0, s, a, pg);
    }
  } else {
    constexpr int QB = 2;  // 2*QB waves must divide the LDS row units; 2 workgroups per CU
    const uint32_t groups = (uint32_t)(a.Nb + QB - 1) / QB;
    XcdGrid grid = make_xcd_grid((uint32_t)a.BH * groups);
    if (a.r_bf16)
      hipLaunchKernelGGL((calib_kernel<D, kCalibRing, QB, true>), dim3(grid.grid()), dim3(128 * QB), 0, s, a, grid);
    else
      hipLaunchKernelGGL((calib_kernel<D, kCalibRing, QB, false>), dim3(grid.grid()), dim3(128 * QB), 0, s, a, grid);
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
