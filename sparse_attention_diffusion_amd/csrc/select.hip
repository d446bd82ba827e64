// Block selector: mean-pooled Q/K per 64-token block, pooled logits, and a
// per-query-block top-k with always-kept (forced) blocks.
//
// Method: the Re-ttention project page keeps a small fraction of the tokens
// (Abstract: 3.1% in its experiments).  How the subset is chosen is not spelled out
// there; this library scores 64-token blocks by the scaled dot product of
// their mean query and mean key and keeps, per query block, the forced blocks
// plus the best remaining ones (ties to the lower block index).
//
// Kernels
//   pool_k_kernel : one wave per (bh, key block) mean of K, HBM-bound (K read
//                   once), written transposed ([bh][d][block]).
//   select_kernel : pools its own query blocks straight from Q (no round trip
//                   of the query means through memory), scores them against
//                   the K means staged 64 blocks at a time in LDS, and takes
//                   each query block's kept list: forced blocks plus the
//                   keep - n_forced best others (rounds of a wave-wide maximum
//                   of 64-bit keys; a bitonic sort in LDS above 32 winners).
#include <mutex>
#include <vector>

#include "internal.h"

namespace rettn {

// Pooled means of the allocation-free entry point (rt_select_blocks_noalloc).
// Each GPU the library runs on holds its own copy until the process ends.  In
// host code this name is only a stand-in for the symbol: the device address
// comes from select_scratch() and is the only form passed to kernels.
static __device__ __align__(256) char scratch[kSelectScratchBytes];

hipError_t select_scratch(void** out) {
  static std::mutex mu;
  static std::vector<void*> ptrs;  // per device id
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte chunk of T elements, widened to float32.
template <typename T>
struct Chunk;
template <>
struct Chunk<float> {
  static constexpr int E = 4;
  __device__ static void widen(u32x4 c, float (&f)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(c[e]);
  }
};
template <>
struct Chunk<__bf16> {
  static constexpr int E = 8;
  __device__ static void widen(u32x4 c, float (&f)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(c[e] << 16);
      f[2 * e + 1] = __uint_as_float(c[e] & 0xFFFF0000u);
    }
  }
};

// Mean of every key block, written transposed ([bh][d][block]) so that the
// selecting kernel reads a chunk of 64 blocks' means per d contiguously.
// One wave per (bh, block): the block's rows are read as 16-byte chunks, all
// at once; float32 partial sums per row group are reduced through LDS.
template <typename T, int D>
__global__ void __launch_bounds__(64) pool_k_kernel(SelectArgs a, XcdGrid grid) {
  constexpr int E = Chunk<T>::E;          // elements per 16-byte chunk
  constexpr int CPR = D / E;              // chunks per row
  constexpr int RPI = 64 / CPR;           // rows per pass of the wave
  constexpr int PASSES = (kBlock + RPI - 1) / RPI;
  static_assert(D % E == 0 && CPR <= 64, "row chunks");
  __shared__ float part[RPI][D];

  const uint32_t lin = grid.linear(blockIdx.x);
  if (lin >= grid.total) return;
  const int Nb = a.Nb, N = a.N;
  const int bh = lin / Nb, i = lin % Nb;
  const int lane = threadIdx.x;
  const int rg = lane / CPR, ch = lane % CPR;  // row in the pass, chunk in the row
  const int r0 = i * kBlock, rows = min(N - r0, kBlock);
  const char* base = (const char*)((const T*)a.k + ((size_t)bh * N + r0) * D);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (rg < RPI) {
    u32x4 c[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = p * RPI + rg;
      c[p] = r < rows ? __builtin_nontemporal_load((const u32x4*)(base + ((size_t)r * D + ch * E) * sizeof(T)))
                      : u32x4{};
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      float f[8];
      Chunk<T>::widen(c[p], f);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += f[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) part[rg][ch * E + e] = acc[e];
  }
  __syncthreads();
  const float inv = 1.f / (float)rows;
  for (int d = lane; d < D; d += 64) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < RPI; ++g) s += part[g][d];
    a.kb[((size_t)bh * D + d) * Nb + i] = s * inv;
  }
}

// Order-preserving map of a float32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// 64-bit value of another lane of the same row of 16, by DPP control C.
template <int C>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)x, C, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(x >> 32), C, 0xF, 0xF, false);
  return ((unsigned long long)hi << 32) | lo;
}

// Maximum over the wave, returned in every lane (uniform).  Within each row of
// 16 lanes: DPP quad permutations (lane ^ 1, lane ^ 2), then the half-row and
// row mirrors; the four row maxima are then read into scalar registers.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
  unsigned long long y;
  y = dpp_u64<0xB1>(x);   // quad_perm [1,0,3,2]
  x = y > x ? y : x;
  y = dpp_u64<0x4E>(x);   // quad_perm [2,3,0,1]
  x = y > x ? y : x;
  y = dpp_u64<0x141>(x);  // row_half_mirror
  x = y > x ? y : x;
  y = dpp_u64<0x140>(x);  // row_mirror
  x = y > x ? y : x;
  unsigned long long m = 0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const unsigned lo = __builtin_amdgcn_readlane((unsigned)x, 16 * r);
    const unsigned hi = __builtin_amdgcn_readlane((unsigned)(x >> 32), 16 * r);
    const unsigned long long v = ((unsigned long long)hi << 32) | lo;
    m = v > m ? v : m;
  }
  return m;
}

// The same for N independent values, each step taken for all of them before
// the next, so that their chains of lane exchanges overlap.
template <int N>
__device__ __forceinline__ void wave_max_u64_n(unsigned long long (&x)[N]) {
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const unsigned long long y = dpp_u64<0xB1>(x[n]);
    x[n] = y > x[n] ? y : x[n];
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const unsigned long long y = dpp_u64<0x4E>(x[n]);
    x[n] = y > x[n] ? y : x[n];
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const unsigned long long y = dpp_u64<0x141>(x[n]);
    x[n] = y > x[n] ? y : x[n];
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const unsigned long long y = dpp_u64<0x140>(x[n]);
    x[n] = y > x[n] ? y : x[n];
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
    unsigned long long m = 0ull;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const unsigned lo = __builtin_amdgcn_readlane((unsigned)x[n], 16 * r);
      const unsigned hi = __builtin_amdgcn_readlane((unsigned)(x[n] >> 32), 16 * r);
      const unsigned long long v = ((unsigned long long)hi << 32) | lo;
      m = v > m ? v : m;
    }
    x[n] = m;
  }
}

// Orders this wave's LDS accesses: one wave's LDS instructions execute in
// order, so every lane's earlier LDS writes are seen by later reads of any
// lane once the compiler keeps them in program order; this is that compiler
// barrier.  (A memory fence would also wait for the wave's global stores.)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kMaxRounds = 32;  // above this many non-forced winners: bitonic sort
constexpr int kMaxSelLds = 64 << 10;  // dynamic LDS of one selecting workgroup at most

// Query blocks per wave, at most: 4 (2 above 512 key blocks, where the
// per-lane scores take more registers), so that many waves share each SIMD.
template <int CH>
constexpr int query_group() { return CH <= 8 ? 4 : 2; }

// Dynamic LDS of select_kernel: a chunk of 64 blocks' K means, one row of
// D + 4 floats per block (16 bytes of padding keep a wave's 16-byte reads of
// 64 rows free of bank conflicts), shared by the workgroup, then per wave:
// pooled queries [QG][D],
// pooling partials [RPI][D] (floats), one flag row (Nb rounded up to 16
// bytes) and, for the bitonic fallback only, P 64-bit keys.
struct SelectLds {
  int kc_bytes, wave_bytes, q_off, part_off, flag_off, flag_stride, keys_off, bytes;
};
inline SelectLds select_lds(int W, int QG, int D, int RPI, int Nb, bool bitonic) {
  SelectLds l;
  l.kc_bytes = (D + 4) * 64 * 4;
  l.q_off = 0;
  l.part_off = QG * D * 4;
  l.flag_off = l.part_off + RPI * D * 4;
  l.flag_stride = (Nb + 15) & ~15;
  l.keys_off = (l.flag_off + l.flag_stride + 7) & ~7;
  int P = 64;
  while (P < Nb) P <<= 1;
  l.wave_bytes = (l.keys_off + (bitonic ? P * 8 : 0) + 15) & ~15;
  l.bytes = l.kc_bytes + W * l.wave_bytes;
  return l;
}

// Writes the kept list of one query block from its flag row (ascending).
__device__ __forceinline__ void emit(const unsigned char* flags, int Nb, int32_t* out) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int base = 0; base < Nb; base += 64) {
    const int j = base + lane;
    const bool f = j < Nb && flags[j];
    const unsigned long long mk = __ballot(f);
    if (f) out[cnt + __popcll(mk & ((1ull << lane) - 1ull))] = j;
    cnt += __popcll(mk);
  }
}

// The selecting kernel: pools its query blocks straight from q, scores them
// against the K means and takes each one's kept list.  One workgroup of
// W waves (4, or 2 where four would need more than 64 KB of LDS) per
// (bh, W * QG query blocks); wave w owns QG consecutive query blocks (QG is
// chosen per call, up to query_group<CH>()).
//   1. pooling: the rows of each of the wave's query blocks are read as
//      16-byte chunks, all at once, summed in float32 per row group and
//      reduced through the wave's LDS (then multiplied by 1/rows);
//   2. scores: the workgroup stages the K means of 64 key blocks at a time in
//      LDS; lane j of every wave scores key block 64c + j against the wave's
//      pooled queries (float32 products summed in ascending d);
//   3. per query block: forced blocks are flagged, the keep - n_forced
//      winners by (score desc, index asc) are taken by rounds of a wave-wide
//      maximum of 64-bit (score bits, ~index) keys (a bitonic sort in the
//      wave's LDS above 32 winners), and the list is written ascending from
//      the flag row with ballots.
// Only the staging of the K means synchronises the workgroup; everything
// else is wave-local, so waves with fewer (or no) query blocks never hold
// the others at a barrier.
template <typename T, int D, int CH, int W, int QG>
__global__ void __launch_bounds__(64 * W) select_kernel(SelectArgs a, XcdGrid grid, SelectLds lay) {
  constexpr int E = Chunk<T>::E, CPR = D / E, RPI = 64 / CPR, PASSES = (kBlock + RPI - 1) / RPI;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int KCS = D + 4;  // floats per key block row of the staged chunk
  float* const kc = (float*)smem;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  char* wb = smem + lay.kc_bytes + wave * lay.wave_bytes;
  float(*qrow)[D] = (float(*)[D])(wb + lay.q_off);
  float(*part)[D] = (float(*)[D])(wb + lay.part_off);
  unsigned char* flags = (unsigned char*)(wb + lay.flag_off);
  unsigned long long* keys = (unsigned long long*)(wb + lay.keys_off);

  const uint32_t lin = grid.linear(blockIdx.x);
  if (lin >= grid.total) return;  // the whole workgroup
  const int Nb = a.Nb, N = a.N, keep = a.keep;
  constexpr int QW = W * QG;
  const int groups = (Nb + QW - 1) / QW;
  const int bh = lin / groups;
  const int i0 = (lin % groups) * QW + wave * QG;  // this wave's first query block
  const int nq = max(0, min(QG, Nb - i0));

  // 1. pooled queries; the rows of block g + 1 are in flight while block g is
  // reduced.  A buffer resource per block zero-fills rows past N (branch-free).
  const int rg = lane / CPR, ch = lane % CPR;
  const int rgl = min(rg, RPI - 1);  // lanes past the last row group load a duplicate, unused
  u32x4 buf[2][PASSES];
  auto issue_rows = [&](u32x4 (&c)[PASSES], int g) {
    const int r0 = (i0 + g) * kBlock, rows = min(N - r0, kBlock);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>((const T*)a.q + ((size_t)bh * N + r0) * D), (short)0, rows * D * (int)sizeof(T), 0x00020000);
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
      c[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, ((p * RPI + rgl) * D + ch * E) * (int)sizeof(T), 0, 0));
  };
  if (nq > 0) issue_rows(buf[0], 0);
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    if (g < nq) {
      const int rows = min(N - (i0 + g) * kBlock, kBlock);
      if (g + 1 < nq) issue_rows(buf[(g + 1) & 1], g + 1);
      if (rg < RPI) {
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          float f[8];
          Chunk<T>::widen(buf[g & 1][p], f);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] += f[e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) part[rg][ch * E + e] = acc[e];
      }
      wave_sync();
      const float inv = 1.f / (float)rows;
      for (int d = lane; d < D; d += 64) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RPI; ++r) sum += part[r][d];
        qrow[g][d] = sum * inv;
      }
      wave_sync();
    } else {
      for (int d = lane; d < D; d += 64) qrow[g][d] = 0.f;  // unused; keeps the scores finite
    }
  }
  for (int e = lane; e < lay.flag_stride / 4; e += 64) ((uint32_t*)flags)[e] = 0u;
  int n_forced = 0;
#pragma unroll
  for (int w = 0; w < kMaxBlocks / 32; ++w) n_forced += __popc(a.forced[w]);
  wave_sync();

  // 2. scores of key blocks j = 64c + lane against the wave's pooled queries
  // The next chunk's means are loaded into registers while this one is scored.
  const float* kt = a.kb + (size_t)bh * D * Nb;  // transposed means [d][j]
  const int nc = (Nb + 63) / 64;
  constexpr int PER = D / W;  // means per thread and chunk
  float nxt[PER];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int e = (int)threadIdx.x + r * 64 * W;
      nxt[r] = kt[(size_t)(e >> 6) * Nb + min(c * 64 + (e & 63), Nb - 1)];
    }
  };
  load_chunk(0);
  float sc[QG][CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c < nc) {  // the same for the whole workgroup
      __syncthreads();  // the previous chunk is consumed
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int e = (int)threadIdx.x + r * 64 * W;
        kc[(e & 63) * KCS + (e >> 6)] = nxt[r];
      }
      __syncthreads();
      if (c + 1 < nc) load_chunk(c + 1);
      float acc[QG];
#pragma unroll
      for (int g = 0; g < QG; ++g) acc[g] = 0.f;
#pragma unroll
      for (int d0 = 0; d0 < D; d0 += 4) {
        const f32x4 kv = *(const f32x4*)&kc[lane * KCS + d0];
#pragma unroll
        for (int g = 0; g < QG; ++g) {
          const f32x4 qv = *(const f32x4*)&qrow[g][d0];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[g] = fmaf(qv[e], kv[e], acc[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < QG; ++g) sc[g][c] = acc[g] * a.alpha + 0.0f;  // + 0: -0 -> +0
    }
  }

  // 3. the kept lists.  64-bit keys: order-preserving score bits, then ~j
  // (ties to the lower j); 0 marks no candidate (a forced block, a block past
  // Nb, a query block the wave does not own).  Forced blocks take no round.
  const int rounds = keep - n_forced;
  if (a.scores) {
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      if (g >= nq) break;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int j = c * 64 + lane;
        if (c < nc && j < Nb) a.scores[((size_t)bh * Nb + i0 + g) * Nb + j] = sc[g][c];
      }
    }
  }
  auto is_forced = [&](int j) { return ((a.forced[j >> 5] >> (j & 31)) & 1u) != 0u; };
  auto key_of = [&](int g, int c) {
    const int j = c * 64 + lane;
    return (g < nq && c < nc && j < Nb && !is_forced(j))
               ? (((unsigned long long)order_key(sc[g][c]) << 32) | (0xFFFFFFFFu - (uint32_t)j))
               : 0ull;
  };
  auto flag_forced = [&]() {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int j = c * 64 + lane;
      if (c < nc && j < Nb && is_forced(j)) flags[j] = 1;
    }
  };
  auto emit_and_clear = [&](int g) {
    wave_sync();
    emit(flags, Nb, a.idx + ((size_t)bh * Nb + i0 + g) * keep);
    wave_sync();
    for (int e = lane; e < lay.flag_stride / 4; e += 64) ((uint32_t*)flags)[e] = 0u;  // for the next block
    wave_sync();
  };
  if (rounds <= kMaxRounds) {
    // The rounds of the wave's QG query blocks run side by side (independent
    // chains of lane exchanges); lane t of win[g] keeps round t's winner of
    // block g, -1 once no candidate is left (more rounds than blocks).
    unsigned long long kk[QG][CH];
    int win[QG];
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      win[g] = -1;
#pragma unroll
      for (int c = 0; c < CH; ++c) kk[g][c] = key_of(g, c);
    }
    for (int t = 0; t < rounds; ++t) {
      unsigned long long best[QG];
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        best[g] = 0ull;
#pragma unroll
        for (int c = 0; c < CH; ++c) best[g] = kk[g][c] > best[g] ? kk[g][c] : best[g];
      }
      wave_max_u64_n<QG>(best);
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        const int jw = best[g] != 0ull ? (int)(0xFFFFFFFFu - (uint32_t)(best[g] & 0xFFFFFFFFull)) : -1;
        if (lane == t) win[g] = jw;
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (jw >= 0 && c == (jw >> 6) && lane == (jw & 63)) kk[g][c] = 0ull;
      }
    }
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      if (g >= nq) break;
      flag_forced();
      if (lane < rounds && win[g] >= 0) flags[win[g]] = 1;
      emit_and_clear(g);
    }
  } else {
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      if (g >= nq) break;
      unsigned long long kk[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) kk[c] = key_of(g, c);
      flag_forced();
      // Bitonic sort of the non-forced keys, descending, in this wave's LDS.
      int P = 64;
      while (P < Nb) P <<= 1;
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (c * 64 < P) keys[c * 64 + lane] = kk[c];
      // P can exceed the CH*64 keys this lane holds (CH = 5 sorts 512 keys):
      // the rest of the sort buffer is padding and must lose every compare.
      for (int t = CH * 64 + lane; t < P; t += 64) keys[t] = 0ull;
      wave_sync();
      for (int k = 2; k <= P; k <<= 1) {
        for (int jx = k >> 1; jx > 0; jx >>= 1) {
          for (int t = lane; t < (P >> 1); t += 64) {
            const int lo = (t / jx) * 2 * jx + (t % jx);
            const int hi = lo + jx;
            const unsigned long long x = keys[lo], y = keys[hi];
            const bool desc = (lo & k) == 0;
            if ((x < y) == desc) {
              keys[lo] = y;
              keys[hi] = x;
            }
          }
          wave_sync();
        }
      }
      // rounds <= Nb - n_forced candidates, so the first `rounds` keys are real;
      // a padding key (0) is still skipped rather than trusted.
      for (int t = lane; t < rounds; t += 64)
        if (keys[t] != 0ull) flags[0xFFFFFFFFu - (uint32_t)(keys[t] & 0xFFFFFFFFull)] = 1;
      emit_and_clear(g);
    }
  }
}

template <typename T, int D, int CH, int QG>
void launch_select_qg(const SelectArgs& a, bool bitonic, hipStream_t s) {
  constexpr int RPI = 64 / (D / Chunk<T>::E);
  const SelectLds l4 = select_lds(4, QG, D, RPI, a.Nb, bitonic);
  if (l4.bytes <= kMaxSelLds) {
    XcdGrid sg = make_xcd_grid((uint32_t)a.BH * (uint32_t)((a.Nb + 4 * QG - 1) / (4 * QG)));
    hipLaunchKernelGGL((select_kernel<T, D, CH, 4, QG>), dim3(sg.grid()), dim3(256), l4.bytes, s, a, sg, l4);
  } else {
    const SelectLds l2 = select_lds(2, QG, D, RPI, a.Nb, bitonic);
    XcdGrid sg = make_xcd_grid((uint32_t)a.BH * (uint32_t)((a.Nb + 2 * QG - 1) / (2 * QG)));
    hipLaunchKernelGGL((select_kernel<T, D, CH, 2, QG>), dim3(sg.grid()), dim3(128), l2.bytes, s, a, sg, l2);
  }
}

// Query blocks per wave: the most (each wave then reads the K means once for
// more query blocks) that still give at least 1536 four-wave workgroups;
// smaller calls are latency-bound and run faster as more, shorter workgroups
// (measured: 4 best at B*H*Nb = 96*278, 2 at 60*278, 1 at 32*64).
template <typename T, int D, int CH>
void launch_select_ch(const SelectArgs& a, hipStream_t s) {
  int n_forced = 0;
  for (int w = 0; w < kMaxBlocks / 32; ++w) n_forced += __builtin_popcount(a.forced[w]);
  const bool bitonic = a.keep - n_forced > kMaxRounds;
  if constexpr (query_group<CH>() == 4) {
    auto wgs = [&](int qg) { return (uint32_t)a.BH * (uint32_t)((a.Nb + 4 * qg - 1) / (4 * qg)); };
    if (wgs(4) >= 1536u) launch_select_qg<T, D, CH, 4>(a, bitonic, s);
    else if (wgs(2) >= 1536u) launch_select_qg<T, D, CH, 2>(a, bitonic, s);
    else launch_select_qg<T, D, CH, 1>(a, bitonic, s);
  } else {
    launch_select_qg<T, D, CH, query_group<CH>()>(a, bitonic, s);
  }
}

template <typename T, int D>
hipError_t launch_typed(const SelectArgs& a, hipStream_t s) {
  XcdGrid pg = make_xcd_grid((uint32_t)a.BH * (uint32_t)a.Nb);
  hipLaunchKernelGGL((pool_k_kernel<T, D>), dim3(pg.grid()), dim3(64), 0, s, a, pg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nc = (a.Nb + 63) / 64;
  if (nc <= 1) launch_select_ch<T, D, 1>(a, s);
  else if (nc <= 2) launch_select_ch<T, D, 2>(a, s);
  else if (nc <= 4) launch_select_ch<T, D, 4>(a, s);
  else if (nc <= 5) launch_select_ch<T, D, 5>(a, s);
  else if (nc <= 8) launch_select_ch<T, D, 8>(a, s);
  else launch_select_ch<T, D, kMaxBlocks / 64>(a, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(bool bf16, int D, const SelectArgs& a, hipStream_t s) {
  if (D == 64) return bf16 ? launch_typed<__bf16, 64>(a, s) : launch_typed<float, 64>(a, s);
  if (D == 80) return bf16 ? launch_typed<__bf16, 80>(a, s) : launch_typed<float, 80>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace rettn
