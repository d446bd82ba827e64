// Block selector: mean-pooled Q/K per 64-token block, pooled logits, and a
// per-query-block top-k with always-kept (forced) blocks.
//
// Method: the Re-ttention project page keeps just a few of the tokens
// (Abstract: as few as 3.1%).  How the subset is chosen is not spelled out
// there; this library scores 64-token blocks by the scaled dot product of
// their mean query and mean key and keeps, per query block, the forced blocks
// plus the best remaining ones (ties to the lower block index).
//
// Kernels
//   pool_kernel   : one wave per (tensor, bh, block).  The block's rows are
//                   read as 16-byte chunks, all at once (HBM-bound: Q and K
//                   are read once); float32 partial sums per row group are
//                   reduced through LDS.  K means are written transposed
//                   ([bh][d][block]) so that scoring reads them coalesced.
//   select_kernel : one wave per (bh, QG = 8 query blocks; 4 above 512 key
//                   blocks).  Lane j scores key
//                   blocks j, j+64, ... against the QG pooled queries (float32
//                   dot products in ascending d), then each query block's
//                   keep - n_forced winners are taken by rounds of a wave-wide
//                   maximum of 64-bit (score, ~index) keys, and the list is
//                   written in ascending order through a flag row and ballots.
//                   Large selections fall back to a bitonic sort in LDS.
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

// grid.x: (bh, block) pairs laid out per XCD; grid.y: 0 = q, 1 = k.
template <typename T, int D>
__global__ void __launch_bounds__(64) pool_kernel(SelectArgs a, XcdGrid grid) {
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
  const bool isk = blockIdx.y != 0;
  const int lane = threadIdx.x;
  const int rg = lane / CPR, ch = lane % CPR;  // row in the pass, chunk in the row
  const int r0 = i * kBlock, rows = min(N - r0, kBlock);
  const char* base = (const char*)((const T*)(isk ? a.k : a.q) + ((size_t)bh * N + r0) * D);
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
    if (isk) a.kb[((size_t)bh * D + d) * Nb + i] = s * inv;  // transposed
    else a.qb[((size_t)bh * Nb + i) * D + d] = s * inv;
  }
}

// Order-preserving map of a float32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)x, o), hi = __shfl_xor((unsigned)(x >> 32), o);
    const unsigned long long y = ((unsigned long long)hi << 32) | lo;
    x = y > x ? y : x;
  }
  return x;
}

constexpr int kMaxRounds = 32;  // above this many non-forced winners: bitonic sort

// Query blocks per wave: 8 while the per-lane scores fit in registers.
template <int CH>
constexpr int query_group() { return CH <= 8 ? 8 : 4; }

// Dynamic LDS of select_kernel: pooled queries [QG][D] floats, flag rows
// [QG][Nb rounded up to 4] bytes, and (bitonic fallback only) P 64-bit keys.
struct SelectLds {
  int flag_stride, keys_off, bytes;
};
inline SelectLds select_lds(int QG, int D, int Nb, bool bitonic) {
  SelectLds l;
  l.flag_stride = (Nb + 3) & ~3;
  const int flags_off = QG * D * 4;
  l.keys_off = (flags_off + QG * l.flag_stride + 7) & ~7;
  int P = 64;
  while (P < Nb) P <<= 1;
  l.bytes = l.keys_off + (bitonic ? P * 8 : 0);
  return l;
}

// Writes the kept list of one query block from its flag row (ascending).
__device__ __forceinline__ void emit(const unsigned char* flags, int Nb, int32_t* out) {
  const int lane = threadIdx.x;
  int cnt = 0;
  for (int base = 0; base < Nb; base += 64) {
    const int j = base + lane;
    const bool f = j < Nb && flags[j];
    const unsigned long long mk = __ballot(f);
    if (f) out[cnt + __popcll(mk & ((1ull << lane) - 1ull))] = j;
    cnt += __popcll(mk);
  }
}

// CH: key blocks per lane (64-block chunks), at least ceil(Nb / 64).
template <int D, int CH>
__global__ void __launch_bounds__(64) select_kernel(SelectArgs a, XcdGrid grid, SelectLds lay) {
  constexpr int QG = query_group<CH>();
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float(*qrow)[D] = (float(*)[D])smem;
  unsigned char* flag0 = (unsigned char*)smem + QG * D * 4;
  unsigned long long* keys = (unsigned long long*)(smem + lay.keys_off);

  const uint32_t lin = grid.linear(blockIdx.x);
  if (lin >= grid.total) return;
  const int Nb = a.Nb, keep = a.keep;
  const int groups = (Nb + QG - 1) / QG;
  const int bh = lin / groups, i0 = (lin % groups) * QG;
  const int nq = min(QG, Nb - i0);
  const int lane = threadIdx.x;
  for (int e = lane; e < QG * D; e += 64) {
    const int g = e / D, d = e % D;
    qrow[g][d] = g < nq ? a.qb[((size_t)bh * Nb + i0 + g) * D + d] : 0.f;
  }
  for (int e = lane; e < QG * lay.flag_stride / 4; e += 64) ((uint32_t*)flag0)[e] = 0u;
  int n_forced = 0;
#pragma unroll
  for (int w = 0; w < kMaxBlocks / 32; ++w) n_forced += __popc(a.forced[w]);
  __syncthreads();

  // Scores of key blocks j = lane + 64c against the QG pooled queries: float32
  // products summed in ascending d; the K means of 16 d at a time are loaded
  // together.
  const float* kt = a.kb + (size_t)bh * D * Nb;  // transposed means [d][j]
  const int nc = (Nb + 63) / 64;
  float sc[QG][CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c < nc) {
      const int jj = min(c * 64 + lane, Nb - 1);
      float acc[QG];
#pragma unroll
      for (int g = 0; g < QG; ++g) acc[g] = 0.f;
#pragma unroll
      for (int d0 = 0; d0 < D; d0 += 16) {
        float kv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) kv[e] = kt[(size_t)(d0 + e) * Nb + jj];
#pragma unroll
        for (int e4 = 0; e4 < 16; e4 += 4)
#pragma unroll
          for (int g = 0; g < QG; ++g) {
            const f32x4 qv = *(const f32x4*)&qrow[g][d0 + e4];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[g] = fmaf(qv[e], kv[e4 + e], acc[g]);
          }
      }
#pragma unroll
      for (int g = 0; g < QG; ++g) sc[g][c] = acc[g] * a.alpha + 0.0f;  // + 0: -0 -> +0
    }
  }

#pragma unroll
  for (int g = 0; g < QG; ++g) {
    if (g >= nq) break;
    const int i = i0 + g;
    unsigned char* flags = flag0 + g * lay.flag_stride;
    if (a.scores) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int j = c * 64 + lane;
        if (c < nc && j < Nb) a.scores[((size_t)bh * Nb + i) * Nb + j] = sc[g][c];
      }
    }
    // 64-bit keys: order-preserving score bits, then ~j (ties to the lower j);
    // forced blocks are marked directly and take no round.
    unsigned long long kk[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int j = c * 64 + lane;
      kk[c] = 0ull;
      if (c < nc && j < Nb) {
        if ((a.forced[j >> 5] >> (j & 31)) & 1u) flags[j] = 1;
        else kk[c] = ((unsigned long long)order_key(sc[g][c]) << 32) | (0xFFFFFFFFu - (uint32_t)j);
      }
    }
    const int rounds = keep - n_forced;
    if (rounds <= kMaxRounds) {
      for (int t = 0; t < rounds; ++t) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int c = 0; c < CH; ++c) best = kk[c] > best ? kk[c] : best;
        best = wave_max_u64(best);
        if (best == 0ull) break;  // no candidate left (more rounds than blocks)
        const int jw = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
        if (lane == (jw & 63)) {
          flags[jw] = 1;
#pragma unroll
          for (int c = 0; c < CH; ++c)
            if (c == (jw >> 6)) kk[c] = 0ull;
        }
      }
    } else {
      // Bitonic sort of the non-forced keys, descending.
      int P = 64;
      while (P < Nb) P <<= 1;
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (c * 64 < P) keys[c * 64 + lane] = kk[c];
      // P can exceed the CH*64 keys this lane holds (CH = 5 sorts 512 keys):
      // the rest of the sort buffer is padding and must lose every compare.
      for (int t = CH * 64 + lane; t < P; t += 64) keys[t] = 0ull;
      __syncthreads();
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
          __syncthreads();
        }
      }
      // rounds <= Nb - n_forced candidates, so the first `rounds` keys are real;
      // a padding key (0) is still skipped rather than trusted.
      for (int t = lane; t < rounds; t += 64)
        if (keys[t] != 0ull) flags[0xFFFFFFFFu - (uint32_t)(keys[t] & 0xFFFFFFFFull)] = 1;
    }
    __syncthreads();
    emit(flags, Nb, a.idx + ((size_t)bh * Nb + i) * keep);
  }
}

template <int D, int CH>
void launch_select_ch(const SelectArgs& a, hipStream_t s) {
  constexpr int QG = query_group<CH>();
  int n_forced = 0;
  for (int w = 0; w < kMaxBlocks / 32; ++w) n_forced += __builtin_popcount(a.forced[w]);
  const SelectLds lay = select_lds(QG, D, a.Nb, a.keep - n_forced > kMaxRounds);
  XcdGrid sg = make_xcd_grid((uint32_t)a.BH * (uint32_t)((a.Nb + QG - 1) / QG));
  hipLaunchKernelGGL((select_kernel<D, CH>), dim3(sg.grid()), dim3(64), lay.bytes, s, a, sg, lay);
}

template <typename T, int D>
hipError_t launch_typed(const SelectArgs& a, hipStream_t s) {
  XcdGrid pg = make_xcd_grid((uint32_t)a.BH * (uint32_t)a.Nb);
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3(pg.grid(), 2), dim3(64), 0, s, a, pg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nc = (a.Nb + 63) / 64;
  if (nc <= 1) launch_select_ch<D, 1>(a, s);
  else if (nc <= 2) launch_select_ch<D, 2>(a, s);
  else if (nc <= 4) launch_select_ch<D, 4>(a, s);
  else if (nc <= 5) launch_select_ch<D, 5>(a, s);
  else if (nc <= 8) launch_select_ch<D, 8>(a, s);
  else launch_select_ch<D, kMaxBlocks / 64>(a, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(bool bf16, int D, const SelectArgs& a, hipStream_t s) {
  if (D == 64) return bf16 ? launch_typed<__bf16, 64>(a, s) : launch_typed<float, 64>(a, s);
  if (D == 80) return bf16 ? launch_typed<__bf16, 80>(a, s) : launch_typed<float, 80>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace rettn
