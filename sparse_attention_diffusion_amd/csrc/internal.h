// Internal interface between the C-ABI host layer (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rettn {

constexpr int kBlock = 64;         // tokens per block
constexpr int kMaxBlocks = 1024;   // Nb limit (N <= 65536)

enum class AttnMode : int { kCalibrate = 0, kSparse = 1 };

// Layout of the cached residual R (float32 or bf16 elements).  Each (b, h)
// holds Nb blocks of 64 rows x D, rows past N being padding.  Inside a block
// the element of row r and column c sits at
//   ((r / 32 * D / 8 + c / 8) * 64 + 32 * (c / 4 % 2) + r % 32) * 4 + c % 4,
// which is the order in which the 32x32 MFMA accumulators of a wave (rows
// 32 * (r / 32) onwards) hold the block: the 4 elements one lane loads or
// stores for an 8-column group are part of one contiguous run over the
// wave's 64 lanes.
__host__ __device__ inline size_t residual_index(size_t bh, int Nb, int D, int row, int col) {
  const int r = row % kBlock;
  const size_t block = (bh * (size_t)Nb + (size_t)(row / kBlock)) * (size_t)(kBlock * D);
  return block + (size_t)((((r >> 5) * (D / 8) + (col >> 3)) * 64 + 32 * ((col >> 2) & 1) + (r & 31)) * 4 + (col & 3));
}

// Everything one attention launch needs.  Tensors are [BH, N, D] row-major.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* idx;      // kept lists [BH, Nb, keep] used by this call
  int32_t* idx_cache;      // calibrate: destination of the list copy (may be null)
  float* m;                // statistics cache rows [BH, N]
  float* z_full;
  float* z_sparse;
  float* R;                // [BH, Nb * 64, D] in residual_index order: float32, or bf16 when r_bf16
  int32_t BH, N, Nb, keep;
  float alpha;             // 1/sqrt(d)
  int32_t r_bf16;          // residual stored as bf16 (bf16 kernels only)
  int32_t variant;         // sparse epilogue: 0 = R1 (residual rescaled by exp(m_c - M)),
                           // 1 = R2 (r * normalised sparse output + R / Z_full)
};

struct SelectArgs {
  const void* q;
  const void* k;
  float* kb;               // workspace: K means [BH, D, Nb] float32 (transposed)
  int32_t* idx;            // [BH, Nb, keep]
  float* scores;           // [BH, Nb, Nb] or null
  int32_t BH, N, Nb, keep;
  float alpha;
  uint32_t forced[kMaxBlocks / 32];  // bitmask of always-kept blocks
};

// Grid of `total` workgroups laid out so that each of the 8 XCDs (workgroups
// are handed to XCDs round-robin by id) receives one contiguous range.
struct XcdGrid {
  uint32_t total, per;
  __host__ __device__ uint32_t grid() const { return per * 8u; }
  __device__ uint32_t linear(uint32_t wg) const { return (wg % 8u) * per + wg / 8u; }
};
inline XcdGrid make_xcd_grid(uint32_t total) { return XcdGrid{total, (total + 7u) / 8u}; }

struct PermuteArgs {
  const void* src;
  void* dst;
  const int32_t* perm;     // [N], device
  int32_t BH, N;
  int32_t cpr;             // 16-byte chunks per row
  int32_t inverse;         // 0: dst[i] = src[perm[i]]; 1: dst[perm[i]] = src[i]
};

// Host: Hilbert-curve order of a grid (text tokens first).  perm has
// n_text + prod(dims) entries.
void hilbert_order(const int32_t* dims, int ndims, int n_text, int32_t* perm);

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
hipError_t launch_attn_bf16(AttnMode mode, int D, const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(AttnMode mode, int D, const AttnArgs& a, hipStream_t s);
hipError_t launch_select(bool bf16, int D, const SelectArgs& a, hipStream_t s);

// Scratch of the allocation-free selector: a static device array of this many
// bytes (select.hip) holding the K means.  select_scratch returns its
// address on the current device, looked up once per device.
constexpr size_t kSelectScratchBytes = size_t(16) << 20;
hipError_t select_scratch(void** ptr);

}  // namespace rettn
