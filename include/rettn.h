/*
 * rettn.h -- C ABI of the Re-ttention sparse-attention library for MI355X (gfx950).
 *
 * What it computes.  The Re-ttention project page ("Re-ttention: Ultra Sparse
 * Visual Generation via Attention Statistical Reshape") describes attention for
 * diffusion transformers that keeps few of the keys (Abstract:
 * down to 3.1% of the tokens) and corrects the resulting softmax
 * normalisation shift with statistics cached at an earlier denoising step
 * (teaser paragraph), namely the ratio of sparse to full softmax denominators
 * and the residual contribution of the masked-out tokens (core-mechanism
 * paragraph under the Abstract).  The library fixes that description as follows,
 * per batch b, head h, query row t (alpha = 1/sqrt(d), blocks of 64 tokens):
 *
 *   rt_select_blocks        Qb_i, Kb_j = mean of the rows of block i (j); pooled
 *                           logits S_ij = alpha <Qb_i, Kb_j> (float32);
 *                           kept list I_i = forced blocks plus the best
 *                           (keep - n_forced) other blocks by (S_ij descending,
 *                           j ascending), stored ascending.
 *   rt_calibrate            dense attention over all keys that also records
 *                           m = max_j s_j, Z_full = sum_j e^{s_j - m},
 *                           Z_sparse = sum over keys of kept blocks of e^{s_j - m},
 *                           R = sum over keys of masked blocks of e^{s_j - m} v_j,
 *                           and the kept list, into the statistics cache.
 *   rt_sparse_attn_reshape  attention over the kept blocks only (m, Z, N) and
 *                           O = (N e^{m-M} + R_c e^{m_c-M}) / (Z e^{m-M} Z_full_c / Z_sparse_c),
 *                           M = max(m, m_c), with the cached (m_c, Z_full_c,
 *                           Z_sparse_c, R_c) of the same layer.
 *   rt_attention_step       the denoising schedule: select + calibrate on steps
 *                           where step % period == 0 (period <= 0: step 0 only),
 *                           the sparse reshape on all other steps.
 *
 * Conventions for every call.
 *  - Tensors are row-major and contiguous: q, k, v, o are [B, H, N, d_pad]
 *    (bf16 or float32 per rt_shape.dtype); channels d..d_pad-1 of q, k, v must
 *    be zero and are written as zero in o.  Device pointers must be 16-byte
 *    aligned.
 *  - All device work is enqueued asynchronously on `stream` (a hipStream_t;
 *    NULL = the null stream).  The library never allocates or frees device
 *    memory, never synchronises the device, and keeps no device state other
 *    than what the caller's buffers hold.
 *  - The caller owns every device buffer (inputs, outputs, workspace, cache
 *    memory).  The library owns only the small host handle rt_stats_cache.
 *  - Validation happens first: a call that returns an error has enqueued
 *    nothing and touched no device memory.  A failed kernel launch returns
 *    RT_E_LAUNCH.  Faults during execution surface at the caller's next
 *    synchronisation.  rt_last_error() gives a thread-local description of
 *    the last failure.
 *  - Empty problems (B, H or N equal to 0) are valid and enqueue nothing;
 *    their pointers may be NULL.
 *  - Limits: block == 64, d_pad in {64, 80}, 1 <= d <= d_pad,
 *    1 <= keep <= Nb = ceil(N/64), N <= 65536, 0 <= n_forced <= keep.
 *  - Kept lists (block_idx, and the copy in the cache) hold `keep` int32 block
 *    indices per query block.  rt_select_blocks writes every row strictly
 *    ascending.  A caller's row must be non-decreasing; every call reads a
 *    row as the set of its entries (an entry equal to its predecessor adds
 *    nothing), so a row with k distinct blocks keeps exactly those k blocks.
 *    Entries outside [0, Nb) are clamped into range.  A row that is not
 *    non-decreasing is outside this contract: its results are unspecified,
 *    but every memory access stays inside the buffers described here.
 *  - Outputs must not overlap inputs or each other (RT_E_ARG): o must be
 *    disjoint from q, k, v, the list it reads and the cache layer; the
 *    selector's block_idx, pooled_scores and workspace from q, k and from one
 *    another.  The one allowed sharing: rt_calibrate may read its list from
 *    the layer's own list copy (to recalibrate with the cached lists).
 *  - Calls on the same cache layer must not overlap in time from several
 *    host threads; calls on different layers may.
 */
#ifndef RETTN_H
#define RETTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RT_OK = 0,
  RT_E_ARG = 1,        /* null pointer, misaligned pointer, bad enum value */
  RT_E_SHAPE = 2,      /* shape outside the limits above */
  RT_E_DTYPE = 3,      /* dtype not supported for this call */
  RT_E_STATE = 4,      /* layer not calibrated, or cache shape mismatch */
  RT_E_WORKSPACE = 5,  /* workspace or cache memory too small */
  RT_E_LAUNCH = 6,     /* the HIP runtime rejected a kernel launch */
  RT_E_DEVICE = 7      /* no usable gfx950 device for the current HIP device */
} rt_status;

typedef enum { RT_BF16 = 0, RT_F32 = 1 } rt_dtype;

typedef struct {
  int32_t B, H, N;   /* batch, heads, tokens */
  int32_t d;         /* true head dim: softmax scale 1/sqrt(d) */
  int32_t d_pad;     /* stored head dim (row length of q, k, v, o, R) */
  int32_t block;     /* tokens per block; must be 64 */
  int32_t keep;      /* kept key blocks per query block, forced ones included */
  int32_t dtype;     /* rt_dtype of q, k, v, o */
} rt_shape;

/* Opaque host handle over caller-owned device memory. */
typedef struct rt_stats_cache rt_stats_cache;

/* Device pointers of one layer of the statistics cache.
 *   m, z_full, z_sparse : float32 [B, H, N]
 *   R                   : B*H*Nb*64*d_pad elements, float32 by default, bf16
 *                         (reinterpret the pointer) when r_dtype == RT_BF16, in
 *                         the order rt_residual_index gives (not row-major)
 *   idx                 : int32   [B, H, Nb, keep], the kept list used at calibration
 * (Differs from a plain pointer struct in two fields: `rows` = B*H*N gives the
 * extent of the row-wise arrays, and `r_dtype` says how R is stored.)
 * `valid` is 1 once the layer has been calibrated (or marked valid).       */
typedef struct {
  float* m;
  float* z_full;
  float* z_sparse;
  float* R;
  int32_t* idx;
  int64_t rows;      /* B*H*N */
  int32_t valid;
  int32_t r_dtype;   /* rt_dtype of R */
} rt_stats_view;

const char* rt_status_string(int32_t status);
const char* rt_last_error(void);
int32_t rt_version(void);

/* Number of key blocks ceil(N / 64), or -1 for an invalid shape. */
int32_t rt_num_blocks(const rt_shape* shape);

/* ---- block selector (project page, Abstract: attention over a subset of tokens) ----
 * Workspace: the float32 means of k's blocks, B*H*Nb*d_pad*4 bytes (rounded up to
 * 256); rt_select_workspace_bytes gives the size.  The query blocks are pooled
 * inside the selecting kernel.
 * q, k      : device [B,H,N,d_pad].
 * forced    : HOST array of n_forced distinct block indices in [0, Nb), or NULL.
 *             They are always kept and count toward `keep`.
 * block_idx : device int32 [B,H,Nb,keep] output, each row ascending.
 * pooled_scores : device float32 [B,H,Nb,Nb] output of S_ij, or NULL.      */
size_t rt_select_workspace_bytes(const rt_shape* shape);
rt_status rt_select_blocks(const rt_shape* shape, const void* q, const void* k,
                           const int32_t* forced, int32_t n_forced,
                           int32_t* block_idx, float* pooled_scores,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---- the same selector without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation) ----
 * Computes exactly what rt_select_blocks computes (the same kernels), with the
 * K means in scratch memory the library holds: one static device array
 * of RT_SELECT_SCRATCH_BYTES per GPU, from the first call on that GPU until
 * the process ends.  The call allocates and frees nothing.  A shape whose
 * rt_select_workspace_bytes exceeds RT_SELECT_SCRATCH_BYTES returns
 * RT_E_WORKSPACE before touching the device (16 MiB covers B*H*Nb*d_pad up to
 * 4M, e.g. 96 heads of 17776 tokens at d_pad 64).  Every call on one GPU uses
 * that GPU's one array and it keeps the last call's contents: calls that
 * overlap in time on one GPU (several streams or threads) race and give
 * unspecified lists; calls ordered on one stream are safe.  Nothing in the
 * scratch needs to start at zero: each call writes every byte it reads.
 * Other arguments and errors as for rt_select_blocks.                       */
#define RT_SELECT_SCRATCH_BYTES (16u << 20)
rt_status rt_select_blocks_noalloc(const rt_shape* shape, const void* q, const void* k,
                                   const int32_t* forced, int32_t n_forced,
                                   int32_t* block_idx, float* pooled_scores, void* stream);

/* ---- statistics cache (teaser paragraph: statistics cached across denoising steps) ----
 * rt_stats_cache_bytes : device bytes for n_layers layers of `shape`.
 * rt_stats_cache_init  : wraps caller-owned device memory `dev_mem` of `bytes`;
 *                        every layer starts invalid.  *out receives a host handle.
 * rt_stats_cache_view  : device pointers of one layer (for inspection, save and
 *                        restore; the memory is the caller's).
 * rt_stats_cache_set_valid : marks a layer valid (1) or invalid (0), e.g. after
 *                        restoring its contents through the view.
 * rt_stats_cache_invalidate : marks one layer, or all layers (layer = -1), invalid.
 * rt_stats_cache_destroy : frees the host handle only; never touches device memory. */
size_t rt_stats_cache_bytes(const rt_shape* shape, int32_t n_layers);
rt_status rt_stats_cache_init(rt_stats_cache** out, const rt_shape* shape, int32_t n_layers,
                              void* dev_mem, size_t bytes);
/* The same with the residual's storage type chosen: RT_F32 (what the two calls
 * above use) or RT_BF16, which halves the residual's bytes (the largest part of
 * the cache and of a sparse call's traffic) at the cost of rounding R to bf16
 * (relative error <= 2^-9 per element).  RT_BF16 requires shape->dtype ==
 * RT_BF16 (RT_E_DTYPE otherwise); any other value is RT_E_DTYPE (init) or 0
 * bytes.  The calibration kernel rounds the float32 residual to nearest even. */
size_t rt_stats_cache_bytes_ex(const rt_shape* shape, int32_t n_layers, int32_t residual_dtype);
rt_status rt_stats_cache_init_ex(rt_stats_cache** out, const rt_shape* shape, int32_t n_layers,
                                 int32_t residual_dtype, void* dev_mem, size_t bytes);
rt_status rt_stats_cache_view(const rt_stats_cache* cache, int32_t layer, rt_stats_view* out);
/* Position, in elements from rt_stats_view.R, of the residual of head
 * bh = b*H + h, row `row` (< N), column `col` (< d_pad).  R is stored in
 * blocks of 64 rows, the last one padded past N (padding rows hold
 * unspecified finite values, or anything after a restore, and never enter a
 * result).  Inside a block the element of row r and column c sits at
 *   ((r/32 * d_pad/8 + c/8) * 64 + 32 * (c/4 % 2) + r % 32) * 4 + c % 4,
 * the order in which the attention kernels' matrix-core accumulators hold a
 * block, so that they load and store it in contiguous runs.  Returns -1 for
 * an invalid shape or an element out of range (rt_last_error says which). */
int64_t rt_residual_index(const rt_shape* shape, int64_t bh, int32_t row, int32_t col);
rt_status rt_stats_cache_set_valid(rt_stats_cache* cache, int32_t layer, int32_t valid);
rt_status rt_stats_cache_invalidate(rt_stats_cache* cache, int32_t layer);
rt_status rt_stats_cache_destroy(rt_stats_cache* cache);

/* ---- calibration step (core-mechanism paragraph: record the sparse/full denominator
 * ratio and the masked tokens' residual) ----
 * block_idx : device int32 [B,H,Nb,keep] kept lists (from rt_select_blocks); copied
 *             into the cache, so the caller may reuse the buffer afterwards.
 * o         : device [B,H,N,d_pad] output = dense softmax attention.
 * The cache shape must equal `shape`.  Marks `layer` valid.                 */
rt_status rt_calibrate(const rt_shape* shape, const void* q, const void* k, const void* v,
                       const int32_t* block_idx, rt_stats_cache* cache, int32_t layer,
                       void* o, void* stream);

/* ---- sparse step with statistical reshape (teaser and core-mechanism paragraphs) ----
 * block_idx : device kept lists, or NULL to use the lists cached at calibration
 *             (the reading this library takes: the masked set stays that of the
 *             calibration step until the next calibration).
 * Returns RT_E_STATE if `layer` is not valid.                               */
rt_status rt_sparse_attn_reshape(const rt_shape* shape, const void* q, const void* k,
                                 const void* v, const int32_t* block_idx,
                                 const rt_stats_cache* cache, int32_t layer, void* o,
                                 void* stream);

/* ---- sparse step, choice of reshape (core-mechanism paragraph) ----
 * The page fixes the reshape on the calibration step (sparse denominator
 * scaled by the cached full/sparse ratio, cached masked residual added) but
 * leaves open how the residual is weighted at a later step; two readings:
 *   RT_RESHAPE_R1 (what rt_sparse_attn_reshape computes): the residual keeps
 *     its calibration-step magnitude relative to the current running max,
 *     O = (N e^{m-M} + R_c e^{m_c-M}) / (Z e^{m-M} Zf_c / Zs_c);
 *   RT_RESHAPE_R2: the calibration step's split of attention mass is reused,
 *     O = r_c N / Z + R_c / Zf_c with r_c = Zs_c / Zf_c; it is independent of
 *     the cached row max and of any uniform logit offset at the later step.
 * Both equal dense attention on the calibration step's own inputs.  Any other
 * `variant` is RT_E_ARG; otherwise arguments and errors as for
 * rt_sparse_attn_reshape.                                                   */
enum { RT_RESHAPE_R1 = 0, RT_RESHAPE_R2 = 1 };
rt_status rt_sparse_attn_reshape_ex(const rt_shape* shape, const void* q, const void* k,
                                    const void* v, const int32_t* block_idx,
                                    const rt_stats_cache* cache, int32_t layer, int32_t variant,
                                    void* o, void* stream);

/* ---- denoising schedule (teaser paragraph: statistics reused across steps) ----
 * 1 if `step` is a calibration step for `period` (period <= 0: only step 0).   */
int32_t rt_schedule_is_calibration(int32_t step, int32_t period);

/* One attention call of a denoising schedule for one layer: on a calibration
 * step, rt_select_blocks (into the workspace) then rt_calibrate; otherwise
 * rt_sparse_attn_reshape with the cached lists.  Workspace bytes:
 * rt_step_workspace_bytes.  *did_calibrate (may be NULL) receives 1 or 0.   */
size_t rt_step_workspace_bytes(const rt_shape* shape);
rt_status rt_attention_step(const rt_shape* shape, const void* q, const void* k, const void* v,
                            const int32_t* forced, int32_t n_forced, rt_stats_cache* cache,
                            int32_t layer, int32_t step, int32_t period, void* o,
                            void* workspace, size_t workspace_bytes, void* stream,
                            int32_t* did_calibrate);

/* The same schedule with a choice of reshape (`variant`, RT_RESHAPE_R1 or
 * RT_RESHAPE_R2) and `flags`:
 *   RT_STEP_RESELECT: on sparse steps too, run rt_select_blocks on this step's
 *     q and k (into the workspace) and attend to those lists instead of the
 *     cached ones.  The cached statistics still describe the calibration
 *     step's masked set, so where the lists differ the reshape is an
 *     approximation: this library applies the same formula with the new kept
 *     set (the pages state no rule for a changing mask).  The cached lists
 *     are not replaced.
 * Unknown flag bits or variants are RT_E_ARG.  rt_attention_step(...) is
 * rt_attention_step_ex(..., RT_RESHAPE_R1, 0, ...).  The workspace is
 * rt_step_workspace_bytes either way; with RT_STEP_RESELECT it is used on
 * every step.                                                               */
enum { RT_STEP_RESELECT = 1 };
rt_status rt_attention_step_ex(const rt_shape* shape, const void* q, const void* k, const void* v,
                               const int32_t* forced, int32_t n_forced, rt_stats_cache* cache,
                               int32_t layer, int32_t step, int32_t period, int32_t variant,
                               int32_t flags, void* o, void* workspace, size_t workspace_bytes,
                               void* stream, int32_t* did_calibrate);

/* ---- locality-preserving token order (HilbertA blog page, sections
 * "Introducing HilbertA" and "Future Directions": tokens reordered along a 2-D
 * or 3-D Hilbert curve so that grid neighbours stay close in the sequence; the
 * reorder is done once before and once after the denoising loop) ----
 *
 * rt_hilbert_order (host only, no device call): fills perm[0..n) with
 * n = n_text + dims[0]*...*dims[ndims-1].  perm[i] < n_text is i (text tokens
 * first, unchanged); the grid tokens, numbered in raster order after the text
 * with dims[0] the slowest axis ((y, x) or (t, y, x)), follow in the order of
 * their index along the standard Hilbert curve of the smallest 2^k cube that
 * encloses the grid (coordinates in the same axis order).  perm[i] is the
 * original position of the token placed at i.  ndims must be 1..3 and every
 * dims[a] >= 1 (RT_E_ARG); more than 65536 tokens is RT_E_SHAPE.            */
rt_status rt_hilbert_order(const int32_t* dims, int32_t ndims, int32_t n_text, int32_t* perm, int32_t n);

/* rt_permute_rows: reorders the rows of a [B,H,N,d_pad] tensor of shape->dtype.
 * inverse = 0: dst[b,h,i,:] = src[b,h,perm[i],:] (into the new order);
 * inverse = 1: dst[b,h,perm[i],:] = src[b,h,i,:] (back to the original order).
 * perm: device int32 [N], a permutation of 0..N-1 (entries are clamped into
 * range; a list that is not a permutation gives unspecified rows).  src and
 * dst are device buffers that must not overlap (RT_E_ARG), 16-byte aligned.
 * Asynchronous on `stream`.                                                 */
rt_status rt_permute_rows(const rt_shape* shape, const void* src, void* dst, const int32_t* perm,
                          int32_t inverse, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RETTN_H */
