// C-ABI host layer: argument validation, statistics-cache layout, schedule,
// and kernel launches on the caller's stream.  No device allocation, no
// device synchronisation (unless RETTN_DEBUG_SYNC=1 is set in the environment).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rettn.h"
#include "internal.h"

using rettn::AttnArgs;
using rettn::AttnMode;
using rettn::SelectArgs;

struct rt_stats_cache {
  rt_shape shape;
  int32_t n_layers;
  char* base;
  size_t bytes;
  size_t off_m, off_zf, off_zs, off_R, off_idx, layer_stride;
  int32_t r_dtype;  // rt_dtype of the residual
  std::vector<int32_t> valid;
};

namespace {

constexpr int32_t kVersion = 1;
constexpr size_t kAlign = 256;

thread_local std::string g_error;

rt_status fail(rt_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t nblocks(int32_t N) { return (N + 63) / 64; }

bool is_empty(const rt_shape* s) { return s->B == 0 || s->H == 0 || s->N == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(const rt_shape* s) { return s->dtype == RT_BF16 ? 2 : 4; }

rt_status check_shape(const rt_shape* s) {
  if (s == nullptr) return fail(RT_E_ARG, "shape is NULL");
  if (s->dtype != RT_BF16 && s->dtype != RT_F32) return fail(RT_E_DTYPE, "dtype %d is not RT_BF16 or RT_F32", s->dtype);
  if (s->B < 0 || s->H < 0 || s->N < 0) return fail(RT_E_SHAPE, "negative B/H/N (%d, %d, %d)", s->B, s->H, s->N);
  if (s->block != 64) return fail(RT_E_SHAPE, "block must be 64 (got %d)", s->block);
  if (s->d_pad != 64 && s->d_pad != 80) return fail(RT_E_SHAPE, "d_pad must be 64 or 80 (got %d)", s->d_pad);
  if (s->d < 1 || s->d > s->d_pad) return fail(RT_E_SHAPE, "need 1 <= d <= d_pad (d=%d, d_pad=%d)", s->d, s->d_pad);
  if (s->N > 65536) return fail(RT_E_SHAPE, "N=%d exceeds 65536", s->N);
  if (is_empty(s)) return RT_OK;
  const int64_t nb = nblocks(s->N);
  if (s->keep < 1 || s->keep > nb) return fail(RT_E_SHAPE, "need 1 <= keep <= Nb (keep=%d, Nb=%lld)", s->keep, (long long)nb);
  if ((int64_t)s->B * s->H * nb > 0x7fffffffLL / 8) return fail(RT_E_SHAPE, "B*H*Nb too large");
  return RT_OK;
}

bool same_shape(const rt_shape& a, const rt_shape& b) {
  return a.B == b.B && a.H == b.H && a.N == b.N && a.d == b.d && a.d_pad == b.d_pad && a.block == b.block &&
         a.keep == b.keep && a.dtype == b.dtype;
}

// Current device must be a gfx950; answered once per device.
rt_status check_device() {
  static std::mutex mu;
  static std::vector<int> known;  // -1 unknown, 0 bad, 1 good
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RT_E_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if ((int)known.size() <= dev) known.resize(dev + 1, -1);
  if (known[dev] < 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(RT_E_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    known[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    if (!known[dev]) return fail(RT_E_DEVICE, "device %d is %s, this library is built for gfx950", dev, p.gcnArchName);
  }
  return known[dev] ? RT_OK : fail(RT_E_DEVICE, "device %d is not a gfx950", dev);
}

bool debug_sync() {
  static int v = [] {
    const char* e = std::getenv("RETTN_DEBUG_SYNC");
    return e != nullptr && e[0] == '1';
  }();
  return v != 0;
}

rt_status launched(hipError_t e, hipStream_t s, const char* what) {
  if (e != hipSuccess) return fail(RT_E_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(RT_E_LAUNCH, "%s failed at sync: %s", what, hipGetErrorString(e));
  }
  return RT_OK;
}

void layout(rt_stats_cache* c) {
  const rt_shape& s = c->shape;
  const size_t rows = (size_t)s.B * s.H * s.N;
  const size_t lists = (size_t)s.B * s.H * nblocks(s.N) * s.keep;
  size_t off = 0;
  c->off_m = off; off += align_up(rows * 4);
  c->off_zf = off; off += align_up(rows * 4);
  c->off_zs = off; off += align_up(rows * 4);
  // R is padded to whole 64-row blocks (rettn::residual_index)
  const size_t r_elems = (size_t)s.B * s.H * nblocks(s.N) * rettn::kBlock * s.d_pad;
  c->off_R = off; off += align_up(r_elems * (c->r_dtype == RT_BF16 ? 2 : 4));
  c->off_idx = off; off += align_up(lists * 4);
  c->layer_stride = off;
}

AttnArgs attn_args(const rt_shape* s, const void* q, const void* k, const void* v, void* o, const int32_t* idx,
                   const rt_stats_cache* c, int32_t layer) {
  AttnArgs a{};
  char* base = c->base + (size_t)layer * c->layer_stride;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.idx = idx;
  a.idx_cache = (int32_t*)(base + c->off_idx);
  a.m = (float*)(base + c->off_m);
  a.z_full = (float*)(base + c->off_zf);
  a.z_sparse = (float*)(base + c->off_zs);
  a.R = (float*)(base + c->off_R);
  a.r_bf16 = c->r_dtype == RT_BF16 ? 1 : 0;
  a.BH = s->B * s->H;
  a.N = s->N;
  a.Nb = (int32_t)nblocks(s->N);
  a.keep = s->keep;
  a.alpha = (float)(1.0 / std::sqrt((double)s->d));
  return a;
}

rt_status check_tensors(const void* const* ptrs, const char* const* names, int n) {
  for (int i = 0; i < n; ++i) {
    if (ptrs[i] == nullptr) return fail(RT_E_ARG, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(RT_E_ARG, "%s is not 16-byte aligned", names[i]);
  }
  return RT_OK;
}

// A device byte range [p, p + bytes).
struct Span {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Span& a, const Span& b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
  return x < y + b.bytes && y < x + a.bytes;
}

// Every output span must be disjoint from every input span and from the other
// outputs (the kernels read inputs while other workgroups write outputs).
rt_status check_disjoint(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return fail(RT_E_ARG, "%s overlaps %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return fail(RT_E_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  return RT_OK;
}

size_t tensor_bytes(const rt_shape* s) { return (size_t)s->B * s->H * s->N * s->d_pad * elem_bytes(s); }

size_t list_bytes(const rt_shape* s) { return (size_t)s->B * s->H * nblocks(s->N) * s->keep * 4; }

rt_status check_cache(const rt_shape* s, const rt_stats_cache* c, int32_t layer) {
  if (c == nullptr) return fail(RT_E_ARG, "cache is NULL");
  if (layer < 0 || layer >= c->n_layers) return fail(RT_E_ARG, "layer %d out of range [0, %d)", layer, c->n_layers);
  if (!same_shape(*s, c->shape)) return fail(RT_E_STATE, "cache was initialised for a different shape");
  return RT_OK;
}

// The selector's workspace: the float32 means of K, [B*H, d_pad, Nb].
size_t select_ws(const rt_shape* s) { return align_up((size_t)s->B * s->H * nblocks(s->N) * s->d_pad * 4); }

}  // namespace

extern "C" {

const char* rt_status_string(int32_t st) {
  switch (st) {
    case RT_OK: return "RT_OK";
    case RT_E_ARG: return "RT_E_ARG: invalid argument";
    case RT_E_SHAPE: return "RT_E_SHAPE: shape outside the supported limits";
    case RT_E_DTYPE: return "RT_E_DTYPE: unsupported dtype";
    case RT_E_STATE: return "RT_E_STATE: cache layer not calibrated or shape mismatch";
    case RT_E_WORKSPACE: return "RT_E_WORKSPACE: workspace or cache memory too small";
    case RT_E_LAUNCH: return "RT_E_LAUNCH: kernel launch failed";
    case RT_E_DEVICE: return "RT_E_DEVICE: no usable gfx950 device";
    default: return "unknown rt_status";
  }
}

const char* rt_last_error(void) { return g_error.c_str(); }

int32_t rt_version(void) { return kVersion; }

int32_t rt_num_blocks(const rt_shape* s) {
  if (s == nullptr || s->N < 0) return -1;
  return (int32_t)nblocks(s->N);
}

size_t rt_select_workspace_bytes(const rt_shape* s) {
  if (check_shape(s) != RT_OK) return 0;
  return select_ws(s);
}

rt_status rt_select_blocks(const rt_shape* s, const void* q, const void* k, const int32_t* forced,
                           int32_t n_forced, int32_t* block_idx, float* pooled_scores, void* workspace,
                           size_t ws_bytes, void* stream) {
  rt_status st = check_shape(s);
  if (st != RT_OK) return st;
  if (is_empty(s)) return RT_OK;
  const void* ptrs[] = {q, k, block_idx, workspace};
  const char* names[] = {"q", "k", "block_idx", "workspace"};
  if ((st = check_tensors(ptrs, names, 4)) != RT_OK) return st;
  if (pooled_scores != nullptr && (reinterpret_cast<uintptr_t>(pooled_scores) & 3u))
    return fail(RT_E_ARG, "pooled_scores is not 4-byte aligned");
  if (ws_bytes < select_ws(s)) return fail(RT_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, select_ws(s));
  const int32_t nb = (int32_t)nblocks(s->N);
  {
    const Span ins[] = {{q, tensor_bytes(s), "q"}, {k, tensor_bytes(s), "k"}};
    const Span outs[] = {{block_idx, list_bytes(s), "block_idx"},
                         {pooled_scores, (size_t)s->B * s->H * nb * nb * 4, "pooled_scores"},
                         {workspace, select_ws(s), "workspace"}};
    if ((st = check_disjoint(outs, 3, ins, 2)) != RT_OK) return st;
  }
  if (n_forced < 0 || n_forced > s->keep) return fail(RT_E_ARG, "need 0 <= n_forced <= keep (n_forced=%d)", n_forced);
  if (n_forced > 0 && forced == nullptr) return fail(RT_E_ARG, "forced is NULL with n_forced=%d", n_forced);
  SelectArgs a{};
  for (int32_t i = 0; i < n_forced; ++i) {
    const int32_t j = forced[i];
    if (j < 0 || j >= nb) return fail(RT_E_ARG, "forced[%d]=%d outside [0, %d)", i, j, nb);
    if ((a.forced[j >> 5] >> (j & 31)) & 1u) return fail(RT_E_ARG, "forced block %d listed twice", j);
    a.forced[j >> 5] |= 1u << (j & 31);
  }
  if ((st = check_device()) != RT_OK) return st;
  a.q = q;
  a.k = k;
  a.kb = (float*)workspace;
  a.idx = block_idx;
  a.scores = pooled_scores;
  a.BH = s->B * s->H;
  a.N = s->N;
  a.Nb = nb;
  a.keep = s->keep;
  a.alpha = (float)(1.0 / std::sqrt((double)s->d));
  hipStream_t hs = (hipStream_t)stream;
  return launched(rettn::launch_select(s->dtype == RT_BF16, s->d_pad, a, hs), hs, "rt_select_blocks");
}

rt_status rt_select_blocks_noalloc(const rt_shape* s, const void* q, const void* k, const int32_t* forced,
                                   int32_t n_forced, int32_t* block_idx, float* pooled_scores, void* stream) {
  static_assert(rettn::kSelectScratchBytes == (size_t)RT_SELECT_SCRATCH_BYTES, "scratch size");
  rt_status st = check_shape(s);
  if (st != RT_OK) return st;
  if (is_empty(s)) return RT_OK;
  if (select_ws(s) > rettn::kSelectScratchBytes)
    return fail(RT_E_WORKSPACE,
                "the selector needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                "(use rt_select_blocks with a workspace)",
                select_ws(s), rettn::kSelectScratchBytes);
  if ((st = check_device()) != RT_OK) return st;
  void* scratch = nullptr;
  const hipError_t e = rettn::select_scratch(&scratch);
  if (e != hipSuccess) return fail(RT_E_DEVICE, "selector scratch: %s", hipGetErrorString(e));
  return rt_select_blocks(s, q, k, forced, n_forced, block_idx, pooled_scores, scratch, rettn::kSelectScratchBytes,
                          stream);
}

size_t rt_stats_cache_bytes_ex(const rt_shape* s, int32_t n_layers, int32_t residual_dtype) {
  if (check_shape(s) != RT_OK || n_layers < 1) return 0;
  if (residual_dtype != RT_F32 && !(residual_dtype == RT_BF16 && s->dtype == RT_BF16)) return 0;
  rt_stats_cache c{};
  c.shape = *s;
  c.r_dtype = residual_dtype;
  layout(&c);
  return c.layer_stride * (size_t)n_layers;
}

int64_t rt_residual_index(const rt_shape* s, int64_t bh, int32_t row, int32_t col) {
  if (s == nullptr || check_shape(s) != RT_OK) return -1;
  if (bh < 0 || bh >= (int64_t)s->B * s->H || row < 0 || row >= s->N || col < 0 || col >= s->d_pad) {
    fail(RT_E_ARG, "residual element (bh=%lld, row=%d, col=%d) out of range", (long long)bh, row, col);
    return -1;
  }
  return (int64_t)rettn::residual_index((size_t)bh, (int)nblocks(s->N), s->d_pad, row, col);
}

size_t rt_stats_cache_bytes(const rt_shape* s, int32_t n_layers) {
  return rt_stats_cache_bytes_ex(s, n_layers, RT_F32);
}

rt_status rt_stats_cache_init(rt_stats_cache** out, const rt_shape* s, int32_t n_layers, void* dev_mem,
                              size_t bytes) {
  return rt_stats_cache_init_ex(out, s, n_layers, RT_F32, dev_mem, bytes);
}

rt_status rt_stats_cache_init_ex(rt_stats_cache** out, const rt_shape* s, int32_t n_layers, int32_t residual_dtype,
                                 void* dev_mem, size_t bytes) {
  if (out == nullptr) return fail(RT_E_ARG, "out is NULL");
  *out = nullptr;
  rt_status st = check_shape(s);
  if (st != RT_OK) return st;
  if (n_layers < 1) return fail(RT_E_ARG, "n_layers must be >= 1 (got %d)", n_layers);
  if (residual_dtype != RT_F32 && residual_dtype != RT_BF16)
    return fail(RT_E_DTYPE, "residual dtype %d is not RT_F32 or RT_BF16", residual_dtype);
  if (residual_dtype == RT_BF16 && s->dtype != RT_BF16)
    return fail(RT_E_DTYPE, "a bf16 residual needs bf16 q/k/v (shape dtype %d)", s->dtype);
  const size_t need = rt_stats_cache_bytes_ex(s, n_layers, residual_dtype);
  if (need > 0 && dev_mem == nullptr && !is_empty(s)) return fail(RT_E_ARG, "dev_mem is NULL");
  if (dev_mem != nullptr && (reinterpret_cast<uintptr_t>(dev_mem) % kAlign) != 0)
    return fail(RT_E_ARG, "dev_mem must be %zu-byte aligned", kAlign);
  if (bytes < need) return fail(RT_E_WORKSPACE, "cache memory %zu < %zu bytes", bytes, need);
  rt_stats_cache* c = new (std::nothrow) rt_stats_cache();
  if (c == nullptr) return fail(RT_E_ARG, "host allocation failed");
  c->shape = *s;
  c->r_dtype = residual_dtype;
  c->n_layers = n_layers;
  c->base = (char*)dev_mem;
  c->bytes = bytes;
  layout(c);
  c->valid.assign(n_layers, 0);
  *out = c;
  return RT_OK;
}

rt_status rt_stats_cache_view(const rt_stats_cache* c, int32_t layer, rt_stats_view* out) {
  if (c == nullptr || out == nullptr) return fail(RT_E_ARG, "cache or out is NULL");
  if (layer < 0 || layer >= c->n_layers) return fail(RT_E_ARG, "layer %d out of range [0, %d)", layer, c->n_layers);
  char* base = c->base + (size_t)layer * c->layer_stride;
  out->m = (float*)(base + c->off_m);
  out->z_full = (float*)(base + c->off_zf);
  out->z_sparse = (float*)(base + c->off_zs);
  out->R = (float*)(base + c->off_R);
  out->idx = (int32_t*)(base + c->off_idx);
  out->rows = (int64_t)c->shape.B * c->shape.H * c->shape.N;
  out->valid = c->valid[layer];
  out->r_dtype = c->r_dtype;
  return RT_OK;
}

rt_status rt_stats_cache_set_valid(rt_stats_cache* c, int32_t layer, int32_t valid) {
  if (c == nullptr) return fail(RT_E_ARG, "cache is NULL");
  if (layer < 0 || layer >= c->n_layers) return fail(RT_E_ARG, "layer %d out of range [0, %d)", layer, c->n_layers);
  c->valid[layer] = valid ? 1 : 0;
  return RT_OK;
}

rt_status rt_stats_cache_invalidate(rt_stats_cache* c, int32_t layer) {
  if (c == nullptr) return fail(RT_E_ARG, "cache is NULL");
  if (layer == -1) {
    for (auto& v : c->valid) v = 0;
    return RT_OK;
  }
  if (layer < 0 || layer >= c->n_layers) return fail(RT_E_ARG, "layer %d out of range [0, %d)", layer, c->n_layers);
  c->valid[layer] = 0;
  return RT_OK;
}

rt_status rt_stats_cache_destroy(rt_stats_cache* c) {
  delete c;
  return RT_OK;
}

rt_status rt_calibrate(const rt_shape* s, const void* q, const void* k, const void* v, const int32_t* block_idx,
                       rt_stats_cache* c, int32_t layer, void* o, void* stream) {
  rt_status st = check_shape(s);
  if (st != RT_OK) return st;
  if ((st = check_cache(s, c, layer)) != RT_OK) return st;
  if (is_empty(s)) {
    c->valid[layer] = 1;
    return RT_OK;
  }
  const void* ptrs[] = {q, k, v, block_idx, o};
  const char* names[] = {"q", "k", "v", "block_idx", "o"};
  if ((st = check_tensors(ptrs, names, 5)) != RT_OK) return st;
  {
    const Span ins[] = {{q, tensor_bytes(s), "q"}, {k, tensor_bytes(s), "k"}, {v, tensor_bytes(s), "v"}};
    const Span outs[] = {{o, tensor_bytes(s), "o"},
                         {c->base + (size_t)layer * c->layer_stride, c->layer_stride, "the cache layer"}};
    if ((st = check_disjoint(outs, 2, ins, 3)) != RT_OK) return st;
    const Span lst[] = {{block_idx, list_bytes(s), "block_idx"}};
    if ((st = check_disjoint(outs, 1, lst, 1)) != RT_OK) return st;  // o vs the list it reads
    // The list may be the layer's own list copy (each workgroup reads its
    // entries before writing the same values back), or lie outside the layer.
    char* layer_base = c->base + (size_t)layer * c->layer_stride;
    if ((const void*)block_idx != (const void*)(layer_base + c->off_idx)) {
      const Span lay[] = {{layer_base, c->layer_stride, "the cache layer"}};
      if ((st = check_disjoint(lst, 1, lay, 1)) != RT_OK) return st;
    }
  }
  if ((st = check_device()) != RT_OK) return st;
  AttnArgs a = attn_args(s, q, k, v, o, block_idx, c, layer);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = s->dtype == RT_BF16 ? rettn::launch_attn_bf16(AttnMode::kCalibrate, s->d_pad, a, hs)
                                     : rettn::launch_attn_f32(AttnMode::kCalibrate, s->d_pad, a, hs);
  if ((st = launched(e, hs, "rt_calibrate")) != RT_OK) return st;
  c->valid[layer] = 1;
  return RT_OK;
}

rt_status rt_sparse_attn_reshape(const rt_shape* s, const void* q, const void* k, const void* v,
                                 const int32_t* block_idx, const rt_stats_cache* c, int32_t layer, void* o,
                                 void* stream) {
  return rt_sparse_attn_reshape_ex(s, q, k, v, block_idx, c, layer, RT_RESHAPE_R1, o, stream);
}

rt_status rt_sparse_attn_reshape_ex(const rt_shape* s, const void* q, const void* k, const void* v,
                                    const int32_t* block_idx, const rt_stats_cache* c, int32_t layer,
                                    int32_t variant, void* o, void* stream) {
  if (variant != RT_RESHAPE_R1 && variant != RT_RESHAPE_R2)
    return fail(RT_E_ARG, "reshape variant must be RT_RESHAPE_R1 or RT_RESHAPE_R2 (got %d)", variant);
  rt_status st = check_shape(s);
  if (st != RT_OK) return st;
  if ((st = check_cache(s, c, layer)) != RT_OK) return st;
  if (!c->valid[layer]) return fail(RT_E_STATE, "layer %d has no valid statistics (calibrate first)", layer);
  if (is_empty(s)) return RT_OK;
  const void* ptrs[] = {q, k, v, o};
  const char* names[] = {"q", "k", "v", "o"};
  if ((st = check_tensors(ptrs, names, 4)) != RT_OK) return st;
  if (block_idx != nullptr && !aligned16(block_idx)) return fail(RT_E_ARG, "block_idx is not 16-byte aligned");
  {
    const Span ins[] = {{q, tensor_bytes(s), "q"},
                        {k, tensor_bytes(s), "k"},
                        {v, tensor_bytes(s), "v"},
                        {block_idx, list_bytes(s), "block_idx"},
                        {c->base + (size_t)layer * c->layer_stride, c->layer_stride, "the cache layer"}};
    const Span outs[] = {{o, tensor_bytes(s), "o"}};
    if ((st = check_disjoint(outs, 1, ins, 5)) != RT_OK) return st;
  }
  if ((st = check_device()) != RT_OK) return st;
  AttnArgs a = attn_args(s, q, k, v, o, nullptr, c, layer);
  a.idx = block_idx != nullptr ? block_idx : a.idx_cache;
  a.idx_cache = nullptr;
  a.variant = variant;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = s->dtype == RT_BF16 ? rettn::launch_attn_bf16(AttnMode::kSparse, s->d_pad, a, hs)
                                     : rettn::launch_attn_f32(AttnMode::kSparse, s->d_pad, a, hs);
  return launched(e, hs, "rt_sparse_attn_reshape");
}

int32_t rt_schedule_is_calibration(int32_t step, int32_t period) {
  if (step < 0) return 0;
  if (period <= 0) return step == 0 ? 1 : 0;
  return step % period == 0 ? 1 : 0;
}

size_t rt_step_workspace_bytes(const rt_shape* s) {
  if (check_shape(s) != RT_OK) return 0;
  const size_t lists = (size_t)s->B * s->H * nblocks(s->N) * s->keep * 4;
  return select_ws(s) + align_up(lists);
}

rt_status rt_attention_step(const rt_shape* s, const void* q, const void* k, const void* v, const int32_t* forced,
                            int32_t n_forced, rt_stats_cache* c, int32_t layer, int32_t step, int32_t period,
                            void* o, void* workspace, size_t ws_bytes, void* stream, int32_t* did_calibrate) {
  return rt_attention_step_ex(s, q, k, v, forced, n_forced, c, layer, step, period, RT_RESHAPE_R1, 0, o, workspace,
                              ws_bytes, stream, did_calibrate);
}

rt_status rt_attention_step_ex(const rt_shape* s, const void* q, const void* k, const void* v,
                               const int32_t* forced, int32_t n_forced, rt_stats_cache* c, int32_t layer,
                               int32_t step, int32_t period, int32_t variant, int32_t flags, void* o,
                               void* workspace, size_t ws_bytes, void* stream, int32_t* did_calibrate) {
  if (did_calibrate != nullptr) *did_calibrate = 0;
  rt_status st = check_shape(s);
  if (st != RT_OK) return st;
  if ((st = check_cache(s, c, layer)) != RT_OK) return st;
  if (step < 0) return fail(RT_E_ARG, "step must be >= 0 (got %d)", step);
  if (variant != RT_RESHAPE_R1 && variant != RT_RESHAPE_R2)
    return fail(RT_E_ARG, "reshape variant must be RT_RESHAPE_R1 or RT_RESHAPE_R2 (got %d)", variant);
  if ((flags & ~RT_STEP_RESELECT) != 0) return fail(RT_E_ARG, "unknown step flags 0x%x", (unsigned)flags);
  const bool calib = rt_schedule_is_calibration(step, period) != 0;
  const bool reselect = (flags & RT_STEP_RESELECT) != 0;
  if (!calib && !c->valid[layer]) return fail(RT_E_STATE, "layer %d has no valid statistics (calibrate first)", layer);
  if (did_calibrate != nullptr) *did_calibrate = calib ? 1 : 0;
  if (!calib && !reselect) return rt_sparse_attn_reshape_ex(s, q, k, v, nullptr, c, layer, variant, o, stream);
  if (is_empty(s)) {
    return calib ? rt_calibrate(s, q, k, v, nullptr, c, layer, o, stream)
                 : rt_sparse_attn_reshape_ex(s, q, k, v, nullptr, c, layer, variant, o, stream);
  }
  if (workspace == nullptr) return fail(RT_E_ARG, "workspace is NULL");
  if (ws_bytes < rt_step_workspace_bytes(s))
    return fail(RT_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, rt_step_workspace_bytes(s));
  int32_t* lists = (int32_t*)((char*)workspace + select_ws(s));
  st = rt_select_blocks(s, q, k, forced, n_forced, lists, nullptr, workspace, select_ws(s), stream);
  if (st != RT_OK) return st;
  if (calib) return rt_calibrate(s, q, k, v, lists, c, layer, o, stream);
  return rt_sparse_attn_reshape_ex(s, q, k, v, lists, c, layer, variant, o, stream);
}

rt_status rt_hilbert_order(const int32_t* dims, int32_t ndims, int32_t n_text, int32_t* perm, int32_t n) {
  if (dims == nullptr || perm == nullptr) return fail(RT_E_ARG, "dims or perm is NULL");
  if (ndims < 1 || ndims > 3) return fail(RT_E_ARG, "ndims must be 1, 2 or 3 (got %d)", ndims);
  if (n_text < 0) return fail(RT_E_ARG, "n_text must be >= 0 (got %d)", n_text);
  int64_t count = 1;
  for (int32_t a = 0; a < ndims; ++a) {
    if (dims[a] < 1) return fail(RT_E_ARG, "dims[%d]=%d must be >= 1", a, dims[a]);
    count *= dims[a];
    if (count > 65536) return fail(RT_E_SHAPE, "grid of more than 65536 tokens");
  }
  if ((int64_t)n != (int64_t)n_text + count)
    return fail(RT_E_ARG, "n=%d but n_text + prod(dims) = %lld", n, (long long)(n_text + count));
  if (n > 65536) return fail(RT_E_SHAPE, "N=%d exceeds 65536", n);
  rettn::hilbert_order(dims, ndims, n_text, perm);
  return RT_OK;
}

rt_status rt_permute_rows(const rt_shape* s, const void* src, void* dst, const int32_t* perm, int32_t inverse,
                          void* stream) {
  rt_status st = check_shape(s);
  if (st != RT_OK) return st;
  if (inverse != 0 && inverse != 1) return fail(RT_E_ARG, "inverse must be 0 or 1 (got %d)", inverse);
  if (is_empty(s)) return RT_OK;
  const void* ptrs[] = {src, dst};
  const char* names[] = {"src", "dst"};
  if ((st = check_tensors(ptrs, names, 2)) != RT_OK) return st;
  if (perm == nullptr || (reinterpret_cast<uintptr_t>(perm) & 3u)) return fail(RT_E_ARG, "perm is NULL or misaligned");
  const size_t esize = s->dtype == RT_BF16 ? 2 : 4;
  const size_t bytes = (size_t)s->B * s->H * s->N * s->d_pad * esize;
  const char* a0 = (const char*)src;
  const char* b0 = (const char*)dst;
  if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(RT_E_ARG, "src and dst overlap (the reorder is not in place)");
  if ((st = check_device()) != RT_OK) return st;
  rettn::PermuteArgs a{};
  a.src = src;
  a.dst = dst;
  a.perm = perm;
  a.BH = s->B * s->H;
  a.N = s->N;
  a.cpr = (int32_t)(s->d_pad * esize / 16);
  a.inverse = inverse;
  hipStream_t hs = (hipStream_t)stream;
  return launched(rettn::launch_permute(a, hs), hs, "rt_permute_rows");
}

}  // extern "C"
