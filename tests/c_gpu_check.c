/* The library driven from plain C on a GPU, with no Python or PyTorch: device
 * memory from the HIP runtime, then rt_select_blocks, rt_calibrate and the
 * sparse step (R1 and R2) on the same inputs, which must reproduce the
 * calibration output (the reshape identity on the calibration step), and a
 * Hilbert reorder and its inverse, which must give the input back bit for
 * bit.  Built by __graft_entry__.build() into tests/_bin/ and run by
 * tests/test_c_abi.py on a GPU.  Prints "ok" and returns 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rettn.h"

#define CHECK(c)                                               \
  do {                                                         \
    if (!(c)) {                                                \
      fprintf(stderr, "failed: %s (line %d) %s\n", #c, __LINE__, rt_last_error()); \
      return 1;                                                \
    }                                                          \
  } while (0)
#define HIPCHECK(x) CHECK((x) == hipSuccess)

static uint16_t to_bf16(float f) { /* nearest even; inputs are finite */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint64_t lcg = 12345;
static float uniform(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((lcg >> 40) & 0xFFFFFF) / 16777216.0f;
}
static float gauss(void) { /* sum of 12 uniforms: mean 0, variance 1 */
  float s = -6.f;
  for (int i = 0; i < 12; ++i) s += uniform();
  return s;
}

static int close_to(const uint16_t* got, const uint16_t* ref, size_t n, const char* what) {
  double dmax = 0, rmax = 0, dsum = 0, rsum = 0;
  for (size_t i = 0; i < n; ++i) {
    const double a = from_bf16(got[i]), b = from_bf16(ref[i]);
    if (!isfinite(a)) {
      fprintf(stderr, "%s: non-finite output at %zu\n", what, i);
      return 0;
    }
    dmax = fmax(dmax, fabs(a - b));
    rmax = fmax(rmax, fabs(b));
    dsum += fabs(a - b);
    rsum += fabs(b);
  }
  if (dmax > 1e-2 * rmax || dsum > 3e-3 * rsum) {
    fprintf(stderr, "%s: max %.3e (ref max %.3e), L1-rel %.3e\n", what, dmax, rmax, dsum / rsum);
    return 0;
  }
  return 1;
}

int main(void) {
  const rt_shape sh = {1, 2, 1000, 64, 64, 64, 4, RT_BF16};
  const int nb = rt_num_blocks(&sh);
  const size_t elems = (size_t)sh.B * sh.H * sh.N * sh.d_pad, bytes = elems * 2;
  const size_t lists = (size_t)sh.B * sh.H * nb * sh.keep;
  uint16_t* h[3];
  for (int t = 0; t < 3; ++t) {
    h[t] = (uint16_t*)malloc(bytes);
    for (size_t i = 0; i < elems; ++i) h[t][i] = to_bf16(gauss());
  }
  void *q, *k, *v, *o_cal, *o_r1, *o_r2, *ws, *cmem, *tmp, *back;
  int32_t *idx, *perm_d;
  HIPCHECK(hipMalloc(&q, bytes));
  HIPCHECK(hipMalloc(&k, bytes));
  HIPCHECK(hipMalloc(&v, bytes));
  HIPCHECK(hipMalloc(&o_cal, bytes));
  HIPCHECK(hipMalloc(&o_r1, bytes));
  HIPCHECK(hipMalloc(&o_r2, bytes));
  HIPCHECK(hipMalloc(&tmp, bytes));
  HIPCHECK(hipMalloc(&back, bytes));
  HIPCHECK(hipMalloc((void**)&idx, lists * 4));
  HIPCHECK(hipMalloc((void**)&perm_d, (size_t)sh.N * 4));
  const size_t wsb = rt_select_workspace_bytes(&sh), cb = rt_stats_cache_bytes(&sh, 1);
  HIPCHECK(hipMalloc(&ws, wsb));
  HIPCHECK(hipMalloc(&cmem, cb));
  HIPCHECK(hipMemcpy(q, h[0], bytes, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(k, h[1], bytes, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(v, h[2], bytes, hipMemcpyHostToDevice));

  const int32_t forced[1] = {0};
  rt_stats_cache* c = NULL;
  CHECK(rt_select_blocks(&sh, q, k, forced, 1, idx, NULL, ws, wsb, NULL) == RT_OK);
  CHECK(rt_stats_cache_init(&c, &sh, 1, cmem, cb) == RT_OK);
  CHECK(rt_calibrate(&sh, q, k, v, idx, c, 0, o_cal, NULL) == RT_OK);
  CHECK(rt_sparse_attn_reshape(&sh, q, k, v, NULL, c, 0, o_r1, NULL) == RT_OK);
  CHECK(rt_sparse_attn_reshape_ex(&sh, q, k, v, NULL, c, 0, RT_RESHAPE_R2, o_r2, NULL) == RT_OK);

  /* Hilbert order of a 40x25 grid (1000 tokens), reorder q and put it back */
  const int32_t dims[2] = {40, 25};
  int32_t* perm = (int32_t*)malloc((size_t)sh.N * 4);
  CHECK(rt_hilbert_order(dims, 2, 0, perm, sh.N) == RT_OK);
  HIPCHECK(hipMemcpy(perm_d, perm, (size_t)sh.N * 4, hipMemcpyHostToDevice));
  CHECK(rt_permute_rows(&sh, q, tmp, perm_d, 0, NULL) == RT_OK);
  CHECK(rt_permute_rows(&sh, tmp, back, perm_d, 1, NULL) == RT_OK);
  HIPCHECK(hipDeviceSynchronize());

  int32_t* hidx = (int32_t*)malloc(lists * 4);
  uint16_t *cal = (uint16_t*)malloc(bytes), *r1 = (uint16_t*)malloc(bytes), *r2 = (uint16_t*)malloc(bytes);
  uint16_t *hb = (uint16_t*)malloc(bytes), *ht = (uint16_t*)malloc(bytes);
  HIPCHECK(hipMemcpy(hidx, idx, lists * 4, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(cal, o_cal, bytes, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(r1, o_r1, bytes, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(r2, o_r2, bytes, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(hb, back, bytes, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(ht, tmp, bytes, hipMemcpyDeviceToHost));

  for (size_t r = 0; r < lists / sh.keep; ++r) { /* lists: ascending, in range, forced block kept */
    const int32_t* l = hidx + r * sh.keep;
    CHECK(l[0] == 0);
    for (int n = 0; n < sh.keep; ++n) CHECK(l[n] >= 0 && l[n] < nb && (n == 0 || l[n] > l[n - 1]));
  }
  CHECK(close_to(r1, cal, elems, "R1 on the calibration inputs"));
  CHECK(close_to(r2, cal, elems, "R2 on the calibration inputs"));
  CHECK(memcmp(hb, h[0], bytes) == 0);
  for (int i = 0; i < sh.N; ++i) /* head 0, row i of the reordered q is row perm[i] of q */
    CHECK(memcmp(ht + (size_t)i * sh.d_pad, h[0] + (size_t)perm[i] * sh.d_pad, (size_t)sh.d_pad * 2) == 0);
  CHECK(rt_stats_cache_destroy(c) == RT_OK);
  printf("ok\n");
  return 0;
}
