/* A plain C consumer of the library's C ABI (compiled with gcc by
 * tests/test_c_abi.py): the header must be valid C and every host-only entry
 * point callable without a device.  Prints "ok" and returns 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rettn.h"

#define CHECK(c)                                               \
  do {                                                         \
    if (!(c)) {                                                \
      fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                \
    }                                                          \
  } while (0)

int main(void) {
  rt_shape sh = {2, 30, 17776, 64, 64, 64, 9, RT_BF16};
  CHECK(rt_version() > 0);
  CHECK(rt_num_blocks(&sh) == 278);
  CHECK(strncmp(rt_status_string(RT_E_SHAPE), "RT_E_SHAPE", 10) == 0);
  CHECK(rt_schedule_is_calibration(0, 0) == 1 && rt_schedule_is_calibration(10, 10) == 1 &&
        rt_schedule_is_calibration(11, 10) == 0);
  /* cache sizes: m, z_full, z_sparse, R float32, lists int32 (each section 256-byte aligned) */
  const size_t rows = (size_t)2 * 30 * 17776;
  const size_t b = rt_stats_cache_bytes(&sh, 1);
  CHECK(b >= rows * 4 * 3 + rows * 64 * 4 + (size_t)2 * 30 * 278 * 9 * 4);
  CHECK(rt_stats_cache_bytes_ex(&sh, 1, RT_BF16) < b);
  CHECK(rt_select_workspace_bytes(&sh) > 0 && rt_step_workspace_bytes(&sh) > rt_select_workspace_bytes(&sh));

  /* a cache handle over fake device memory: host bookkeeping only */
  rt_stats_cache* c = NULL;
  void* mem = (void*)(uintptr_t)0x100000;
  CHECK(rt_stats_cache_init(&c, &sh, 3, mem, b * 3) == RT_OK && c != NULL);
  rt_stats_view v;
  CHECK(rt_stats_cache_view(c, 2, &v) == RT_OK && v.valid == 0 && v.rows == (int64_t)rows && v.r_dtype == RT_F32);
  CHECK(rt_stats_cache_set_valid(c, 2, 1) == RT_OK);
  CHECK(rt_stats_cache_view(c, 2, &v) == RT_OK && v.valid == 1);
  CHECK(rt_stats_cache_view(c, 3, &v) == RT_E_ARG);
  CHECK(rt_stats_cache_invalidate(c, -1) == RT_OK);
  CHECK(rt_stats_cache_view(c, 2, &v) == RT_OK && v.valid == 0);
  /* sparse before calibration is rejected before any device call */
  CHECK(rt_sparse_attn_reshape(&sh, mem, mem, mem, NULL, c, 0, mem, NULL) == RT_E_STATE);
  CHECK(rt_sparse_attn_reshape_ex(&sh, mem, mem, mem, NULL, c, 0, 5, mem, NULL) == RT_E_ARG);
  CHECK(strlen(rt_last_error()) > 0);
  CHECK(rt_stats_cache_destroy(c) == RT_OK);

  /* residual layout: row 33 is in the second 32-row half of block 0, column 9
     in the second 8-column group, first 4-column half: ((1*8 + 1)*64 + 1)*4 + 1;
     row 17775 is row 47 of block 277 of head 59 */
  CHECK(rt_residual_index(&sh, 0, 33, 9) == 2309);
  CHECK(rt_residual_index(&sh, 59, 17775, 63) ==
        ((int64_t)59 * 278 + 277) * 64 * 64 + ((1 * 8 + 7) * 64 + 32 + 15) * 4 + 3);
  CHECK(rt_residual_index(&sh, 60, 0, 0) == -1 && rt_residual_index(&sh, 0, 17776, 0) == -1);

  /* shape validation */
  rt_shape bad = sh;
  bad.block = 32;
  CHECK(rt_num_blocks(&bad) == 278 && rt_select_workspace_bytes(&bad) == 0);

  /* Hilbert order: a 4x4 grid after 3 text tokens */
  const int32_t dims[2] = {4, 4};
  int32_t perm[19];
  CHECK(rt_hilbert_order(dims, 2, 3, perm, 19) == RT_OK);
  CHECK(perm[0] == 0 && perm[1] == 1 && perm[2] == 2 && perm[3] == 3);
  int seen[19] = {0};
  for (int i = 0; i < 19; ++i) {
    CHECK(perm[i] >= 0 && perm[i] < 19 && !seen[perm[i]]);
    seen[perm[i]] = 1;
  }
  for (int i = 4; i < 18; ++i) {  /* consecutive grid tokens are grid neighbours */
    const int a = perm[i] - 3, c2 = perm[i + 1] - 3;
    CHECK(abs(a / 4 - c2 / 4) + abs(a % 4 - c2 % 4) == 1);
  }
  CHECK(rt_hilbert_order(dims, 2, 3, perm, 18) == RT_E_ARG);
  printf("ok\n");
  return 0;
}
