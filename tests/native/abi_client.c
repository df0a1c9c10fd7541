/*
 * A plain C client of include/armx.h, linked against libarmx.so: what a user
 * without Python sees.  Built by tests/test_abi_client.py.
 *
 *   abi_client cpu   argument checks and workspace sizes (no device needed)
 *   abi_client gpu   sums of n = 2^24 - 5 ones on the device: reduce_sum,
 *                    reduce_sum_exact and reduce_sum_fixed_order must all
 *                    give exactly n (every partial sum is an integer below
 *                    2^24, exactly representable, so no order rounds)
 * Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "armx.h"

/* The few HIP runtime entry points the gpu mode needs, declared here so the
 * client builds with a plain C compiler (hip_runtime_api.h is C++). */
typedef int hipError_t;
extern hipError_t hipMalloc(void** ptr, size_t size);
extern hipError_t hipFree(void* ptr);
extern hipError_t hipMemcpy(void* dst, const void* src, size_t size, int kind);
extern hipError_t hipMemset(void* dst, int value, size_t size);
extern hipError_t hipDeviceSynchronize(void);
enum { kHostToDevice = 1, kDeviceToHost = 2 };

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
              __LINE__, #cond);                                        \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static int cpu_checks(void) {
  char* fake = (char*)(uintptr_t)(1u << 20); /* never dereferenced */
  armx_config bad = {96, 0, 0, 0, NULL, NULL};
  EXPECT(armx_version() == 8);
  {
    armx_plan_info info;
    EXPECT(armx_launch_plan(ARMX_OP_FIXED, (size_t)1 << 26, 0, NULL, &info) == ARMX_OK);
    EXPECT(info.grid_blocks > 0 && info.block_threads == 128 && info.chain_r == 8);
    EXPECT(info.launches == 1 && info.workspace_bytes ==
                                     armx_workspace_bytes(ARMX_OP_FIXED, (size_t)1 << 26, 0, NULL));
    EXPECT(armx_launch_plan(ARMX_OP_SUM, 10, 0, &bad, &info) == ARMX_ERR_CONFIG);
  }
  EXPECT(reduce_sum(NULL, 10, (float*)fake, fake, 1 << 20, NULL, NULL) == ARMX_ERR_NULL);
  EXPECT(reduce_sum(fake + 2, 10, (float*)fake, fake, 1 << 20, NULL, NULL) == ARMX_ERR_ALIGN);
  EXPECT(reduce_sum(fake, 10, (float*)fake, fake, 1 << 20, &bad, NULL) == ARMX_ERR_CONFIG);
  EXPECT(reduce_sum_exact(fake, 10, (float*)fake, (int64_t*)(fake + 4), fake, 1 << 20, NULL,
                          NULL) == ARMX_ERR_ALIGN);
  EXPECT(reduce_rows(fake, 4, 100, 96, (float*)fake, NULL, 0, NULL, NULL) == ARMX_ERR_SHAPE);
  EXPECT(reduce_rows_fixed_order(fake, 4, 100, 100, (float*)fake, NULL, 0, NULL, NULL) ==
         ARMX_ERR_ALIGN);
  EXPECT(armx_workspace_bytes(ARMX_OP_ROWS, 4096, 65536, NULL) == 0);
  EXPECT(armx_workspace_bytes(ARMX_OP_SUM, 0, 0, NULL) == 0);
  EXPECT(armx_workspace_bytes(99, 10, 0, NULL) == (size_t)-1);
  EXPECT(armx_status_string(ARMX_ERR_WORKSPACE)[5] == 'E');
  return failures;
}

static int gpu_checks(void) {
  const size_t n = ((size_t)1 << 24) - 5;
  uint16_t* host = (uint16_t*)malloc(n * sizeof(uint16_t));
  void *x = NULL, *ws = NULL;
  float *out = NULL, got[3];
  int64_t *fixed = NULL, q[2];
  size_t ws_bytes = 0;
  const int ops[3] = {ARMX_OP_SUM, ARMX_OP_EXACT, ARMX_OP_FIXED};
  if (!host) return 1;
  for (size_t i = 0; i < n; ++i) host[i] = 0x3C00; /* binary16 1.0 */
  for (int k = 0; k < 3; ++k) {
    size_t b = armx_workspace_bytes(ops[k], n, 0, NULL);
    if (b > ws_bytes) ws_bytes = b;
  }
  EXPECT(hipMalloc(&x, n * sizeof(uint16_t)) == 0);
  EXPECT(hipMalloc((void**)&out, 3 * sizeof(float)) == 0);
  EXPECT(hipMalloc((void**)&fixed, 2 * sizeof(int64_t)) == 0);
  EXPECT(hipMalloc(&ws, ws_bytes) == 0);
  if (failures) return failures;
  EXPECT(hipMemset(ws, 0, ws_bytes) == 0); /* the counter region starts at zero */
  EXPECT(hipMemcpy(x, host, n * sizeof(uint16_t), kHostToDevice) == 0);
  EXPECT(reduce_sum(x, n, out + 0, ws, ws_bytes, NULL, NULL) == ARMX_OK);
  EXPECT(reduce_sum_exact(x, n, out + 1, fixed, ws, ws_bytes, NULL, NULL) == ARMX_OK);
  EXPECT(reduce_sum_fixed_order(x, n, out + 2, ws, ws_bytes, NULL, NULL) == ARMX_OK);
  EXPECT(hipDeviceSynchronize() == 0);
  EXPECT(hipMemcpy(got, out, sizeof(got), kDeviceToHost) == 0);
  EXPECT(hipMemcpy(q, fixed, sizeof(q), kDeviceToHost) == 0);
  for (int k = 0; k < 3; ++k) {
    if (got[k] != (float)n) fprintf(stderr, "entry %d: got %.1f want %zu\n", k, got[k], n);
    EXPECT(got[k] == (float)n);
  }
  EXPECT(q[0] == (int64_t)n << 24 && q[1] == 0);
  hipFree(x);
  hipFree(out);
  hipFree(fixed);
  hipFree(ws);
  free(host);
  return failures;
}

int main(int argc, char** argv) {
  const int gpu = argc > 1 && argv[1][0] == 'g';
  int f = cpu_checks();
  if (gpu) f += gpu_checks();
  printf("%s checks: %s\n", gpu ? "cpu+gpu" : "cpu", f ? "FAILED" : "ok");
  return f ? 1 : 0;
}
