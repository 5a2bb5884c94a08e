/*
 * abi_roundtrip.c -- a plain C program that uses libkvfp4 through its C ABI alone:
 * hipMalloc'd device buffers, a HIP stream of its own, every scale rule, several group
 * layouts, both quantize forms (KVFP4_OPT_APPEND_FUSED), and host-side argument errors.  Its outputs are compared byte for byte with the
 * oracle (test infrastructure, loaded as its own library).  Exit status 0 = all equal.
 *
 * Input: bf16 bit patterns drawn from a fixed-seed xorshift generator with the exponent
 * limited to [2^-17, 2^13) (finite, every group amax inside the contract), plus an
 * all-zero group.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvfp4.h"

/* oracle (test infrastructure) */
int kvfp4_oracle_quantize(const uint16_t* x, int64_t rows, int d, int64_t rows_per_group,
                          int rule, uint8_t* codes, uint8_t* scales, float* group_amax);
int kvfp4_oracle_dequantize(const uint8_t* codes, const uint8_t* scales, const float* group_amax,
                            int64_t rows, int d, int64_t rows_per_group, uint16_t* y);

#define CHECK_HIP(call)                                                                 \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "%s:%d: %s failed: %s\n", __FILE__, __LINE__, #call,              \
              hipGetErrorString(e_));                                                   \
      exit(2);                                                                          \
    }                                                                                   \
  } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return g_state;
}

static int run_case(int64_t rows, int d, int64_t rpg, int rule, hipStream_t st) {
  const int64_t n = rows * d, ng = (rows + rpg - 1) / rpg;
  uint16_t* x = (uint16_t*)malloc(n * 2);
  for (int64_t i = 0; i < n; ++i) {
    uint64_t r = next_u64();
    uint16_t e = (uint16_t)(110 + r % 30);  /* biased exponent 110..139 */
    x[i] = (uint16_t)(((r >> 8) & 1) << 15 | e << 7 | ((r >> 16) & 127));
  }
  if (rows >= 2 * rpg) memset(x + rpg * d, 0, rpg * d * 2); /* second group all zero */

  uint8_t *oc = malloc(n / 2), *os = malloc(n / 16), *gc = malloc(n / 2), *gs = malloc(n / 16);
  float *oa = malloc(ng * 4), *ga = malloc(ng * 4);
  uint16_t *oy = malloc(n * 2), *gy = malloc(n * 2);
  if (kvfp4_oracle_quantize(x, rows, d, rpg, rule, oc, os, oa) ||
      kvfp4_oracle_dequantize(oc, os, oa, rows, d, rpg, oy)) {
    fprintf(stderr, "oracle rejected the case\n");
    return 1;
  }

  void *dx, *dc, *ds, *da, *dy;
  CHECK_HIP(hipMalloc(&dx, n * 2));
  CHECK_HIP(hipMalloc(&dc, n / 2));
  CHECK_HIP(hipMalloc(&ds, n / 16));
  CHECK_HIP(hipMalloc(&da, ng * 4));
  CHECK_HIP(hipMalloc(&dy, n * 2));
  CHECK_HIP(hipMemcpyAsync(dx, x, n * 2, hipMemcpyHostToDevice, st));
  int rc = kvfp4_quantize((const uint16_t*)dx, rows, d, rpg, rule, (uint8_t*)dc, (uint8_t*)ds,
                          (float*)da, st);
  if (rc == KVFP4_OK)
    rc = kvfp4_dequantize((const uint8_t*)dc, (const uint8_t*)ds, (const float*)da, rows, d, rpg,
                          (uint16_t*)dy, st);
  if (rc != KVFP4_OK) {
    fprintf(stderr, "kvfp4 call failed: %s\n", kvfp4_status_str(rc));
    return 1;
  }
  CHECK_HIP(hipMemcpyAsync(gc, dc, n / 2, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipMemcpyAsync(gs, ds, n / 16, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipMemcpyAsync(ga, da, ng * 4, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipMemcpyAsync(gy, dy, n * 2, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipStreamSynchronize(st));
  int bad = memcmp(gc, oc, n / 2) || memcmp(gs, os, n / 16) || memcmp(ga, oa, ng * 4) ||
            memcmp(gy, oy, n * 2);
  printf("rows %lld d %d rows_per_group %lld rule %d: %s\n", (long long)rows, d, (long long)rpg,
         rule, bad ? "MISMATCH" : "bit-exact");
  CHECK_HIP(hipFree(dx));
  CHECK_HIP(hipFree(dc));
  CHECK_HIP(hipFree(ds));
  CHECK_HIP(hipFree(da));
  CHECK_HIP(hipFree(dy));
  free(x); free(oc); free(os); free(gc); free(gs); free(oa); free(ga); free(oy); free(gy);
  return bad;
}

int main(void) {
  if (kvfp4_abi_version() != KVFP4_ABI_VERSION) {
    fprintf(stderr, "ABI version mismatch\n");
    return 1;
  }
  hipStream_t st;
  CHECK_HIP(hipStreamCreate(&st));
  int bad = 0;
  /* both quantize forms (the one-kernel form applies to the first and third layouts) */
  for (int fused = 1; fused >= 0; --fused) {
    if (kvfp4_set_option(KVFP4_OPT_APPEND_FUSED, fused) != KVFP4_OK) bad = 1;
    printf("append form: %s\n", fused ? "one kernel where it applies" : "three kernels");
    for (int rule = 0; rule < 3; ++rule) {
      bad |= run_case(1000, 128, 300, rule, st);
      bad |= run_case(37, 64, 10, rule, st);
      bad |= run_case(513, 256, 513, rule, st);
    }
  }
  if (kvfp4_set_option(KVFP4_OPT_APPEND_FUSED, 1) != KVFP4_OK) bad = 1;
  /* host-side argument errors: nothing is enqueued */
  void* p;
  CHECK_HIP(hipMalloc(&p, 1 << 16));
  uint8_t* b = (uint8_t*)p;
  int e1 = kvfp4_quantize((const uint16_t*)(b + 8), 4, 64, 4, 0, b + 4096, b + 8192, (float*)(b + 12288), st);
  int e2 = kvfp4_dequantize(b, b + 4096, (const float*)(b + 8192), 4, 96, 4, (uint16_t*)(b + 12288), st);
  int e3 = kvfp4_quantize((const uint16_t*)b, 4, 64, 4, 7, b + 4096, b + 8192, (float*)(b + 12288), st);
  int64_t ov = -1;
  int e4 = kvfp4_set_option(99, 0);
  int e5 = kvfp4_get_option(KVFP4_OPT_APPEND_WAIT_US, &ov);
  printf("errors: misaligned x -> %d, head_dim 96 -> %d, rule 7 -> %d, option 99 -> %d\n", e1,
         e2, e3, e4);
  bad |= !(e1 == KVFP4_EALIGN && e2 == KVFP4_EUNSUPPORTED && e3 == KVFP4_EINVAL &&
           e4 == KVFP4_EINVAL && e5 == KVFP4_OK && ov >= 0);
  CHECK_HIP(hipFree(p));
  CHECK_HIP(hipStreamDestroy(st));
  printf("%s\n", bad ? "FAILED" : "OK");
  return bad;
}
