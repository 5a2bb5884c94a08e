/*
 * abi_roundtrip.c -- a plain C program that uses libkvfp4 through its C ABI alone:
 * hipMalloc'd device buffers, a HIP stream of its own, every scale rule, several group
 * layouts, both quantize forms (per-call options of kvfp4_quantize_ex), and host-side
 * argument errors.  Its outputs are compared byte for byte with the oracle (test infrastructure, loaded as its own library).  Exit status 0 = all equal.
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
int kvfp4_oracle_quantize_paged(const uint16_t* x, int64_t n_blocks, int64_t rows_per_page, int d,
                                int rule, const int32_t* table, int64_t n_pages, uint8_t* codes,
                                uint8_t* scales, float* page_amax);
int kvfp4_oracle_dequantize_paged(const uint8_t* codes, const uint8_t* scales,
                                  const float* page_amax, const int32_t* table, int64_t n_blocks,
                                  int64_t rows_per_page, int d, int64_t n_pages, uint16_t* y);
int kvfp4_oracle_rtn_quantize(const uint16_t* x, int64_t rows, int d, int bits, uint8_t* codes,
                              uint16_t* scales);
int kvfp4_oracle_rtn_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t rows, int d,
                                int bits, uint16_t* y);
int kvfp4_oracle_attend_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t tk,
                             int heads, int d, double scale, const int64_t* rows, int64_t n_rows,
                             uint16_t* out, double* scratch);

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

/* random bf16 patterns with biased exponents e0 .. e0 + span - 1 and random signs */
static void fill_bf16(uint16_t* x, int64_t n, int e0, int span) {
  for (int64_t i = 0; i < n; ++i) {
    uint64_t r = next_u64();
    uint16_t e = (uint16_t)(e0 + r % span);
    x[i] = (uint16_t)(((r >> 8) & 1) << 15 | e << 7 | ((r >> 16) & 127));
  }
}

static double bf16_value(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return (double)f;
}

static int run_case(int64_t rows, int d, int64_t rpg, int rule,
                    const struct kvfp4_quantize_opts* opts, hipStream_t st) {
  const int64_t n = rows * d, ng = (rows + rpg - 1) / rpg;
  uint16_t* x = (uint16_t*)malloc(n * 2);
  fill_bf16(x, n, 110, 30);  /* magnitudes 2^-17 .. 2^13 */
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
  int rc = kvfp4_quantize_ex((const uint16_t*)dx, rows, d, rpg, rule, (uint8_t*)dc,
                             (uint8_t*)ds, (float*)da, opts, st);
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

/* Paged cache: 9 logical blocks of 5 rows into 12 pages in shuffled order, one entry out of
 * range (skipped); quantize into the pages, then gather back. */
static int run_paged(int rule, const struct kvfp4_quantize_opts* opts, hipStream_t st) {
  enum { NB = 9, RPP = 5, D = 128, NP = 12 };
  const int32_t table[NB] = {7, 2, 11, 0, 5, -1, 9, 3, 1};
  const int64_t n = (int64_t)NB * RPP * D, pn = (int64_t)NP * RPP * D;
  uint16_t* x = malloc(n * 2);
  fill_bf16(x, n, 115, 20);
  uint8_t *oc = calloc(pn / 2, 1), *os = calloc(pn / 16, 1), *gc = malloc(pn / 2),
          *gs = malloc(pn / 16);
  float *oa = calloc(NP, 4), *ga = malloc(NP * 4);
  uint16_t *oy = calloc(n, 2), *gy = malloc(n * 2);
  if (kvfp4_oracle_quantize_paged(x, NB, RPP, D, rule, table, NP, oc, os, oa) ||
      kvfp4_oracle_dequantize_paged(oc, os, oa, table, NB, RPP, D, NP, oy)) {
    fprintf(stderr, "oracle rejected the paged case\n");
    return 1;
  }
  void *dx, *dt, *dc, *ds, *da, *dy;
  CHECK_HIP(hipMalloc(&dx, n * 2));
  CHECK_HIP(hipMalloc(&dt, sizeof table));
  CHECK_HIP(hipMalloc(&dc, pn / 2));
  CHECK_HIP(hipMalloc(&ds, pn / 16));
  CHECK_HIP(hipMalloc(&da, NP * 4));
  CHECK_HIP(hipMalloc(&dy, n * 2));
  CHECK_HIP(hipMemsetAsync(dc, 0, pn / 2, st));
  CHECK_HIP(hipMemsetAsync(ds, 0, pn / 16, st));
  CHECK_HIP(hipMemsetAsync(da, 0, NP * 4, st));
  CHECK_HIP(hipMemsetAsync(dy, 0, n * 2, st));
  CHECK_HIP(hipMemcpyAsync(dx, x, n * 2, hipMemcpyHostToDevice, st));
  CHECK_HIP(hipMemcpyAsync(dt, table, sizeof table, hipMemcpyHostToDevice, st));
  int rc = kvfp4_quantize_paged_ex((const uint16_t*)dx, NB, RPP, D, rule, (const int32_t*)dt,
                                   NP, (uint8_t*)dc, (uint8_t*)ds, (float*)da, opts, st);
  if (rc == KVFP4_OK)
    rc = kvfp4_dequantize_paged((const uint8_t*)dc, (const uint8_t*)ds, (const float*)da,
                                (const int32_t*)dt, NB, RPP, D, NP, (uint16_t*)dy, st);
  if (rc != KVFP4_OK) {
    fprintf(stderr, "kvfp4 paged call failed: %s\n", kvfp4_status_str(rc));
    return 1;
  }
  CHECK_HIP(hipMemcpyAsync(gc, dc, pn / 2, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipMemcpyAsync(gs, ds, pn / 16, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipMemcpyAsync(ga, da, NP * 4, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipMemcpyAsync(gy, dy, n * 2, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipStreamSynchronize(st));
  int bad = memcmp(gc, oc, pn / 2) || memcmp(gs, os, pn / 16) || memcmp(ga, oa, NP * 4) ||
            memcmp(gy, oy, n * 2);
  printf("paged %d blocks x %d rows into %d pages, rule %d: %s\n", NB, RPP, NP, rule,
         bad ? "MISMATCH" : "bit-exact");
  CHECK_HIP(hipFree(dx));
  CHECK_HIP(hipFree(dt));
  CHECK_HIP(hipFree(dc));
  CHECK_HIP(hipFree(ds));
  CHECK_HIP(hipFree(da));
  CHECK_HIP(hipFree(dy));
  free(x); free(oc); free(os); free(gc); free(gs); free(oa); free(ga); free(oy); free(gy);
  return bad;
}

/* RTN INT4 / INT2 round trip (no recent tail). */
static int run_rtn(int bits, hipStream_t st) {
  const int64_t rows = 100, d = 128, n = rows * d, cb = n * bits / 8, sn = n / 16;
  uint16_t* x = malloc(n * 2);
  fill_bf16(x, n, 110, 30);
  uint8_t *oc = malloc(cb), *gc = malloc(cb);
  uint16_t *os = malloc(sn * 2), *gs = malloc(sn * 2), *oy = malloc(n * 2), *gy = malloc(n * 2);
  if (kvfp4_oracle_rtn_quantize(x, rows, (int)d, bits, oc, os) ||
      kvfp4_oracle_rtn_dequantize(oc, os, rows, (int)d, bits, oy)) {
    fprintf(stderr, "oracle rejected the RTN case\n");
    return 1;
  }
  void *dx, *dc, *ds, *dy;
  CHECK_HIP(hipMalloc(&dx, n * 2));
  CHECK_HIP(hipMalloc(&dc, cb));
  CHECK_HIP(hipMalloc(&ds, sn * 2));
  CHECK_HIP(hipMalloc(&dy, n * 2));
  CHECK_HIP(hipMemcpyAsync(dx, x, n * 2, hipMemcpyHostToDevice, st));
  int rc = kvfp4_rtn_quantize((const uint16_t*)dx, rows, (int32_t)d, bits, (uint8_t*)dc,
                              (uint16_t*)ds, st);
  if (rc == KVFP4_OK)
    rc = kvfp4_rtn_dequantize((const uint8_t*)dc, (const uint16_t*)ds, rows, (int32_t)d, bits,
                              NULL, 0, (uint16_t*)dy, st);
  if (rc != KVFP4_OK) {
    fprintf(stderr, "kvfp4 RTN call failed: %s\n", kvfp4_status_str(rc));
    return 1;
  }
  CHECK_HIP(hipMemcpyAsync(gc, dc, cb, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipMemcpyAsync(gs, ds, sn * 2, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipMemcpyAsync(gy, dy, n * 2, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipStreamSynchronize(st));
  int bad = memcmp(gc, oc, cb) || memcmp(gs, os, sn * 2) || memcmp(gy, oy, n * 2);
  printf("rtn int%d %lld rows x %lld: %s\n", bits, (long long)rows, (long long)d,
         bad ? "MISMATCH" : "bit-exact");
  CHECK_HIP(hipFree(dx));
  CHECK_HIP(hipFree(dc));
  CHECK_HIP(hipFree(ds));
  CHECK_HIP(hipFree(dy));
  free(x); free(oc); free(gc); free(os); free(gs); free(oy); free(gy);
  return bad;
}

/* Attention over the packed cache vs the oracle's double attention over its own dequantized
 * K and V: max |err| <= 2e-2 and RMS(err) <= 1e-2 RMS(ref). */
static int run_attend(hipStream_t st) {
  enum { TQ = 40, TK = 200, H = 2, D = 64, TPG = 50 };
  const int64_t nq = (int64_t)TQ * H * D, nk = (int64_t)TK * H * D, rpg = (int64_t)TPG * H;
  const int64_t ng = (TK + TPG - 1) / TPG;
  uint16_t *q = malloc(nq * 2), *k = malloc(nk * 2), *v = malloc(nk * 2);
  fill_bf16(q, nq, 122, 6);  /* magnitudes 2^-5 .. 2^1 */
  fill_bf16(k, nk, 122, 6);
  fill_bf16(v, nk, 122, 6);
  uint8_t *kc = malloc(nk / 2), *ks = malloc(nk / 16), *vc = malloc(nk / 2), *vs = malloc(nk / 16);
  float *ka = malloc(ng * 4), *va = malloc(ng * 4);
  uint16_t *kd = malloc(nk * 2), *vd = malloc(nk * 2), *ref = malloc(nq * 2), *got = malloc(nq * 2);
  int64_t rows[TQ * H];
  for (int i = 0; i < TQ * H; ++i) rows[i] = i;
  double* scratch = malloc(TK * sizeof(double));
  if (kvfp4_oracle_quantize(k, (int64_t)TK * H, D, rpg, 0, kc, ks, ka) ||
      kvfp4_oracle_dequantize(kc, ks, ka, (int64_t)TK * H, D, rpg, kd) ||
      kvfp4_oracle_quantize(v, (int64_t)TK * H, D, rpg, 0, vc, vs, va) ||
      kvfp4_oracle_dequantize(vc, vs, va, (int64_t)TK * H, D, rpg, vd) ||
      kvfp4_oracle_attend_rows(q, kd, vd, TK, H, D, 0.125, rows, TQ * H, ref, scratch)) {
    fprintf(stderr, "oracle rejected the attention case\n");
    return 1;
  }
  void *dq, *dk, *dv, *dkc, *dks, *dka, *dvc, *dvs, *dva, *dout;
  CHECK_HIP(hipMalloc(&dq, nq * 2));
  CHECK_HIP(hipMalloc(&dk, nk * 2));
  CHECK_HIP(hipMalloc(&dv, nk * 2));
  CHECK_HIP(hipMalloc(&dkc, nk / 2));
  CHECK_HIP(hipMalloc(&dks, nk / 16));
  CHECK_HIP(hipMalloc(&dka, ng * 4));
  CHECK_HIP(hipMalloc(&dvc, nk / 2));
  CHECK_HIP(hipMalloc(&dvs, nk / 16));
  CHECK_HIP(hipMalloc(&dva, ng * 4));
  CHECK_HIP(hipMalloc(&dout, nq * 2));
  CHECK_HIP(hipMemcpyAsync(dq, q, nq * 2, hipMemcpyHostToDevice, st));
  CHECK_HIP(hipMemcpyAsync(dk, k, nk * 2, hipMemcpyHostToDevice, st));
  CHECK_HIP(hipMemcpyAsync(dv, v, nk * 2, hipMemcpyHostToDevice, st));
  int rc = kvfp4_quantize((const uint16_t*)dk, (int64_t)TK * H, D, rpg, 0, (uint8_t*)dkc,
                          (uint8_t*)dks, (float*)dka, st);
  if (rc == KVFP4_OK)
    rc = kvfp4_quantize((const uint16_t*)dv, (int64_t)TK * H, D, rpg, 0, (uint8_t*)dvc,
                        (uint8_t*)dvs, (float*)dva, st);
  if (rc == KVFP4_OK)
    rc = kvfp4_attend((const uint16_t*)dq, TQ, (const uint8_t*)dkc, (const uint8_t*)dks,
                      (const float*)dka, (const uint8_t*)dvc, (const uint8_t*)dvs,
                      (const float*)dva, TK, H, D, TPG, 0.125f, (uint16_t*)dout, st);
  if (rc != KVFP4_OK) {
    fprintf(stderr, "kvfp4 attention call failed: %s\n", kvfp4_status_str(rc));
    return 1;
  }
  CHECK_HIP(hipMemcpyAsync(got, dout, nq * 2, hipMemcpyDeviceToHost, st));
  CHECK_HIP(hipStreamSynchronize(st));
  double mx = 0.0, se = 0.0, sr = 0.0;
  for (int64_t i = 0; i < nq; ++i) {
    const double a = bf16_value(got[i]), b = bf16_value(ref[i]), e = a > b ? a - b : b - a;
    if (e > mx) mx = e;
    se += e * e;
    sr += b * b;
  }
  const double rel = sr > 0.0 ? __builtin_sqrt(se / sr) : 0.0;
  const int bad = !(mx <= 2e-2 && rel <= 1e-2);
  printf("attend %d x %d keys, %d heads, d %d: max err %.3g, rel RMS %.3g: %s\n", TQ, TK, H, D,
         mx, rel, bad ? "OUT OF TOLERANCE" : "within tolerance");
  void* bufs[] = {dq, dk, dv, dkc, dks, dka, dvc, dvs, dva, dout};
  for (int i = 0; i < 10; ++i) CHECK_HIP(hipFree(bufs[i]));
  free(q); free(k); free(v); free(kc); free(ks); free(vc); free(vs); free(ka); free(va);
  free(kd); free(vd); free(ref); free(got); free(scratch);
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
  const struct kvfp4_quantize_opts forms[2] = {{KVFP4_FORM_ONE_KERNEL, 20000},
                                               {KVFP4_FORM_THREE_KERNEL, 20000}};
  for (int f = 0; f < 2; ++f) {
    printf("append form: %s\n", f == 0 ? "one kernel where it applies" : "three kernels");
    for (int rule = 0; rule < 3; ++rule) {
      bad |= run_case(1000, 128, 300, rule, &forms[f], st);
      bad |= run_case(37, 64, 10, rule, &forms[f], st);
      bad |= run_case(513, 256, 513, rule, &forms[f], st);
    }
  }
  /* the plain entry point (NULL options) */
  bad |= run_case(1000, 128, 300, KVFP4_RULE_MSE, NULL, st);
  bad |= run_paged(0, NULL, st);
  bad |= run_paged(2, &forms[1], st);
  bad |= run_rtn(4, st);
  bad |= run_rtn(2, st);
  bad |= run_attend(st);
  /* host-side argument errors: nothing is enqueued */
  void* p;
  CHECK_HIP(hipMalloc(&p, 1 << 16));
  uint8_t* b = (uint8_t*)p;
  int e1 = kvfp4_quantize((const uint16_t*)(b + 8), 4, 64, 4, 0, b + 4096, b + 8192, (float*)(b + 12288), st);
  int e2 = kvfp4_dequantize(b, b + 4096, (const float*)(b + 8192), 4, 96, 4, (uint16_t*)(b + 12288), st);
  int e3 = kvfp4_quantize((const uint16_t*)b, 4, 64, 4, 7, b + 4096, b + 8192, (float*)(b + 12288), st);
  const struct kvfp4_quantize_opts bad_form = {7, 20000}, bad_wait = {KVFP4_FORM_AUTO, -1};
  int e4 = kvfp4_quantize_ex((const uint16_t*)b, 4, 64, 4, 0, b + 4096, b + 8192,
                             (float*)(b + 12288), &bad_form, st);
  int e5 = kvfp4_fake_quantize_ex((const uint16_t*)b, 4, 64, 4, 0, (float*)(b + 12288),
                                  (uint16_t*)(b + 16384), &bad_wait, st);
  printf("errors: misaligned x -> %d, head_dim 96 -> %d, rule 7 -> %d, form 7 -> %d, "
         "wait -1 -> %d\n", e1, e2, e3, e4, e5);
  bad |= !(e1 == KVFP4_EALIGN && e2 == KVFP4_EUNSUPPORTED && e3 == KVFP4_EINVAL &&
           e4 == KVFP4_EINVAL && e5 == KVFP4_EINVAL);
  CHECK_HIP(hipFree(p));
  CHECK_HIP(hipStreamDestroy(st));
  printf("%s\n", bad ? "FAILED" : "OK");
  return bad;
}
