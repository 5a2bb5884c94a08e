/*
 * kvfp4_oracle.c -- plain, slow, single-threaded CPU reference for NVFP4 KV-cache
 * quantization, dequantization and attention over a dequantized cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this file's library.  It shares no code, header, table or
 * constant generator with the HIP library; it includes only the C standard library.
 *
 * Pages cited (titles as published):
 *   [P-KV]    "How to Use KV Cache Quantization with LongLive's LongLiveQuantizationConfig"
 *   [P-NVFP4] "How NVFP4 Quantization Works in LongLive 2.0 for Transformer Inference"
 *   [P-SF]    "KV Cache Quantization for Self-Forcing Video Generation: A 33-Method
 *              Empirical Study"
 *
 * Arithmetic contract: every floating-point step is one IEEE binary32 operation with
 * round-to-nearest-even, no contraction (build with -ffp-contract=off), denormals kept;
 * fmaf() appears only where the mse error sum names it.  Format conversions are done by
 * scanning the value table in double and taking the nearest entry (ties to the even
 * code), never by bit tricks, so that they can be read against the format definitions.
 *
 * Readings of the pages that this file fixes (each listed with its reason in the
 * design notes of the repository):
 *   - the 4-bit element is E2M1 (grid 0, .5, 1, 1.5, 2, 3, 4, 6); the page's "e4m3"
 *     label is taken as garbled because its own static-6 divisor and its e2m1_max name
 *     only fit E2M1 ([P-NVFP4] "Understanding the NVFP4 Format", "Stage 3");
 *   - block scales are OCP FP8 E4M3 (max 448), rounded to nearest even, saturating;
 *   - one global amax per scale group (one appended chunk of K or of V);
 *   - s_dec = A/2688 and s_enc = 2688/A for every rule (2688 = e2m1_max * e4m3_max);
 *   - per-block reciprocal inv = 1/S, then y = x*inv per element;
 *   - a product with a zero operand is zero, also where binary32 would form 0*inf = NaN
 *     (s_enc = 2688/A overflows when A < 2688/FLT_MAX, inv = 1/S when S < 1/FLT_MAX): an
 *     all-zero block gets u = 0 (scale byte 0x00), a zero element y = +-0 (its own sign),
 *     a zero RTN element q = 0; nonzero operands keep x*inf = +-inf, which saturates;
 *   - element 2j goes in the low nibble, 2j+1 in the high nibble;
 *   - mse: squared error of the fp32 reconstruction, fma chains over each half
 *     block, 4-max chosen only when strictly better.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------
 * Element format: E2M1.  [P-NVFP4] "Understanding the NVFP4 Format and Architecture"
 * (4-bit floating-point element, scale = amax / 6.0, two values per uint8).
 * Magnitude grid by 3-bit code; bit 3 of the code is the sign.
 * ---------------------------------------------------------------------------------- */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double kvfp4_oracle_e2m1_value(int code) {
  double mag = E2M1_GRID[code & 7];
  return (code & 8) ? -mag : mag; /* code 8 decodes to -0.0 */
}

/* Nearest grid point to |y|; on an exact tie the even code wins; |y| >= 6 gives 6.
 * The sign bit of the code is the sign bit of y (so a small negative y gives code 8). */
int kvfp4_oracle_e2m1_encode(float y) {
  int sign = signbit(y) ? 8 : 0;
  double a = fabs((double)y);
  if (a >= 6.0) return sign | 7;
  int best = 0;
  double bestd = a; /* distance to grid[0] = 0 */
  for (int c = 1; c < 8; ++c) {
    double d = fabs(a - E2M1_GRID[c]);
    if (d < bestd || (d == bestd && (c % 2) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return sign | best;
}

/* ------------------------------------------------------------------------------------
 * Block-scale format: FP8 E4M3 (OCP flavour: bias 7, subnormals, no infinities, 0x7F is
 * NaN, so the largest finite byte is 0x7E = 448).  [P-NVFP4] "Understanding the NVFP4
 * Format and Architecture" (per-block scales quantized to FP8) and "Stage 3" (e4m3_max).
 * Only non-negative scale bytes 0x00..0x7E occur.
 * ---------------------------------------------------------------------------------- */
double kvfp4_oracle_e4m3_value(int byte) {
  int e = (byte >> 3) & 15;
  int m = byte & 7;
  if (e == 0) return ldexp((double)m, -9);   /* subnormal: m * 2^-9 */
  return ldexp(1.0 + m / 8.0, e - 7);        /* normal: (1 + m/8) * 2^(e-7) */
}

/* u >= 0, finite.  u >= 448 saturates to 0x7E; otherwise nearest finite E4M3 value,
 * ties to the even byte. */
int kvfp4_oracle_e4m3_encode(float u) {
  double v = (double)u;
  if (v >= 448.0) return 0x7E;
  int best = 0;
  double bestd = fabs(v);
  for (int b = 1; b <= 0x7E; ++b) {
    double d = fabs(v - kvfp4_oracle_e4m3_value(b));
    if (d < bestd || (d == bestd && (b % 2) == 0)) {
      best = b;
      bestd = d;
    }
  }
  return best;
}

/* ------------------------------------------------------------------------------------
 * bfloat16 <-> binary32.  A bf16 value is a binary32 value whose low 16 bits are zero.
 * ---------------------------------------------------------------------------------- */
static float f32_from_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, sizeof f);
  return f;
}
static uint32_t bits_from_f32(float f) {
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  return b;
}

float kvfp4_oracle_bf16_to_float(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Round to the nearer of the two bf16 values that bracket f (ties: even bf16 mantissa).
 * The candidate above the largest finite bf16 is treated as 2^128 (IEEE overflow rule). */
uint16_t kvfp4_oracle_float_to_bf16(float f) {
  uint32_t bits = bits_from_f32(f);
  if (isnan(f)) return (uint16_t)((bits >> 16) | 0x0040u);
  uint32_t lo = bits & 0xFFFF0000u;           /* toward zero */
  if (lo == bits) return (uint16_t)(bits >> 16);
  uint32_t hi = lo + 0x00010000u;             /* next bf16 away from zero */
  double vlo = (double)f32_from_bits(lo);
  double vhi = ((hi & 0x7F800000u) == 0x7F800000u) ? copysign(ldexp(1.0, 128), (double)f)
                                                    : (double)f32_from_bits(hi);
  double dlo = fabs((double)f - vlo);
  double dhi = fabs(vhi - (double)f);
  uint32_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = ((lo >> 16) & 1u) ? hi : lo;
  return (uint16_t)(pick >> 16);
}

/* Round a double to the nearest bf16 value, ties to the even bf16 mantissa, in one step
 * (no intermediate binary32 rounding).  bf16 has 8 significant bits above 2^-126 and a
 * fixed spacing of 2^-133 below it; a magnitude that rounds to 2^128 or more overflows to
 * infinity. */
uint16_t kvfp4_oracle_double_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0u;
  const uint16_t sign = signbit(v) ? 0x8000u : 0x0000u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                                  /* a = f * 2^e, f in [0.5, 1) */
  int q = e - 8;                                 /* spacing 2^q for 8 significant bits */
  if (q < -133) q = -133;                        /* subnormal range: spacing 2^-133 */
  double scaled = ldexp(a, -q);                  /* exact: a power-of-two scaling */
  double k = floor(scaled);
  double below = scaled - k, above = (k + 1.0) - scaled;   /* both exact */
  if (above < below || (above == below && fmod(k, 2.0) != 0.0)) k += 1.0;
  double r = ldexp(k, q);                        /* exact unless it overflows */
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | (bits_from_f32((float)r) >> 16));  /* r is a bf16 value */
}

/* ------------------------------------------------------------------------------------
 * Quantization.  [P-NVFP4] "Stage 1" (per-block amax, per-block scale by the static-6
 * rule, two codes per uint8, one global amax for the whole tensor) and "Stage 3"
 * (global_scale = amax / (e2m1_max * e4m3_max)); [P-KV] "Programmatic Configuration" and
 * "Configuration Parameters Reference" (scale rules static_6, static_4, mse);
 * [P-SF] Table 3 (block size 16).
 * ---------------------------------------------------------------------------------- */
enum { RULE_STATIC6 = 0, RULE_STATIC4 = 1, RULE_MSE = 2 };
#define E2M1_MAX 6.0f
#define E4M3_MAX 448.0f

/* Q1: global amax of one scale group = max |x| over its elements. */
float kvfp4_oracle_group_amax(const uint16_t* x, int64_t n) {
  float a = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float v = fabsf(kvfp4_oracle_bf16_to_float(x[i]));
    if (v > a) a = v;
  }
  return a;
}

/* One candidate scaling of a 16-element block (Q4, Q5). */
typedef struct {
  int sf;       /* E4M3 scale byte */
  float S;      /* decoded block scale times s_dec */
  int code[16]; /* E2M1 codes */
} candidate_t;

static void make_candidate(const float* xb, float m, float dv, float s_enc, float s_dec,
                           candidate_t* c) {
  float t = m / dv;
  float u = (t == 0.0f) ? 0.0f : t * s_enc; /* zero block: u = 0 even if s_enc = inf */
  c->sf = kvfp4_oracle_e4m3_encode(u);
  float S = (float)kvfp4_oracle_e4m3_value(c->sf) * s_dec;
  float inv = (S > 0.0f) ? 1.0f / S : 0.0f;
  c->S = S;
  for (int i = 0; i < 16; ++i) {
    float y = (xb[i] == 0.0f) ? xb[i] : xb[i] * inv; /* +-0 stays +-0 even if inv = inf */
    c->code[i] = kvfp4_oracle_e2m1_encode(y);
  }
}

/* Q6: squared reconstruction error of a candidate: fma chain over elements 0..7, another
 * over 8..15, then their sum. */
static float candidate_error(const float* xb, const candidate_t* c) {
  float e_lo = 0.0f, e_hi = 0.0f;
  for (int i = 0; i < 8; ++i) {
    float r = (float)kvfp4_oracle_e2m1_value(c->code[i]) * c->S;
    float d = xb[i] - r;
    e_lo = fmaf(d, d, e_lo);
  }
  for (int i = 8; i < 16; ++i) {
    float r = (float)kvfp4_oracle_e2m1_value(c->code[i]) * c->S;
    float d = xb[i] - r;
    e_hi = fmaf(d, d, e_hi);
  }
  return e_lo + e_hi;
}

/* Q2-Q7 for `rows` rows of width d whose group amax is A. */
int kvfp4_oracle_quantize_rows(const uint16_t* x, int64_t rows, int d, float A, int rule,
                               uint8_t* codes, uint8_t* scales) {
  if (rows < 0 || d <= 0 || d % 16 != 0) return 1;
  if (rule != RULE_STATIC6 && rule != RULE_STATIC4 && rule != RULE_MSE) return 1;
  float s_enc = (A > 0.0f) ? (E2M1_MAX * E4M3_MAX) / A : 0.0f;
  float s_dec = A / (E2M1_MAX * E4M3_MAX);
  int nb = d / 16;
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < nb; ++b) {
      float xb[16];
      float m = 0.0f;
      for (int i = 0; i < 16; ++i) {
        xb[i] = kvfp4_oracle_bf16_to_float(x[r * d + b * 16 + i]);
        if (fabsf(xb[i]) > m) m = fabsf(xb[i]);
      }
      candidate_t c6, c4;
      const candidate_t* pick;
      if (rule == RULE_STATIC6) {
        make_candidate(xb, m, 6.0f, s_enc, s_dec, &c6);
        pick = &c6;
      } else if (rule == RULE_STATIC4) {
        make_candidate(xb, m, 4.0f, s_enc, s_dec, &c4);
        pick = &c4;
      } else {
        make_candidate(xb, m, 6.0f, s_enc, s_dec, &c6);
        make_candidate(xb, m, 4.0f, s_enc, s_dec, &c4);
        float err6 = candidate_error(xb, &c6);
        float err4 = candidate_error(xb, &c4);
        pick = (err4 < err6) ? &c4 : &c6;
      }
      scales[r * nb + b] = (uint8_t)pick->sf;
      for (int j = 0; j < 8; ++j)
        codes[r * (d / 2) + b * 8 + j] =
            (uint8_t)((pick->code[2 * j] & 15) | ((pick->code[2 * j + 1] & 15) << 4));
    }
  }
  return 0;
}

/* Whole tensor: groups of rows_per_group rows (the last may be shorter). */
int kvfp4_oracle_quantize(const uint16_t* x, int64_t rows, int d, int64_t rows_per_group,
                          int rule, uint8_t* codes, uint8_t* scales, float* group_amax) {
  if (rows < 0 || rows_per_group <= 0 || d <= 0 || d % 16 != 0) return 1;
  for (int64_t r0 = 0, g = 0; r0 < rows; r0 += rows_per_group, ++g) {
    int64_t n = (rows - r0 < rows_per_group) ? rows - r0 : rows_per_group;
    float A = kvfp4_oracle_group_amax(x + r0 * d, n * d);
    group_amax[g] = A;
    int rc = kvfp4_oracle_quantize_rows(x + r0 * d, n, d, A, rule, codes + r0 * (d / 2),
                                        scales + r0 * (d / 16));
    if (rc) return rc;
  }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Dequantization.  [P-NVFP4] "Stage 3" (each byte expands to two 4-bit values, which are
 * multiplied by the per-block and the global scale; the output is float32 or bf16); [P-KV]
 * "CUDA De-quantization Pipeline" (bf16 reconstruction before attention).
 * v = E2M1(c) * S,  S = E4M3(sf) * (A / 2688), each product rounded to binary32;
 * the float32 output is v itself, the bf16 output is v rounded to bf16.
 * ---------------------------------------------------------------------------------- */
static float dequant_value(const uint8_t* codes, const uint8_t* scales, int64_t r, int d, int i,
                           float s_dec) {
  int nb = d / 16;
  float S = (float)kvfp4_oracle_e4m3_value(scales[r * nb + i / 16]) * s_dec;
  uint8_t byte = codes[r * (d / 2) + i / 2];
  int c = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
  return (float)kvfp4_oracle_e2m1_value(c) * S;
}

int kvfp4_oracle_dequantize_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                 int d, float A, uint16_t* y) {
  if (rows < 0 || d <= 0 || d % 16 != 0) return 1;
  float s_dec = A / (E2M1_MAX * E4M3_MAX);
  for (int64_t r = 0; r < rows; ++r)
    for (int i = 0; i < d; ++i)
      y[r * d + i] = kvfp4_oracle_float_to_bf16(dequant_value(codes, scales, r, d, i, s_dec));
  return 0;
}

int kvfp4_oracle_dequantize_rows_f32(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                     int d, float A, float* y) {
  if (rows < 0 || d <= 0 || d % 16 != 0) return 1;
  float s_dec = A / (E2M1_MAX * E4M3_MAX);
  for (int64_t r = 0; r < rows; ++r)
    for (int i = 0; i < d; ++i) y[r * d + i] = dequant_value(codes, scales, r, d, i, s_dec);
  return 0;
}

int kvfp4_oracle_dequantize(const uint8_t* codes, const uint8_t* scales,
                            const float* group_amax, int64_t rows, int d,
                            int64_t rows_per_group, uint16_t* y) {
  if (rows < 0 || rows_per_group <= 0 || d <= 0 || d % 16 != 0) return 1;
  for (int64_t r0 = 0, g = 0; r0 < rows; r0 += rows_per_group, ++g) {
    int64_t n = (rows - r0 < rows_per_group) ? rows - r0 : rows_per_group;
    int rc = kvfp4_oracle_dequantize_rows(codes + r0 * (d / 2), scales + r0 * (d / 16), n, d,
                                          group_amax[g], y + r0 * d);
    if (rc) return rc;
  }
  return 0;
}

int kvfp4_oracle_dequantize_f32(const uint8_t* codes, const uint8_t* scales,
                                const float* group_amax, int64_t rows, int d,
                                int64_t rows_per_group, float* y) {
  if (rows < 0 || rows_per_group <= 0 || d <= 0 || d % 16 != 0) return 1;
  for (int64_t r0 = 0, g = 0; r0 < rows; r0 += rows_per_group, ++g) {
    int64_t n = (rows - r0 < rows_per_group) ? rows - r0 : rows_per_group;
    int rc = kvfp4_oracle_dequantize_rows_f32(codes + r0 * (d / 2), scales + r0 * (d / 16), n,
                                              d, group_amax[g], y + r0 * d);
    if (rc) return rc;
  }
  return 0;
}

/* Fake quantization: the tensor as the cache would return it, i.e. quantize (every step
 * above) and dequantize to bf16, without keeping the packed form.  [P-NVFP4] "Stage 1"
 * (the fake-quant variant of the static block-scale path, used where a 16-bit tensor
 * stands in for the 4-bit one).  Also returns each group's amax. */
int kvfp4_oracle_fake_quantize(const uint16_t* x, int64_t rows, int d, int64_t rows_per_group,
                               int rule, float* group_amax, uint16_t* y) {
  if (rows < 0 || rows_per_group <= 0 || d <= 0 || d % 16 != 0) return 1;
  if (rows == 0) return 0;
  uint8_t* codes = (uint8_t*)malloc((size_t)(rows * (d / 2)));
  uint8_t* scales = (uint8_t*)malloc((size_t)(rows * (d / 16)));
  int rc = (codes && scales) ? 0 : 2;
  if (!rc) rc = kvfp4_oracle_quantize(x, rows, d, rows_per_group, rule, codes, scales, group_amax);
  if (!rc) rc = kvfp4_oracle_dequantize(codes, scales, group_amax, rows, d, rows_per_group, y);
  free(codes);
  free(scales);
  return rc;
}

/* ------------------------------------------------------------------------------------
 * Paged cache.  [P-NVFP4] "Code Implementation" / "Runtime KV-Cache De-quantization" (the
 * cache as a list of blocks of block_token_size tokens, gathered for attention) and "Stage 3"
 * (each block reshaped to [block_token_size, num_heads, head_dim]).  A page is one scale
 * group; logical block b lives in page table[b]; entries outside [0, n_pages) are skipped.
 * ---------------------------------------------------------------------------------- */
int kvfp4_oracle_quantize_paged(const uint16_t* x, int64_t n_blocks, int64_t rows_per_page, int d,
                                int rule, const int32_t* table, int64_t n_pages, uint8_t* codes,
                                uint8_t* scales, float* page_amax) {
  if (n_blocks < 0 || rows_per_page <= 0 || d <= 0 || d % 16 != 0) return 1;
  for (int64_t b = 0; b < n_blocks; ++b) {
    int64_t pg = table[b];
    if (pg < 0 || pg >= n_pages) continue;
    const uint16_t* xb = x + b * rows_per_page * d;
    float A = kvfp4_oracle_group_amax(xb, rows_per_page * d);
    page_amax[pg] = A;
    int rc = kvfp4_oracle_quantize_rows(xb, rows_per_page, d, A, rule,
                                        codes + pg * rows_per_page * (d / 2),
                                        scales + pg * rows_per_page * (d / 16));
    if (rc) return rc;
  }
  return 0;
}

int kvfp4_oracle_dequantize_paged(const uint8_t* codes, const uint8_t* scales,
                                  const float* page_amax, const int32_t* table, int64_t n_blocks,
                                  int64_t rows_per_page, int d, int64_t n_pages, uint16_t* y) {
  if (n_blocks < 0 || rows_per_page <= 0 || d <= 0 || d % 16 != 0) return 1;
  for (int64_t b = 0; b < n_blocks; ++b) {
    int64_t pg = table[b];
    if (pg < 0 || pg >= n_pages) continue;
    int rc = kvfp4_oracle_dequantize_rows(codes + pg * rows_per_page * (d / 2),
                                          scales + pg * rows_per_page * (d / 16), rows_per_page,
                                          d, page_amax[pg], y + b * rows_per_page * d);
    if (rc) return rc;
  }
  return 0;
}

int kvfp4_oracle_dequantize_paged_f32(const uint8_t* codes, const uint8_t* scales,
                                      const float* page_amax, const int32_t* table,
                                      int64_t n_blocks, int64_t rows_per_page, int d,
                                      int64_t n_pages, float* y) {
  if (n_blocks < 0 || rows_per_page <= 0 || d <= 0 || d % 16 != 0) return 1;
  for (int64_t b = 0; b < n_blocks; ++b) {
    int64_t pg = table[b];
    if (pg < 0 || pg >= n_pages) continue;
    int rc = kvfp4_oracle_dequantize_rows_f32(codes + pg * rows_per_page * (d / 2),
                                              scales + pg * rows_per_page * (d / 16),
                                              rows_per_page, d, page_amax[pg],
                                              y + b * rows_per_page * d);
    if (rc) return rc;
  }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Round-to-nearest symmetric blockwise integer quantization.  [P-SF] Table 3 (RTN_INT2,
 * RTN_INT4, RTN_K2_V4, RTN_INT4 RECENT2: symmetric blockwise quantization of K and V,
 * block_size=16, packed storage plus per-block scales; on read the quantized prefix is
 * dequantized and the bf16 recent tail copied back in).
 * Per 16-element block: qmax = 2^(bits-1) - 1; s = bf16(m / qmax) with m = max |x|;
 * inv = s > 0 ? 1/s : 0; q = clamp(nearest-even(x * inv), -qmax, qmax) in two's complement
 * (q = 0 for a zero x, also when inv = inf),
 * element 2j (INT4) or 4j+k (INT2) in the lowest bits first; dequant = bf16(q * s).
 * ---------------------------------------------------------------------------------- */
int kvfp4_oracle_rtn_quantize(const uint16_t* x, int64_t rows, int d, int bits, uint8_t* codes,
                              uint16_t* scales) {
  if (rows < 0 || d <= 0 || d % 16 != 0 || (bits != 2 && bits != 4)) return 1;
  const int qmax = (1 << (bits - 1)) - 1;
  const int per_byte = 8 / bits;
  const int nb = d / 16;
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < nb; ++b) {
      float xb[16];
      float m = 0.0f;
      for (int i = 0; i < 16; ++i) {
        xb[i] = kvfp4_oracle_bf16_to_float(x[r * d + b * 16 + i]);
        if (fabsf(xb[i]) > m) m = fabsf(xb[i]);
      }
      uint16_t sh = kvfp4_oracle_float_to_bf16(m / (float)qmax);
      float sv = kvfp4_oracle_bf16_to_float(sh);
      float inv = (sv > 0.0f) ? 1.0f / sv : 0.0f;
      scales[r * nb + b] = sh;
      for (int i = 0; i < 16; ++i) {
        float v = (xb[i] == 0.0f) ? 0.0f : rintf(xb[i] * inv); /* 0 even if inv = inf */
        if (v > (float)qmax) v = (float)qmax;
        if (v < (float)-qmax) v = (float)-qmax;
        int q = (int)v;
        int e = b * 16 + i;
        uint8_t* byte = &codes[r * (d * bits / 8) + e / per_byte];
        int shift = (e % per_byte) * bits;
        if (shift == 0) *byte = 0;
        *byte |= (uint8_t)((q & ((1 << bits) - 1)) << shift);
      }
    }
  }
  return 0;
}

int kvfp4_oracle_rtn_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t rows, int d,
                                int bits, uint16_t* y) {
  if (rows < 0 || d <= 0 || d % 16 != 0 || (bits != 2 && bits != 4)) return 1;
  const int per_byte = 8 / bits;
  const int nb = d / 16;
  for (int64_t r = 0; r < rows; ++r) {
    for (int e = 0; e < d; ++e) {
      float sv = kvfp4_oracle_bf16_to_float(scales[r * nb + e / 16]);
      int raw = (codes[r * (d * bits / 8) + e / per_byte] >> ((e % per_byte) * bits)) &
                ((1 << bits) - 1);
      int q = (raw >= (1 << (bits - 1))) ? raw - (1 << bits) : raw;
      y[r * d + e] = kvfp4_oracle_float_to_bf16((float)q * sv);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Attention over a dequantized cache.  [P-KV] "CUDA De-quantization Pipeline" (the bf16
 * K/V reconstructed before attention feed the attention operation); [P-SF] Table 3 (the
 * active cache is dequantized to dense BF16 before attention).  The operation itself is
 * the textbook one: O = softmax(scale * Q K^T) V per head, non-causal, here in double,
 * with the double result rounded to bf16 once.
 * Layouts: q [tq, heads, d], k and v [tk, heads, d], all bf16; out [tq, heads, d] bf16.
 * Only the listed (token, head) query rows are computed: rows[i] = token * heads + head.
 * ---------------------------------------------------------------------------------- */
int kvfp4_oracle_attend_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             int64_t tk, int heads, int d, double scale,
                             const int64_t* rows, int64_t n_rows, uint16_t* out,
                             double* scratch /* tk doubles */) {
  if (tk <= 0 || heads <= 0 || d <= 0) return 1;
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t t = rows[i] / heads;
    int h = (int)(rows[i] % heads);
    const uint16_t* qr = q + (t * heads + h) * d;
    double mx = -INFINITY;
    for (int64_t j = 0; j < tk; ++j) {
      const uint16_t* kr = k + (j * heads + h) * d;
      double s = 0.0;
      for (int c = 0; c < d; ++c)
        s += (double)kvfp4_oracle_bf16_to_float(qr[c]) * (double)kvfp4_oracle_bf16_to_float(kr[c]);
      s *= scale;
      scratch[j] = s;
      if (s > mx) mx = s;
    }
    double den = 0.0;
    for (int64_t j = 0; j < tk; ++j) {
      scratch[j] = exp(scratch[j] - mx);
      den += scratch[j];
    }
    for (int c = 0; c < d; ++c) {
      double o = 0.0;
      for (int64_t j = 0; j < tk; ++j)
        o += scratch[j] * (double)kvfp4_oracle_bf16_to_float(v[(j * heads + h) * d + c]);
      out[i * d + c] = kvfp4_oracle_double_to_bf16(o / den);   /* one rounding */
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Array helpers for the tests (element-wise application of the scalar definitions).
 * ---------------------------------------------------------------------------------- */
void kvfp4_oracle_e2m1_encode_n(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)kvfp4_oracle_e2m1_encode(y[i]);
}
void kvfp4_oracle_e4m3_encode_n(const float* u, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)kvfp4_oracle_e4m3_encode(u[i]);
}
void kvfp4_oracle_float_to_bf16_n(const float* f, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvfp4_oracle_float_to_bf16(f[i]);
}
void kvfp4_oracle_double_to_bf16_n(const double* f, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvfp4_oracle_double_to_bf16(f[i]);
}
