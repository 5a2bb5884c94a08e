/*
 * kvfp4.h -- C ABI of libkvfp4: NVFP4 (E2M1 codes, E4M3 block scales, fp32 group amax)
 * compression of a transformer KV cache on MI355X (gfx950).
 *
 * Pages cited (titles as published):
 *   [P-KV]    "How to Use KV Cache Quantization with LongLive's LongLiveQuantizationConfig"
 *   [P-NVFP4] "How NVFP4 Quantization Works in LongLive 2.0 for Transformer Inference"
 *   [P-SF]    "KV Cache Quantization for Self-Forcing Video Generation: A 33-Method
 *              Empirical Study"
 *
 * Packed format (one "scale group" = rows_per_group consecutive rows, e.g. one appended
 * chunk of K or of V; row = one (token, head) vector of head_dim elements):
 *   codes   uint8  [rows, head_dim/2]   two E2M1 codes per byte, element 2j in the low
 *                                       nibble, 2j+1 in the high nibble; code bit 3 = sign
 *   scales  uint8  [rows, head_dim/16]  one OCP FP8 E4M3 block scale per 16 consecutive
 *                                       elements of a row (0x00..0x7E)
 *   amax    float  [ceil(rows/rows_per_group)]  max |x| of each scale group
 * That is 4.5 bits per element plus 4 bytes per group (3.56x smaller than bf16).
 *
 * Arithmetic (every step one IEEE binary32 operation, round to nearest even):
 *   s_enc = A > 0 ? 2688/A : 0,  s_dec = A/2688          (2688 = e2m1_max 6 * e4m3_max 448)
 *   per 16-element block with m = max|x|, for divisor Dv (6 for static_6, 4 for static_4):
 *     sf = E4M3_RNE_SAT((m/Dv) * s_enc),  S = E4M3(sf) * s_dec,  inv = S > 0 ? 1/S : 0
 *     code_i = sign(x_i*inv) | E2M1_RNE_SAT(|x_i*inv|)   (ties to even, saturate at 6)
 *   mse: both candidates; err = fma-chain of (x_i - E2M1(c_i)*S)^2 over elements 0..7 plus
 *        the chain over 8..15; the 4-max candidate wins only if its err is strictly lower.
 *   dequantize: y_i = bf16_rne(E2M1(c_i) * (E4M3(sf) * (A/2688)))
 *   a product with a zero operand is zero, also where binary32 would form 0*inf = NaN (a
 *   group amax below about 2^-119 overflows s_enc or inv): an all-zero block gets scale
 *   byte 0x00, a zero element code 0x0 / 0x8 by its sign; nonzero x*inf saturates.
 *   Inputs must be finite; every finite input is in the domain.
 *
 * Conventions for every entry point:
 *   - pointers are DEVICE pointers unless stated; the caller allocates and frees all of
 *     them; the library never allocates, never synchronizes, keeps no mutable state besides
 *     a thread-local copy of the last HIP error (everything a call needs arrives with the
 *     call), and is reentrant across streams and threads;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); work is only
 *     enqueued, the call returns before it runs;
 *   - argument errors are detected on the host and returned before anything is enqueued;
 *     rows == 0 (or q_tokens == 0) is a no-op that returns KVFP4_OK;
 *   - inputs and outputs must not overlap (kvfp4_fake_quantize alone allows y == x);
 *   - no C++ exception crosses the ABI.
 */
#ifndef KVFP4_H
#define KVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVFP4_ABI_VERSION 2

/* Status codes returned by every entry point. */
enum kvfp4_status {
  KVFP4_OK = 0,
  KVFP4_EINVAL = 1,      /* null pointer with work to do, negative size, rows_per_group <= 0,
                            unknown rule, size overflow */
  KVFP4_EALIGN = 2,      /* a pointer is not aligned as its argument requires */
  KVFP4_EUNSUPPORTED = 3,/* head_dim not a multiple of 64 in [64, 1024] (attend: 64 or 128) */
  KVFP4_EHIP = 4         /* a kernel launch failed; kvfp4_last_hip_error() has the code;
                            outputs are undefined */
};

/* Block-scale rules: [P-KV] "Programmatic Configuration" and "Configuration Parameters
 * Reference" (static_6 default; static_4 and mse alternatives). */
enum kvfp4_rule {
  KVFP4_RULE_STATIC6 = 0, /* block amax mapped to 6: scale = amax/6 ([P-NVFP4] "Understanding
                             the NVFP4 Format and Architecture") */
  KVFP4_RULE_STATIC4 = 1, /* block amax mapped to 4 */
  KVFP4_RULE_MSE = 2      /* per block, whichever of the two has the lower squared error */
};

/*
 * kvfp4_quantize -- quantize-on-append of K or V blocks.
 * [P-KV] "FP4 Quantization in the Causal Model" (each key and value block is compressed
 * independently on write); [P-NVFP4] "Stage 1" (per-block amax, per-block scale, two codes
 * per uint8, one global amax per tensor) and "Stage 3" (global scale formula);
 * [P-SF] Table 3 (blockwise, block size 16, quantize on write).
 *
 *   x               bf16 bit patterns [rows, head_dim], row-major; 16-byte aligned
 *   rows            number of rows (>= 0)
 *   head_dim        elements per row: a multiple of 64 in [64, 1024]
 *   rows_per_group  rows per scale group (> 0); group g = rows [g*rpg, min((g+1)*rpg, rows))
 *   rule            enum kvfp4_rule
 *   codes   (out)   uint8 [rows, head_dim/2]; 16-byte aligned
 *   scales  (out)   uint8 [rows, head_dim/16]; 4-byte aligned
 *   group_amax (out) float [ceil(rows/rows_per_group)]; 4-byte aligned
 * Appending a chunk to a cache = passing pointers offset to the chunk's first row and
 * group.  Inputs must be finite.  Enqueues three kernels: for inputs of at least 40 MiB
 * (80 MiB under mse) whose every group (the last one included) has at least 528 elements, a
 * hand-off clear, one kernel that computes the group amax and encodes (it borrows three
 * dwords of each group's codes for the hand-off; the codes are complete when the call's work
 * ends), and a finish kernel; otherwise amax clear, group amax, encode.  Both give the same bytes.  (These are the default options of
 * kvfp4_quantize_ex, below.)
 */
int kvfp4_quantize(const uint16_t* x, int64_t rows, int32_t head_dim, int64_t rows_per_group,
                   int32_t rule, uint8_t* codes, uint8_t* scales, float* group_amax,
                   void* stream);

/*
 * kvfp4_dequantize -- reconstruct bf16 K/V from the packed cache before attention.
 * [P-KV] "CUDA De-quantization Pipeline" (bf16 reconstruction of the cache before
 * attention); [P-NVFP4] "Stage 3" (each byte expands to two 4-bit values multiplied by the
 * per-block and the global scale; bf16 output); [P-SF] Table 3 (the active cache is
 * dequantized back to dense BF16 before attention).
 *
 *   codes, scales, group_amax   as written by kvfp4_quantize (same alignment rules)
 *   rows, head_dim, rows_per_group   as for kvfp4_quantize
 *   y      (out)   bf16 bit patterns [rows, head_dim]; 16-byte aligned
 * One kernel launch for any number of rows and groups (64-bit indexing).
 */
int kvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* group_amax,
                     int64_t rows, int32_t head_dim, int64_t rows_per_group, uint16_t* y,
                     void* stream);

/*
 * kvfp4_attend -- attention over the packed cache, dequantizing K and V on chip.
 * [P-KV] "CUDA De-quantization Pipeline" (K/V reconstructed to bf16 for the attention
 * operation); [P-SF] abstract and Figure 6 (the bf16 reconstruction buffers are what keep
 * peak memory high -- here they never exist).
 *
 *   O[t, h, :] = sum_j softmax_j(softmax_scale * <Q[t, h, :], K[j, h, :]>) V[j, h, :]
 * per head h, non-causal, where K and V are the dequantized packed caches (exactly the
 * bf16 values kvfp4_dequantize would produce).  Scores, softmax and accumulation are fp32
 * (bf16 MFMA inputs; the softmax weights are rounded to bf16 for the second product, and
 * the row sums are taken over those same bf16 weights); the output is rounded to bf16.
 *
 *   q                 bf16 [q_tokens, heads, head_dim]; 16-byte aligned
 *   k_codes, v_codes  uint8 [kv_tokens, heads, head_dim/2]; 16-byte aligned
 *   k_scales, v_scales uint8 [kv_tokens, heads, head_dim/16]; 4-byte aligned
 *   k_amax, v_amax    float [ceil(kv_tokens / tokens_per_group)]; 4-byte aligned
 *                     (the packed layout kvfp4_quantize writes with
 *                      rows_per_group = tokens_per_group * heads)
 *   kv_tokens         > 0 when q_tokens > 0
 *   heads             1..65535
 *   head_dim          64 or 128
 *   softmax_scale     finite and > 0, typically 1/sqrt(head_dim)
 *   out (out)         bf16 [q_tokens, heads, head_dim]; 16-byte aligned
 * One kernel launch; no workspace.
 */
int kvfp4_attend(const uint16_t* q, int64_t q_tokens, const uint8_t* k_codes,
                 const uint8_t* k_scales, const float* k_amax, const uint8_t* v_codes,
                 const uint8_t* v_scales, const float* v_amax, int64_t kv_tokens, int32_t heads,
                 int32_t head_dim, int64_t tokens_per_group, float softmax_scale, uint16_t* out,
                 void* stream);

/*
 * Paged cache.  [P-NVFP4] "Code Implementation" / "Runtime KV-Cache De-quantization"
 * (dequantize_kv_cache over a list of cache blocks with max_blocks, num_heads and
 * block_token_size) and "Stage 3" (output reshaped to [block_token_size, num_heads, head_dim]).
 *
 * The packed cache is an array of physical pages; a page holds rows_per_page rows
 * (block_token_size tokens x heads) and is its own scale group:
 *   codes      uint8 [n_pages, rows_per_page, head_dim/2]; 16-byte aligned
 *   scales     uint8 [n_pages, rows_per_page, head_dim/16]; 4-byte aligned
 *   page_amax  float [n_pages]; 4-byte aligned
 *   block_table int32 [n_blocks] (device): logical block b lives in page block_table[b];
 *              entries outside [0, n_pages) are skipped (nothing is read or written for
 *              that block); 4-byte aligned
 * The dense side is [n_blocks * rows_per_page, head_dim] bf16, block-major (block b = rows
 * [b*rows_per_page, (b+1)*rows_per_page)); 16-byte aligned.
 *
 * kvfp4_quantize_paged: quantize the dense rows block by block into their pages (group amax
 * = the block's amax, stored in page_amax[page]), with the same kernels as kvfp4_quantize
 * (in the one-kernel form the hand-off words sit in each named page's codes).  Two blocks
 * naming the same page race.
 * kvfp4_dequantize_paged: gather the listed pages into dense bf16 rows; a page may be named
 * more than once.  Same arithmetic, errors and stream rules as the unpaged calls.
 */
int kvfp4_quantize_paged(const uint16_t* x, int64_t n_blocks, int64_t rows_per_page,
                         int32_t head_dim, int32_t rule, const int32_t* block_table,
                         int64_t n_pages, uint8_t* codes, uint8_t* scales, float* page_amax,
                         void* stream);
int kvfp4_dequantize_paged(const uint8_t* codes, const uint8_t* scales, const float* page_amax,
                           const int32_t* block_table, int64_t n_blocks, int64_t rows_per_page,
                           int32_t head_dim, int64_t n_pages, uint16_t* y, void* stream);

/*
 * Float32 output and fake quantization.  [P-NVFP4] "Stage 3" (the dequantize kernel emits
 * float32 or bf16) and "Stage 1" (the fake-quant form of the block-scale path, where a
 * 16-bit tensor carries exactly the values the 4-bit one represents).
 *
 * kvfp4_dequantize_f32 / kvfp4_dequantize_paged_f32: as kvfp4_dequantize /
 * kvfp4_dequantize_paged, but y receives the binary32 products E2M1(c) * S with
 * S = E4M3(sf) * (A/2688) -- the values whose bf16 rounding the bf16 calls return.
 *   y (out) float [rows, head_dim] (paged: [n_blocks * rows_per_page, head_dim]); 16-byte
 *           aligned.
 *
 * kvfp4_fake_quantize: quantize x exactly as kvfp4_quantize does (same rule, groups and
 * group_amax output) and write dequantize(quantize(x)) in bf16 to y, bit-identical to
 * calling the two, without storing codes or scale bytes.
 *   x, rows, head_dim, rows_per_group, rule   as for kvfp4_quantize
 *   group_amax (out) float [ceil(rows/rows_per_group)]; 4-byte aligned
 *   y (out)    bf16 [rows, head_dim]; 16-byte aligned; y == x (in place) is allowed, any
 *              other overlap is undefined.
 * Errors, alignment and stream rules as for the calls above.
 */
int kvfp4_dequantize_f32(const uint8_t* codes, const uint8_t* scales, const float* group_amax,
                         int64_t rows, int32_t head_dim, int64_t rows_per_group, float* y,
                         void* stream);
int kvfp4_dequantize_paged_f32(const uint8_t* codes, const uint8_t* scales,
                               const float* page_amax, const int32_t* block_table,
                               int64_t n_blocks, int64_t rows_per_page, int32_t head_dim,
                               int64_t n_pages, float* y, void* stream);
int kvfp4_fake_quantize(const uint16_t* x, int64_t rows, int32_t head_dim, int64_t rows_per_group,
                        int32_t rule, float* group_amax, uint16_t* y, void* stream);

/*
 * Round-to-nearest symmetric blockwise integer quantization (INT4 or INT2) -- the RTN
 * baselines of [P-SF] Table 3: RTN_INT4, RTN_INT2, RTN_K2_V4 (2-bit keys, 4-bit values: two
 * calls with different `bits`) and RTN_INT4 RECENT2 (the newest frame-blocks stay bf16 and
 * are copied back behind the dequantized prefix on read: `tail`).
 *
 * Per 16-element block along head_dim: qmax = 2^(bits-1) - 1 (7 or 1), s = bf16_rne(m/qmax)
 * with m = max|x| (binary32 division), inv = s > 0 ? 1/s : 0, q = clamp(rne(x*inv), -qmax,
 * qmax) (q = 0 for x = +-0 also when inv = inf) stored as a two's-complement bit field, element 8k+i at bits [bits*i, bits*(i+1)) of
 * its 8-element group (INT4: element 2j in the low nibble of byte j; INT2: element 4j+k at
 * bits 2k of byte j); dequant = bf16_rne(q * s).  No group amax.  One 16-bit scale per 16
 * elements: 5 bits/element (INT4), 3 bits/element (INT2, the 5.33x of [P-SF] Tables 4-5).
 *
 *   x       bf16 [rows, head_dim]; 16-byte aligned
 *   bits    2 or 4 (else KVFP4_EINVAL)
 *   codes   uint8 [rows, head_dim*bits/8]; 16-byte aligned
 *   scales  bf16 bit patterns [rows, head_dim/16]; 4-byte aligned
 *   tail    bf16 [tail_rows, head_dim] copied verbatim after the dequantized rows (may be
 *           NULL when tail_rows == 0); 16-byte aligned
 *   y (out) bf16 [rows + tail_rows, head_dim]; 16-byte aligned
 */
int kvfp4_rtn_quantize(const uint16_t* x, int64_t rows, int32_t head_dim, int32_t bits,
                       uint8_t* codes, uint16_t* scales, void* stream);
int kvfp4_rtn_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t rows,
                         int32_t head_dim, int32_t bits, const uint16_t* tail, int64_t tail_rows,
                         uint16_t* y, void* stream);

/* Host-side size helper: bytes of codes and scales and the number of group amax floats
 * for a tensor of `rows` rows.  Returns KVFP4_EINVAL / KVFP4_EUNSUPPORTED like the calls
 * above.  Any output pointer may be NULL. */
int kvfp4_packed_sizes(int64_t rows, int32_t head_dim, int64_t rows_per_group,
                       int64_t* codes_bytes, int64_t* scales_bytes, int64_t* n_groups);

/*
 * Per-call quantize options: how kvfp4_quantize_ex, kvfp4_quantize_paged_ex and
 * kvfp4_fake_quantize_ex enqueue their work.  They never change an output byte.  [P-KV]
 * "Programmatic Configuration" carries its settings in a configuration object handed to the
 * call that uses them; these options travel the same way (no process-wide settings).
 *   form     KVFP4_FORM_ONE_KERNEL: one kernel computes the group amax and encodes wherever
 *            that applies (not in place, every group -- the last one included -- at least
 *            528 elements, 32-bit grid); otherwise three kernels (clear the amax words,
 *            group amax, encode).  KVFP4_FORM_THREE_KERNEL: always three kernels.
 *            KVFP4_FORM_AUTO (the default): the one-kernel form where it applies and the
 *            call's input holds at least 40 MiB of bf16 (80 MiB under the mse rule), else
 *            three kernels -- the measured crossover: below it the three passes, each at
 *            full parallelism, finish first.
 *   wait_us  in the one-kernel form, the longest time in microseconds an encode workgroup
 *            waits for its group amax before it computes the amax itself from the input
 *            (the same value); 0 = never wait; default 20000; at most 60000000.
 * opts == NULL means the defaults, which is what the calls without the _ex suffix use.  An
 * unknown form or a wait_us out of range returns KVFP4_EINVAL before anything is enqueued.
 * The struct is read during the call only (host memory, owned by the caller).
 */
enum kvfp4_form {
  KVFP4_FORM_AUTO = 0,
  KVFP4_FORM_THREE_KERNEL = 1,
  KVFP4_FORM_ONE_KERNEL = 2
};
struct kvfp4_quantize_opts {
  int32_t form;     /* enum kvfp4_form */
  int64_t wait_us;  /* 0 .. 60000000 */
};
#define KVFP4_QUANTIZE_OPTS_DEFAULT {KVFP4_FORM_AUTO, 20000}

/* kvfp4_quantize, kvfp4_quantize_paged and kvfp4_fake_quantize with explicit options (same
 * arguments otherwise, same results). */
int kvfp4_quantize_ex(const uint16_t* x, int64_t rows, int32_t head_dim, int64_t rows_per_group,
                      int32_t rule, uint8_t* codes, uint8_t* scales, float* group_amax,
                      const struct kvfp4_quantize_opts* opts, void* stream);
int kvfp4_quantize_paged_ex(const uint16_t* x, int64_t n_blocks, int64_t rows_per_page,
                            int32_t head_dim, int32_t rule, const int32_t* block_table,
                            int64_t n_pages, uint8_t* codes, uint8_t* scales, float* page_amax,
                            const struct kvfp4_quantize_opts* opts, void* stream);
int kvfp4_fake_quantize_ex(const uint16_t* x, int64_t rows, int32_t head_dim,
                           int64_t rows_per_group, int32_t rule, float* group_amax, uint16_t* y,
                           const struct kvfp4_quantize_opts* opts, void* stream);

/* Diagnostics. */
const char* kvfp4_status_str(int status); /* static string, never NULL */
int kvfp4_abi_version(void);              /* KVFP4_ABI_VERSION */
int kvfp4_last_hip_error(void);           /* hipError_t of this thread's last failed launch */

#ifdef __cplusplus
}
#endif

#endif /* KVFP4_H */
