// kvfp4_attend.hip -- fused NVFP4 dequantization + attention for MI355X (gfx950).
//
// Pages cited (titles as published):
//   [P-KV]    "How to Use KV Cache Quantization with LongLive's LongLiveQuantizationConfig"
//   [P-SF]    "KV Cache Quantization for Self-Forcing Video Generation: A 33-Method
//              Empirical Study"
//
// [P-KV] "CUDA De-quantization Pipeline" has the packed cache reconstructed to bf16 right
// before attention, and [P-SF] (abstract, Figure 6) finds that materialising those bf16
// buffers is what keeps peak memory high.  This kernel never writes the bf16 cache: each
// workgroup dequantizes a 64-key tile of K and V into LDS (bf16, the same binary32 product
// and rounding as kvfp4_dequantize) and feeds it straight to bf16 MFMA.
//
// Computation: O = softmax(scale * Q K^T) V per head, non-causal, fp32 accumulation and
// an online (running max / running sum) softmax in fp32; P is rounded to bf16 for the
// second product and the row sums are taken over those bf16 weights; O is rounded to bf16.
//
// Mapping (v_mfma_f32_32x32x16_bf16; a lane holds 8 consecutive k of one row of A and of
// one column of B; accumulator register j of lane l is row 8*(j/4) + 4*(l/32) + j%4,
// column l%32):
//   - a workgroup is 8 MFMA waves x 32 queries of one head plus 4 staging waves (one per
//     SIMD) that only dequantize K/V into LDS, so each SIMD always has vector work to issue
//     beside its two MFMA waves; a step covers 64 keys;
//   - S^T = K Q^T: A = K rows from LDS, B = the wave's Q^T held in registers, so each lane
//     ends up owning one query (column) and 32 of the 64 keys of the step; the other 32
//     keys of that query sit in lane l ^ 32, and one exchange combines the two halves
//     (of the final row sum, and of the row max on the rare steps that move it);
//   - O^T = V^T P^T: B = P^T comes straight from the S^T registers (rounded to bf16), so a
//     lane's 8 k values are the keys {0..3, 8..11} + 4 (l / 32) of a 16-key block; A = V^T
//     with the same keys, gathered from the row-major V tile in LDS by two transposing
//     reads (ds_read_b64_tr_b16, 4 keys each);
//   - O^T's columns are queries again, so the softmax rescale is lane-local.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvfp4.h"
#include "kvfp4_device.hpp"

namespace kvfp4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

constexpr int kAtWaves = 8;                  // MFMA + softmax waves per workgroup
constexpr int kAtProdWaves = 4;              // K/V staging waves per workgroup (one per SIMD)
constexpr int kAtThreads = 64 * (kAtWaves + kAtProdWaves);
constexpr int kAtStage = 64 * kAtProdWaves;  // staging threads
constexpr int kAtWaveQ = 32;                 // queries per wave
constexpr int kAtBM = kAtWaveQ * kAtWaves;   // queries per workgroup
constexpr int kAtBN = 64;                    // keys per step

template <int D>
struct AttShape {
  static constexpr int KCH = D / 16;      // 16-wide d chunks of S^T = K Q^T
  static constexpr int DB = D / 32;       // 32-row d blocks of O^T
  static constexpr int UPR = D / 8;       // code dwords per row
  static constexpr int KSTR = D + 8;      // K tile row stride in bf16 (16 B pad: no bank clash)
  static constexpr int VSTR = 160;        // V tile row stride in bf16 (80 dwords: the 4 rows x
                                          // 64 B that 32 lanes of a transposing read touch
                                          // start 16 banks apart, so no bank conflicts)
};

// Per-thread share of one 64-key step among the staging threads (t = 0 .. kAtStage-1): KU
// units of K and the same units of V (u = t + kAtStage r: key u / UPR, d-chunk u % UPR).
// Offsets are byte offsets from the step's first row and are the same for every step
// (32-bit, so the loads take a uniform 64-bit base plus a per-lane 32-bit offset).
// KEXACT / VEXACT: every thread has all its units (no idle lanes), so full steps need no
// per-lane predicate.
template <int D>
struct Share {
  static constexpr int UPR = D / 8;
  static constexpr int KU = (kAtBN * UPR + kAtStage - 1) / kAtStage;
  static constexpr int VU = KU;
  static constexpr bool KEXACT = (kAtBN * UPR) % kAtStage == 0;
  static constexpr bool VEXACT = KEXACT;
  int kkey[KU];            // key index in the step (>= kAtBN: no unit)
  int kj[KU];              // d-chunk
  uint32_t kb[KU];         // code byte offset
  uint32_t ksb[KU];        // scale byte offset
};

template <int D>
__device__ __forceinline__ void make_share(Share<D>& sh, int H, int head) {
  using Sh = Share<D>;
  const int tid = threadIdx.x - 64 * kAtWaves;
#pragma unroll
  for (int r = 0; r < Sh::KU; ++r) {
    const int ui = tid + kAtStage * r;
    const int key = ui < kAtBN * Sh::UPR ? ui / Sh::UPR : kAtBN;
    const int j = ui % Sh::UPR;
    sh.kkey[r] = key;
    sh.kj[r] = j;
    const uint32_t row = (uint32_t)((key < kAtBN ? key : 0) * H + head);
    sh.kb[r] = (row * Sh::UPR + j) * 4u;
    sh.ksb[r] = row * (D / 16) + (j >> 1);
  }
}

// Packed K/V data of one step held in registers between its load and its dequantization.
template <int D>
struct Raw {
  uint32_t kc[Share<D>::KU], ks[Share<D>::KU];
  uint32_t vc[Share<D>::VU], vs[Share<D>::VU];
};

// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family parts: 32-bit data
// format, no swizzle; loads at byte offsets >= the resource's num_records return 0.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRawBufferWord3);
}

// Load the packed data of the step whose first key is t0; `nk` = keys present in the step
// (64 except in the last one).  Each tensor is addressed through a buffer resource that
// spans exactly the step's nk * H rows, so the per-lane 32-bit offsets need no address
// arithmetic, and keys past the end fall outside the resource and read as code 0 / scale
// 0 with no per-lane predicate.
template <int D>
__device__ __forceinline__ void load_raw(Raw<D>& r, const Share<D>& sh, int64_t t0, int nk, int H,
                                         const uint32_t* __restrict__ kcodes,
                                         const uint8_t* __restrict__ kscales,
                                         const uint32_t* __restrict__ vcodes,
                                         const uint8_t* __restrict__ vscales) {
  using Sh = Share<D>;
  const int64_t row0 = t0 * H;
  const uint32_t rows = (uint32_t)nk * (uint32_t)H;
  const auto kc = raw_buffer((const uint8_t*)kcodes + row0 * (D / 2), rows * (D / 2));
  const auto ks = raw_buffer(kscales + row0 * (D / 16), rows * (D / 16));
  const auto vc = raw_buffer((const uint8_t*)vcodes + row0 * (D / 2), rows * (D / 2));
  const auto vs = raw_buffer(vscales + row0 * (D / 16), rows * (D / 16));
#pragma unroll
  for (int i = 0; i < Sh::KU; ++i) {
    r.kc[i] = __builtin_amdgcn_raw_buffer_load_b32(kc, (int)sh.kb[i], 0, 0);
    r.ks[i] = __builtin_amdgcn_raw_buffer_load_b8(ks, (int)sh.ksb[i], 0, 0);
  }
#pragma unroll
  for (int i = 0; i < Sh::VU; ++i) {  // V units at the same offsets as K's
    r.vc[i] = __builtin_amdgcn_raw_buffer_load_b32(vc, (int)sh.kb[i], 0, 0);
    r.vs[i] = __builtin_amdgcn_raw_buffer_load_b8(vs, (int)sh.ksb[i], 0, 0);
  }
}

// Group decode scales (A/2688) of the keys of one step.  With groups of at least kAtBN
// tokens a step holds keys of at most two groups: keys below `split` use d0, the rest d1.
// SHORT (groups shorter than a step) looks every key's group up.
struct StepScales {
  float kd0, kd1, vd0, vd1;
  int split;
};

// Dequantize the step held in `raw` (first key t0) into one LDS buffer pair, K and V both
// row-major [key][d] (one 16 B store per unit).
template <int D, bool SHORT>
__device__ __forceinline__ void stage_tile(const Raw<D>& raw, const Share<D>& sh, int64_t t0,
                                           const StepScales& sc, int64_t tpg, int64_t n_groups,
                                           const float* __restrict__ kamax,
                                           const float* __restrict__ vamax, __bf16* k_buf,
                                           __bf16* v_buf, const float* e4m3_tab) {
  using S = AttShape<D>;
#pragma unroll
  for (int i = 0; i < Share<D>::KU; ++i) {
    const int key = sh.kkey[i];
    if (Share<D>::KEXACT || key < kAtBN) {
      float sd = key < sc.split ? sc.kd0 : sc.kd1;
      if constexpr (SHORT) sd = kamax[min((t0 + key) / tpg, n_groups - 1)] / kGlobalDiv;
      *(uint4*)(k_buf + key * S::KSTR + sh.kj[i] * 8) =
          decode8(raw.kc[i], e4m3_tab[raw.ks[i]] * sd);
    }
  }
#pragma unroll
  for (int i = 0; i < Share<D>::VU; ++i) {
    const int key = sh.kkey[i];
    if (Share<D>::VEXACT || key < kAtBN) {
      float sd = key < sc.split ? sc.vd0 : sc.vd1;
      if constexpr (SHORT) sd = vamax[min((t0 + key) / tpg, n_groups - 1)] / kGlobalDiv;
      *(uint4*)(v_buf + key * S::VSTR + sh.kj[i] * 8) =
          decode8(raw.vc[i], e4m3_tab[raw.vs[i]] * sd);
    }
  }
}

// Tracks the group of the current step's first key as the steps advance, with the decode
// scales of that group and the next (computed only when the group changes; a step of
// kAtBN keys crosses at most one boundary when groups hold at least kAtBN tokens).
struct GroupCursor {
  int64_t g, bnd;            // group of the step's first key, first token of the next group
  float kd0, vd0, kd1, vd1;  // A/2688 of groups g and g+1 (g+1 clamped to the last group)
};

__device__ __forceinline__ void cursor_load(GroupCursor& gc, int64_t n_groups,
                                            const float* __restrict__ kamax,
                                            const float* __restrict__ vamax) {
  const int64_t g1 = gc.g + 1 < n_groups ? gc.g + 1 : gc.g;
  gc.kd0 = kamax[gc.g] / kGlobalDiv;
  gc.vd0 = vamax[gc.g] / kGlobalDiv;
  gc.kd1 = kamax[g1] / kGlobalDiv;
  gc.vd1 = vamax[g1] / kGlobalDiv;
}

template <bool SHORT>
__device__ __forceinline__ StepScales step_scales(GroupCursor& gc, int64_t t0, int64_t tpg,
                                                  int64_t n_groups, const float* __restrict__ kamax,
                                                  const float* __restrict__ vamax) {
  StepScales sc;
  if constexpr (SHORT) {
    sc.kd0 = sc.kd1 = sc.vd0 = sc.vd1 = 0.0f;
    sc.split = kAtBN;
  } else {
    // Steps advance by kAtBN <= tpg: at most one group per step.  (Steps past the end,
    // which the loop stages harmlessly, stay on the last group.)
    if (gc.bnd <= t0 && gc.g + 1 < n_groups) {
      ++gc.g;
      gc.bnd += tpg;
      cursor_load(gc, n_groups, kamax, vamax);
    }
    const bool two = gc.bnd < t0 + kAtBN && gc.g + 1 < n_groups;
    sc.split = two ? (int)(gc.bnd - t0) : kAtBN;
    sc.kd0 = gc.kd0;
    sc.vd0 = gc.vd0;
    sc.kd1 = gc.kd1;
    sc.vd1 = gc.vd1;
  }
  return sc;
}

// Software pipeline over 64-key steps with two LDS buffers: while the MFMA waves run step i
// on buffer i%2, the staging waves dequantize step i+1 (loaded into their registers one step
// earlier) into the other buffer and issue the loads of step i+2; one barrier per step,
// which every wave of both kinds executes.
template <int D, bool SHORT>
__global__ __launch_bounds__(kAtThreads, 1) void attend_kernel(
    const uint16_t* __restrict__ q, int64_t Tq, const uint32_t* __restrict__ kcodes,
    const uint8_t* __restrict__ kscales, const float* __restrict__ kamax,
    const uint32_t* __restrict__ vcodes, const uint8_t* __restrict__ vscales,
    const float* __restrict__ vamax, int64_t Tk, int H, int64_t tpg, int64_t n_groups,
    float qk_scale_log2, uint16_t* __restrict__ out) {
  using S = AttShape<D>;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kAtBN * S::KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kAtBN * S::VSTR];

  const int head = blockIdx.y;
  const int64_t q0 = (int64_t)blockIdx.x * kAtBM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  // Transposing LDS reads: within each 16-lane group, lane r addresses row (key) r / 4 and
  // columns (d) 4 (r % 4) .. +3 of a 4 x 16 block and receives column r of it (checked on
  // the device: lane i gets element i % 4 of the chunks addressed by lanes 4k + i / 4).
  // Group g = lane / 16 covers d 16 (g % 2) .. +15 and keys 4 (g / 2) .. +3; the second read
  // takes the keys 8 further on.
  const int tr_key = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Decoded values of all 256 scale bytes (the dequantizer's own decode; bytes above 0x7E are
  // never written by the quantizers), looked up instead of decoded per unit.
  __shared__ float e4m3_tab[256];
  if (tid < 256) e4m3_tab[tid] = e4m3_decode((uint32_t)tid);
  __syncthreads();

  if (wave >= kAtWaves) {
    // Staging waves: dequantize each step into the buffer the MFMA waves read next; one
    // barrier per step, as the MFMA waves.
    Share<D> sh;
    make_share<D>(sh, H, head);
    GroupCursor gc;
    gc.g = 0;
    gc.bnd = tpg;
    if constexpr (!SHORT) cursor_load(gc, n_groups, kamax, vamax);
    Raw<D> raw;
    const auto keys_in = [&](int64_t t) {
      return (int)(Tk - t >= kAtBN ? kAtBN : (Tk - t > 0 ? Tk - t : 0));
    };
    const auto load = [&](int64_t t) {
      load_raw<D>(raw, sh, t, keys_in(t), H, kcodes, kscales, vcodes, vscales);
    };
    load(0);
    stage_tile<D, SHORT>(raw, sh, 0, step_scales<SHORT>(gc, 0, tpg, n_groups, kamax, vamax),
                         tpg, n_groups, kamax, vamax, k_lds[0], v_lds[0], e4m3_tab);
    load(kAtBN);
    __syncthreads();
    int buf = 0;
    for (int64_t t0 = 0; t0 < Tk; t0 += kAtBN, buf ^= 1) {
      const int64_t t1 = t0 + kAtBN;
      const StepScales sc = step_scales<SHORT>(gc, t1, tpg, n_groups, kamax, vamax);
      stage_tile<D, SHORT>(raw, sh, t1, sc, tpg, n_groups, kamax, vamax, k_lds[buf ^ 1],
                           v_lds[buf ^ 1], e4m3_tab);
      load(t1 + kAtBN);
      __syncthreads();
    }
    return;
  }

  // Q^T operands: query q0 + 32*wave + l32, d = 16*kc + 8*hh .. +7.
  const int64_t qrow = q0 + wave * kAtWaveQ + l32;
  bf16x8 qb[S::KCH];
  {
    const bool ok = qrow < Tq;
    const uint4* qp = (const uint4*)(q + (ok ? (qrow * H + head) * D : 0));
#pragma unroll
    for (int kc = 0; kc < S::KCH; ++kc) {
      const uint4 v = ok ? qp[2 * kc + hh] : make_uint4(0, 0, 0, 0);
      qb[kc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db) o[db] = f32x16{};
  // Running max (base-2 logits) and running sum.  The max is only moved when a weight would
  // exceed 2^8, so most steps skip the rescale of O.
  float m_run = -INFINITY, l_run = 0.0f;

  __syncthreads();  // step 0 staged

  int buf = 0;
  for (int64_t t0 = 0; t0 < Tk; t0 += kAtBN, buf ^= 1) {
    const __bf16* kb = k_lds[buf];
    const __bf16* vb = v_lds[buf];
    // One basic block: S^T = K Q^T for 64 keys (two 32-key row blocks) x the wave's 32
    // queries; the next step dequantized into the other buffer (unconditionally: past the
    // end it stages zeros that nobody reads); the loads of the step after.
    f32x16 s[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      s[rb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < S::KCH; ++kc) {
        const bf16x8 a = *(const bf16x8*)(kb + (32 * rb + l32) * S::KSTR + 16 * kc + 8 * hh);
        s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[kc], s[rb], 0, 0, 0);
      }
    }

    // Online softmax for query l32 in base 2: weights exp2(c s - m) with c = scale*log2(e)
    // > 0 and m the running max of c s.  Keys past Tk (last step only) are masked to -inf.
    if (t0 + kAtBN > Tk) {
      const int nk = (int)(Tk - t0);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = 32 * rb + 8 * (j >> 2) + 4 * hh + (j & 3);
          if (key >= nk) s[rb][j] = -INFINITY;
        }
    }
    // Weights against the current running max, packed to bf16 (the B operand of O^T += V^T
    // P^T), and this lane's share of their sum, accumulated from the same bf16 values with
    // dot2 against (1, 1).
    bf16x8 pb[2][2];
    const auto weights = [&]() {
      float sum = 0.0f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            const float p0 = __builtin_amdgcn_exp2f(
                __builtin_fmaf(s[rb][8 * s2 + i], qk_scale_log2, -m_run));
            const float p1 = __builtin_amdgcn_exp2f(
                __builtin_fmaf(s[rb][8 * s2 + i + 1], qk_scale_log2, -m_run));
            const f32x2 pp = {p0, p1};
            const bf16x2 pk = __builtin_convertvector(pp, bf16x2);
            pb[rb][s2][i] = pk.x;
            pb[rb][s2][i + 1] = pk.y;
            sum = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes2, sum, false);
          }
      return sum;
    };
    float ps = weights();
    // The running max moves (and O and l are rescaled) only when some weight of the wave
    // exceeds 2^8 -- detected from the lane sums, which exceed 2^8 if any term does (and are
    // +inf or NaN on the first step, where the running max is still -inf).  Then the weights
    // are recomputed against the new max.  If a sum exceeds 2^8 the step's max is above the
    // running max, so the max always moves forward.
    if (__builtin_amdgcn_ballot_w64(!(ps <= 256.0f)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[rb][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * qk_scale_log2;
      const float m_new = fmaxf(m_run, mx);  // finite: key t0 < Tk is in this step
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < S::DB; ++db) o[db] *= alpha;
      ps = weights();
    }
    l_run += ps;

    // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int db = 0; db < S::DB; ++db) {
          // A = V^T rows d = 32 db + l32, keys 32 rb + 16 s2 + 4 hh + {0..3, 8..11}, from
          // the row-major V tile by two transposing reads (4 keys each).
          const __bf16* p = vb + (32 * rb + 16 * s2 + tr_key) * S::VSTR + 32 * db + tr_d;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
          const v4i16 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 8 * S::VSTR));
          const bf16x8 a = __builtin_bit_cast(bf16x8, (v8i16){lo[0], lo[1], lo[2], lo[3],
                                                              hi[0], hi[1], hi[2], hi[3]});
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[rb][s2], o[db], 0, 0, 0);
        }
      }
    __syncthreads();  // the other buffer is complete; this one may be overwritten next step
  }

  // O = O^T / l: lane l32 owns query qrow; its d values come four at a time.
  const float inv = 1.0f / (l_run + __shfl_xor(l_run, 32));
  if (qrow < Tq) {
    uint16_t* op = out + (qrow * H + head) * D;
#pragma unroll
    for (int db = 0; db < S::DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * db + 8 * jj + 4 * hh;
        const uint32_t lo = pack_bf16x2(o[db][4 * jj] * inv, o[db][4 * jj + 1] * inv);
        const uint32_t hi = pack_bf16x2(o[db][4 * jj + 2] * inv, o[db][4 * jj + 3] * inv);
        *(uint2*)(op + d0) = make_uint2(lo, hi);
      }
  }
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

int set_last_hip_error(int e);  // defined with the other entry points (kvfp4.hip)

}  // namespace kvfp4

extern "C" int kvfp4_attend(const uint16_t* q, int64_t q_tokens, const uint8_t* k_codes,
                            const uint8_t* k_scales, const float* k_amax, const uint8_t* v_codes,
                            const uint8_t* v_scales, const float* v_amax, int64_t kv_tokens,
                            int32_t heads, int32_t head_dim, int64_t tokens_per_group,
                            float softmax_scale, uint16_t* out, void* stream) {
  using namespace kvfp4;
  if (q_tokens < 0 || kv_tokens < 0 || heads <= 0 || tokens_per_group <= 0 ||
      !isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return KVFP4_EINVAL;
  if (head_dim != 64 && head_dim != 128) return KVFP4_EUNSUPPORTED;
  if (heads > 65535 || (q_tokens + kAtBM - 1) / kAtBM > INT32_MAX ||
      kv_tokens > (INT64_C(1) << 52) / ((int64_t)heads * head_dim) ||
      q_tokens > (INT64_C(1) << 52) / ((int64_t)heads * head_dim))
    return KVFP4_EINVAL;
  if (q_tokens == 0) return KVFP4_OK;
  if (kv_tokens == 0) return KVFP4_EINVAL;  // softmax over no keys is undefined
  if (!q || !k_codes || !k_scales || !k_amax || !v_codes || !v_scales || !v_amax || !out)
    return KVFP4_EINVAL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_scales, 4) || !aligned(v_scales, 4) || !aligned(k_amax, 4) ||
      !aligned(v_amax, 4))
    return KVFP4_EALIGN;
  const int64_t n_groups = (kv_tokens - 1) / tokens_per_group + 1;
  const float qk_scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  const dim3 grid((unsigned)((q_tokens + kAtBM - 1) / kAtBM), (unsigned)heads);
  const bool short_groups = tokens_per_group < kAtBN;
  const hipStream_t st = (hipStream_t)stream;
#define KVFP4_ATTEND_LAUNCH(D_, SHORT_)                                                           \
  hipLaunchKernelGGL((attend_kernel<D_, SHORT_>), grid, dim3(kAtThreads), 0, st, q, q_tokens,     \
                     (const uint32_t*)k_codes, k_scales, k_amax, (const uint32_t*)v_codes,        \
                     v_scales, v_amax, kv_tokens, (int)heads, tokens_per_group, n_groups,         \
                     qk_scale_log2, out)
  if (head_dim == 128) {
    if (short_groups) KVFP4_ATTEND_LAUNCH(128, true);
    else KVFP4_ATTEND_LAUNCH(128, false);
  } else {
    if (short_groups) KVFP4_ATTEND_LAUNCH(64, true);
    else KVFP4_ATTEND_LAUNCH(64, false);
  }
#undef KVFP4_ATTEND_LAUNCH
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVFP4_OK : set_last_hip_error((int)e);
}
