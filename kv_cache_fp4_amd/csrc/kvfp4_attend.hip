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
// second product; O is rounded to bf16.
//
// Mapping (v_mfma_f32_32x32x16_bf16; a lane holds 8 consecutive k of one row of A and of
// one column of B; accumulator register j of lane l is row 8*(j/4) + 4*(l/32) + j%4,
// column l%32):
//   - a workgroup is 8 waves x 32 queries of one head; a step covers 64 keys;
//   - S^T = K Q^T: A = K rows from LDS, B = the wave's Q^T held in registers, so each lane
//     ends up owning one query (column) and 32 of the 64 keys of the step; the other 32
//     keys of that query sit in lane l ^ 32, one exchange gives the row max / row sum;
//   - O^T = V^T P^T: B = P^T comes straight from the S^T registers (rounded to bf16), A =
//     V^T read from LDS, where V is stored transposed with bits 2 and 3 of the key index
//     swapped inside each 16-key block so that the 8 keys a lane needs are contiguous;
//   - O^T's columns are queries again, so the softmax rescale is lane-local.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvfp4.h"
#include "kvfp4_device.hpp"

namespace kvfp4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAtWaves = 8;                  // waves per workgroup (2 per SIMD)
constexpr int kAtThreads = 64 * kAtWaves;
constexpr int kAtWaveQ = 32;                 // queries per wave
constexpr int kAtBM = kAtWaveQ * kAtWaves;   // queries per workgroup
constexpr int kAtBN = 64;                    // keys per step

template <int D>
struct AttShape {
  static constexpr int KCH = D / 16;      // 16-wide d chunks of S^T = K Q^T
  static constexpr int DB = D / 32;       // 32-row d blocks of O^T
  static constexpr int UPR = D / 8;       // code dwords per row
  static constexpr int KSTR = D + 8;      // K tile row stride in bf16 (16 B pad: no bank clash)
  static constexpr int VSTR = kAtBN + 8;  // V^T tile row stride in bf16
};

// Position of key r (0..15) inside its 16-key block of the V^T tile: bits 2 and 3 swapped.
__device__ __forceinline__ int vperm(int r) { return (r & 3) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Raw (still packed) K/V data of one 64-key step held by one thread: KU units of K
// (key = u / UPR, d-chunk = u % UPR for u = tid + kAtThreads * r) and VU pairs of
// consecutive V keys of one d-chunk (pair p = tid + kAtThreads * r: d-chunk p / 32, keys
// 2 (p % 32) and 2 (p % 32) + 1).
template <int D>
struct Raw {
  static constexpr int KU = (kAtBN * (D / 8) + kAtThreads - 1) / kAtThreads;
  static constexpr int VU = ((kAtBN / 2) * (D / 8) + kAtThreads - 1) / kAtThreads;
  uint32_t kc[KU], ks[KU];
  uint32_t vc[VU][2], vs[VU][2];
};

template <int D>
__device__ __forceinline__ void load_raw(Raw<D>& r, int64_t t0, int64_t Tk, int H, int head,
                                         const uint32_t* __restrict__ kcodes,
                                         const uint8_t* __restrict__ kscales,
                                         const uint32_t* __restrict__ vcodes,
                                         const uint8_t* __restrict__ vscales) {
  using S = AttShape<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int r_ = 0; r_ < Raw<D>::KU; ++r_) {
    const int ui = tid + kAtThreads * r_;
    const int key = ui / S::UPR, j = ui % S::UPR;
    const int64_t t = t0 + key;
    const bool ok = ui < kAtBN * S::UPR && t < Tk;
    const int64_t row = t * H + head;
    r.kc[r_] = ok ? kcodes[row * S::UPR + j] : 0u;
    r.ks[r_] = ok ? (uint32_t)kscales[row * (D / 16) + (j >> 1)] : 0u;
  }
#pragma unroll
  for (int r_ = 0; r_ < Raw<D>::VU; ++r_) {
    const int pi = tid + kAtThreads * r_;
    const int j = pi / (kAtBN / 2), kp = pi % (kAtBN / 2);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int64_t t = t0 + 2 * kp + kk;
      const bool ok = pi < (kAtBN / 2) * S::UPR && t < Tk;
      const int64_t row = t * H + head;
      r.vc[r_][kk] = ok ? vcodes[row * S::UPR + j] : 0u;
      r.vs[r_][kk] = ok ? (uint32_t)vscales[row * (D / 16) + (j >> 1)] : 0u;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kAtThreads, 1) void attend_kernel(
    const uint16_t* __restrict__ q, int64_t Tq, const uint32_t* __restrict__ kcodes,
    const uint8_t* __restrict__ kscales, const float* __restrict__ kamax,
    const uint32_t* __restrict__ vcodes, const uint8_t* __restrict__ vscales,
    const float* __restrict__ vamax, int64_t Tk, int H, int64_t tpg, int64_t n_groups,
    float qk_scale_log2, uint16_t* __restrict__ out) {
  using S = AttShape<D>;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[kAtBN * S::KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[D * S::VSTR];

  const int head = blockIdx.y;
  const int64_t q0 = (int64_t)blockIdx.x * kAtBM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

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
  // Running max (base-2 logits) and running sum.  The max is only moved when a new score
  // exceeds it by more than 8, so most steps skip the rescale of O; weights stay <= 2^8.
  float m_run = -INFINITY, l_run = 0.0f;
  const bool short_groups = tpg < kAtBN;

  Raw<D> raw;
  load_raw<D>(raw, 0, Tk, H, head, kcodes, kscales, vcodes, vscales);

  for (int64_t t0 = 0; t0 < Tk; t0 += kAtBN) {
    // Group decode scales of this step's keys: a step crosses at most one group boundary
    // when groups are at least kAtBN tokens long; shorter groups look each key up.
    const int64_t g0 = t0 / tpg;
    const int64_t bnd = (g0 + 1) * tpg;
    const bool two = bnd < t0 + kAtBN && g0 + 1 < n_groups;
    const float kd0 = kamax[g0] / kGlobalDiv, vd0 = vamax[g0] / kGlobalDiv;
    const float kd1 = two ? kamax[g0 + 1] / kGlobalDiv : kd0;
    const float vd1 = two ? vamax[g0 + 1] / kGlobalDiv : vd0;

    __syncthreads();  // the previous step's LDS reads are done
    // K tile -> LDS, row-major [key][d]: 16 B per unit.
#pragma unroll
    for (int r_ = 0; r_ < Raw<D>::KU; ++r_) {
      const int ui = tid + kAtThreads * r_;
      if (ui < kAtBN * S::UPR) {
        const int key = ui / S::UPR, j = ui % S::UPR;
        const int64_t t = t0 + key;
        const float sd = short_groups ? (t < Tk ? kamax[t / tpg] / kGlobalDiv : 0.0f)
                                      : (t < bnd ? kd0 : kd1);
        *(uint4*)(k_lds + key * S::KSTR + j * 8) = decode8(raw.kc[r_], e4m3_decode(raw.ks[r_]) * sd);
      }
    }
    // V tile -> LDS transposed [d][key'], two consecutive keys per thread so that each d
    // row gets one 4-byte write; key' = vperm order inside 16-key blocks (keeps pairs).
#pragma unroll
    for (int r_ = 0; r_ < Raw<D>::VU; ++r_) {
      const int pi = tid + kAtThreads * r_;
      if (pi < (kAtBN / 2) * S::UPR) {
        const int j = pi / (kAtBN / 2), kp = pi % (kAtBN / 2);
        uint4 w[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int64_t t = t0 + 2 * kp + kk;
          const float sd = short_groups ? (t < Tk ? vamax[t / tpg] / kGlobalDiv : 0.0f)
                                        : (t < bnd ? vd0 : vd1);
          w[kk] = decode8(raw.vc[r_][kk], e4m3_decode(raw.vs[r_][kk]) * sd);
        }
        const int pos = (2 * kp & ~15) | vperm((2 * kp) & 15);
        const uint32_t* w0 = &w[0].x;
        const uint32_t* w1 = &w[1].x;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {  // d = 8 j + 2 i2 and 8 j + 2 i2 + 1
          *(uint32_t*)(v_lds + (8 * j + 2 * i2) * S::VSTR + pos) =
              (w0[i2] & 0xFFFFu) | (w1[i2] << 16);
          *(uint32_t*)(v_lds + (8 * j + 2 * i2 + 1) * S::VSTR + pos) =
              (w0[i2] >> 16) | (w1[i2] & 0xFFFF0000u);
        }
      }
    }
    __syncthreads();
    // Fetch the next step's packed K/V now; the loads complete while this step computes.
    if (t0 + kAtBN < Tk) load_raw<D>(raw, t0 + kAtBN, Tk, H, head, kcodes, kscales, vcodes, vscales);

    // S^T = K Q^T for 64 keys (two 32-key row blocks) x the wave's 32 queries.
    f32x16 s[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      s[rb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < S::KCH; ++kc) {
        const bf16x8 a = *(const bf16x8*)(k_lds + (32 * rb + l32) * S::KSTR + 16 * kc + 8 * hh);
        s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[kc], s[rb], 0, 0, 0);
      }
    }
    // Online softmax for query l32 in base 2: weights exp2(c s - m) with c = scale*log2(e)
    // > 0, so the max is taken on the raw scores and scaled once.  Keys past Tk (last step
    // only) are masked to -inf.
    float mx = -INFINITY;
    if (t0 + kAtBN > Tk) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = 32 * rb + 8 * (j >> 2) + 4 * hh + (j & 3);
          if (t0 + key >= Tk) s[rb][j] = -INFINITY;
        }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[rb][j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * qk_scale_log2;
    // Move the running max (and rescale O and l) only when some query of the wave needs it.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, mx);  // finite: key t0 < Tk is in this step
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < S::DB; ++db) o[db] *= alpha;
    }
    float ps = 0.0f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][j], qk_scale_log2, -m_run));
        s[rb][j] = p;
        ps += p;
      }
    l_run += ps;

    // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (__bf16)s[rb][8 * s2 + i];
#pragma unroll
        for (int db = 0; db < S::DB; ++db) {
          const bf16x8 a = *(const bf16x8*)(v_lds + (32 * db + l32) * S::VSTR + 32 * rb +
                                            16 * s2 + 8 * hh);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[db], 0, 0, 0);
        }
      }
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
  if (head_dim == 128)
    hipLaunchKernelGGL(attend_kernel<128>, grid, dim3(kAtThreads), 0, (hipStream_t)stream, q,
                       q_tokens, (const uint32_t*)k_codes, k_scales, k_amax,
                       (const uint32_t*)v_codes, v_scales, v_amax, kv_tokens, (int)heads,
                       tokens_per_group, n_groups, qk_scale_log2, out);
  else
    hipLaunchKernelGGL(attend_kernel<64>, grid, dim3(kAtThreads), 0, (hipStream_t)stream, q,
                       q_tokens, (const uint32_t*)k_codes, k_scales, k_amax,
                       (const uint32_t*)v_codes, v_scales, v_amax, kv_tokens, (int)heads,
                       tokens_per_group, n_groups, qk_scale_log2, out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVFP4_OK : set_last_hip_error((int)e);
}
