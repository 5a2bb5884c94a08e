// kvfp4.hip -- libkvfp4: NVFP4 KV-cache quantize / dequantize kernels for MI355X (gfx950)
// and their C ABI (declared in include/kvfp4.h).
//
// Pages cited (titles as published):
//   [P-KV]    "How to Use KV Cache Quantization with LongLive's LongLiveQuantizationConfig"
//   [P-NVFP4] "How NVFP4 Quantization Works in LongLive 2.0 for Transformer Inference"
//   [P-SF]    "KV Cache Quantization for Self-Forcing Video Generation: A 33-Method
//              Empirical Study"
//
// Work decomposition.  All three streaming kernels see a tensor as a flat sequence of
// 8-element "units" (16 B of bf16, 4 B of codes, half a 16-element scale block).  A scale
// group (rows_per_group rows) is a contiguous run of units, and the grid is
// n_groups x slices_per_group workgroups: workgroup (g, s) owns a contiguous slice of
// group g.  Every workgroup therefore has one group amax, read once into a uniform
// register, and never needs a per-lane division to find its group.  Inside a slice each
// wave of 64 lanes takes 64*UNR consecutive units per step; the k-th load/store of a step
// covers 64 consecutive units, so every wave instruction touches one contiguous span
// (1 KiB of bf16, 256 B of codes, 32 B of scales).  Index math is 64-bit throughout.
//
// Quantize (per [P-NVFP4] "Stage 1"): (1) clear the group amax words, (2) group amax by a
// max over 15-bit bf16 magnitude patterns, one atomicMax per workgroup, (3) encode: two
// lanes per 16-element block exchange their half-block amax through DPP, both derive the
// same E4M3 scale, and each packs its 8 codes into one dword.
// Dequantize (per [P-NVFP4] "Stage 3"): one pass, each lane turns one code dword and one
// scale byte into 8 bf16 (one 16 B store).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvfp4.h"
#include "kvfp4_device.hpp"

namespace kvfp4 {
namespace {

constexpr int kThreads = 256;           // amax / encode workgroups: 4 waves of 64
constexpr int kWaves = kThreads / 64;
constexpr int kQuantUnroll = 2;
constexpr int kAmaxUnroll = 4;
constexpr int64_t kTargetWorkgroups = 4096;  // 16 per CU on 256 CUs

// Dequantize: many short workgroups of 2 waves, each wave writing one contiguous 2 KiB
// run (2 x 1 KiB stores per lane group) with non-temporal stores.  Workgroups are
// dispatched in index order, so the set of addresses being written at any moment is a
// compact window of the output; measured on MI355X this beats persistent or longer
// workgroups by 10-40% on the 7.7 GB whole-cache read (6.6 TB/s vs 4.6-6.0 TB/s).
constexpr int kDqThreads = 128;
constexpr int kDqUnroll = 2;
constexpr int64_t kDqTileUnits = kDqThreads * kDqUnroll;  // 256 units = 2048 elements

// Flat partition of a tensor into (group, slice) workgroups; sizes in 8-element units.
struct Part {
  int64_t units_total;
  int64_t units_per_group;
  int64_t slice_units;
  uint32_t slices_per_group;
};

struct Range {
  int64_t beg, end;
  uint32_t g;
};

__device__ __forceinline__ Range wg_range(const Part& p) {
  Range r;
  r.g = blockIdx.x / p.slices_per_group;
  const uint32_t s = blockIdx.x - r.g * p.slices_per_group;
  const int64_t gbeg = (int64_t)r.g * p.units_per_group;
  const int64_t gend = min(gbeg + p.units_per_group, p.units_total);
  r.beg = gbeg + (int64_t)s * p.slice_units;
  r.end = min(r.beg + p.slice_units, gend);
  return r;
}

// Value from the partner lane (lane ^ 1) through DPP quad_perm [1,0,3,2].
__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float swap_pair(float v) {
  return __uint_as_float(swap_pair(__float_as_uint(v)));
}

// ---- kernel 1: clear group amax ---------------------------------------------------------
__global__ __launch_bounds__(kThreads) void clear_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = 0u;
}

// ---- kernel 2: group amax ([P-NVFP4] "Stage 1", global amax scalar) ---------------------
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint4* __restrict__ x,
                                                        uint32_t* __restrict__ amax_bits, Part p) {
  const Range r = wg_range(p);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t mx = 0;
  for (int64_t base = r.beg + wave * 64 * kAmaxUnroll; base < r.end;
       base += kWaves * 64 * kAmaxUnroll) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int k = 0; k < kAmaxUnroll; ++k) {
      const int64_t u = base + k * 64 + lane;
      v[k] = (u < r.end) ? x[u] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kAmaxUnroll; ++k) mx = max(mx, absmax8_bits(v[k]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  __shared__ uint32_t red[kWaves];
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0 && r.beg < r.end) {
    uint32_t m = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = max(m, red[w]);
    // A non-negative binary32 orders like its bit pattern; bf16 -> fp32 is a 16-bit shift.
    atomicMax(&amax_bits[r.g], m << 16);
  }
}

// ---- kernel 3: encode ([P-NVFP4] "Stage 1"; [P-KV] scale rules) -------------------------

// One candidate scaling of a block for this lane's 8 elements.
struct Cand {
  uint32_t sf;     // E4M3 byte
  float S;         // decoded block scale * s_dec
  uint32_t codes;  // 8 packed E2M1 codes
};

__device__ __forceinline__ Cand make_cand(const float xf[8], float m, float dv, float s_enc,
                                          float s_dec) {
  Cand c;
  const float t = m / dv;   // IEEE division (correctly rounded)
  const float u = t * s_enc;
  c.sf = e4m3_encode(u);
  c.S = e4m3_decode(c.sf) * s_dec;
  const float inv = (c.S > 0.0f) ? 1.0f / c.S : 0.0f;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = xf[i] * inv;
  c.codes = e2m1_encode8(y);
  return c;
}

// Squared error of this lane's half block: fma chain in element order from +0.
__device__ __forceinline__ float half_err(const float xf[8], const Cand& c) {
  f32x2 v[4] = {e2m1_decode2<0>(c.codes), e2m1_decode2<1>(c.codes), e2m1_decode2<2>(c.codes),
                e2m1_decode2<3>(c.codes)};
  float e = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float d0 = xf[2 * j] - v[j].x * c.S;
    e = __builtin_fmaf(d0, d0, e);
    const float d1 = xf[2 * j + 1] - v[j].y * c.S;
    e = __builtin_fmaf(d1, d1, e);
  }
  return e;
}

template <int RULE>
__global__ __launch_bounds__(kThreads) void quant_kernel(const uint4* __restrict__ x,
                                                         const float* __restrict__ amax,
                                                         uint32_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, Part p) {
  const Range r = wg_range(p);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float A = amax[r.g];
  const float s_enc = (A > 0.0f) ? kGlobalDiv / A : 0.0f;
  const float s_dec = A / kGlobalDiv;
  for (int64_t base = r.beg + wave * 64 * kQuantUnroll; base < r.end;
       base += kWaves * 64 * kQuantUnroll) {
    uint4 v[kQuantUnroll];
#pragma unroll
    for (int k = 0; k < kQuantUnroll; ++k) {
      const int64_t u = base + k * 64 + lane;
      v[k] = (u < r.end) ? x[u] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kQuantUnroll; ++k) {
      const int64_t u = base + k * 64 + lane;
      float xf[8] = {bf16_lo(v[k].x), bf16_hi(v[k].x), bf16_lo(v[k].y), bf16_hi(v[k].y),
                     bf16_lo(v[k].z), bf16_hi(v[k].z), bf16_lo(v[k].w), bf16_hi(v[k].w)};
      // Block amax: this lane's 8 elements, then the partner lane's (the two lanes of a
      // pair hold the two halves of one 16-element block; all lanes execute the swap).
      uint32_t mb = absmax8_bits(v[k]);
      mb = max(mb, swap_pair(mb));
      const float m = __uint_as_float(mb << 16);
      Cand pick;
      if constexpr (RULE == KVFP4_RULE_STATIC6) {
        pick = make_cand(xf, m, 6.0f, s_enc, s_dec);
      } else if constexpr (RULE == KVFP4_RULE_STATIC4) {
        pick = make_cand(xf, m, 4.0f, s_enc, s_dec);
      } else {
        const Cand c6 = make_cand(xf, m, 6.0f, s_enc, s_dec);
        const Cand c4 = make_cand(xf, m, 4.0f, s_enc, s_dec);
        // err = (chain over elements 0..7) + (chain over 8..15); the sum of two values is
        // the same in either operand order, so both lanes of the pair agree.
        const float h6 = half_err(xf, c6), h4 = half_err(xf, c4);
        const float err6 = h6 + swap_pair(h6);
        const float err4 = h4 + swap_pair(h4);
        pick = (err4 < err6) ? c4 : c6;
      }
      if (u < r.end) {
        codes[u] = pick.codes;
        if ((lane & 1) == 0) scales[u >> 1] = (uint8_t)pick.sf;
      }
    }
  }
}

// ---- dequantize ([P-NVFP4] "Stage 3"; [P-KV] "CUDA De-quantization Pipeline") -----------

__device__ __forceinline__ uint4 decode8(uint32_t w, float S) {
  const f32x2 a = e2m1_decode2<0>(w), b = e2m1_decode2<1>(w);
  const f32x2 c = e2m1_decode2<2>(w), d = e2m1_decode2<3>(w);
  uint4 o;
  o.x = pack_bf16x2(a.x * S, a.y * S);
  o.y = pack_bf16x2(b.x * S, b.y * S);
  o.z = pack_bf16x2(c.x * S, c.y * S);
  o.w = pack_bf16x2(d.x * S, d.y * S);
  return o;
}

__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, (u32x4*)p);
}

// One tile of kDqTileUnits units per workgroup (the partition's slices are exactly one
// tile; a group's last slice may be shorter).
__global__ __launch_bounds__(kDqThreads) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ amax,
                                                             uint4* __restrict__ y, Part p) {
  const Range r = wg_range(p);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float s_dec = amax[r.g] / kGlobalDiv;
  const int64_t base = r.beg + wave * 64 * kDqUnroll;
  uint32_t c[kDqUnroll], sf[kDqUnroll];
#pragma unroll
  for (int k = 0; k < kDqUnroll; ++k) {
    const int64_t u = base + k * 64 + lane;
    const bool ok = u < r.end;
    c[k] = ok ? codes[u] : 0u;
    sf[k] = ok ? (uint32_t)scales[u >> 1] : 0u;
  }
#pragma unroll
  for (int k = 0; k < kDqUnroll; ++k) {
    const int64_t u = base + k * 64 + lane;
    if (u < r.end) store_nt(y + u, decode8(c[k], e4m3_decode(sf[k]) * s_dec));
  }
}

// ---- host side ----------------------------------------------------------------------------

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shared argument checks; fills the partition on success.  fixed_slice > 0 makes every
// slice exactly that many units (one tile per workgroup); otherwise slices are sized so
// that about kTargetWorkgroups workgroups cover the tensor, rounded to unit_multiple.
int plan(int64_t rows, int32_t head_dim, int64_t rpg, int64_t unit_multiple, int64_t fixed_slice,
         Part* part, int64_t* n_groups) {
  if (rows < 0 || rpg <= 0) return KVFP4_EINVAL;
  if (head_dim < 64 || head_dim > 1024 || head_dim % 64 != 0) return KVFP4_EUNSUPPORTED;
  const int64_t upr = head_dim / 8;  // units per row
  if (rows > (INT64_C(1) << 52) / head_dim) return KVFP4_EINVAL;
  const int64_t ng = rows == 0 ? 0 : (rows - 1) / rpg + 1;
  const int64_t rpg_eff = rpg < rows ? rpg : (rows > 0 ? rows : 1);
  const int64_t upg = rpg_eff * upr;
  int64_t slice;
  if (fixed_slice > 0) {
    slice = fixed_slice;
  } else {
    const int64_t want = (kTargetWorkgroups + ng - 1) / (ng > 0 ? ng : 1);
    slice = (upg + want - 1) / want;
    slice = (slice + unit_multiple - 1) / unit_multiple * unit_multiple;
  }
  const int64_t spg = (upg + slice - 1) / slice;
  if (ng * spg > INT32_MAX) return KVFP4_EINVAL;
  part->units_total = rows * upr;
  part->units_per_group = upg;
  part->slice_units = slice;
  part->slices_per_group = (uint32_t)spg;
  *n_groups = ng;
  return KVFP4_OK;
}

int launched() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return KVFP4_EHIP;
  }
  return KVFP4_OK;
}

}  // namespace
}  // namespace kvfp4

using namespace kvfp4;

extern "C" int kvfp4_quantize(const uint16_t* x, int64_t rows, int32_t head_dim,
                              int64_t rows_per_group, int32_t rule, uint8_t* codes,
                              uint8_t* scales, float* group_amax, void* stream) {
  if (rule != KVFP4_RULE_STATIC6 && rule != KVFP4_RULE_STATIC4 && rule != KVFP4_RULE_MSE)
    return KVFP4_EINVAL;
  Part part;
  int64_t ng = 0;
  int rc = plan(rows, head_dim, rows_per_group, 64, 0, &part, &ng);
  if (rc != KVFP4_OK) return rc;
  if (rows == 0) return KVFP4_OK;
  if (!x || !codes || !scales || !group_amax) return KVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(group_amax, 4))
    return KVFP4_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const unsigned grid = (unsigned)(ng * part.slices_per_group);
  const int64_t cblocks = (ng + kThreads - 1) / kThreads;
  const unsigned cgrid = (unsigned)(cblocks < 1024 ? cblocks : 1024);
  hipLaunchKernelGGL(clear_kernel, dim3(cgrid), dim3(kThreads), 0, s, (uint32_t*)group_amax, ng);
  if ((rc = launched()) != KVFP4_OK) return rc;
  hipLaunchKernelGGL(amax_kernel, dim3(grid), dim3(kThreads), 0, s, (const uint4*)x,
                     (uint32_t*)group_amax, part);
  if ((rc = launched()) != KVFP4_OK) return rc;
  switch (rule) {
    case KVFP4_RULE_STATIC6:
      hipLaunchKernelGGL(quant_kernel<KVFP4_RULE_STATIC6>, dim3(grid), dim3(kThreads), 0, s,
                         (const uint4*)x, (const float*)group_amax, (uint32_t*)codes, scales, part);
      break;
    case KVFP4_RULE_STATIC4:
      hipLaunchKernelGGL(quant_kernel<KVFP4_RULE_STATIC4>, dim3(grid), dim3(kThreads), 0, s,
                         (const uint4*)x, (const float*)group_amax, (uint32_t*)codes, scales, part);
      break;
    default:
      hipLaunchKernelGGL(quant_kernel<KVFP4_RULE_MSE>, dim3(grid), dim3(kThreads), 0, s,
                         (const uint4*)x, (const float*)group_amax, (uint32_t*)codes, scales, part);
      break;
  }
  return launched();
}

extern "C" int kvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                                const float* group_amax, int64_t rows, int32_t head_dim,
                                int64_t rows_per_group, uint16_t* y, void* stream) {
  Part part;
  int64_t ng = 0;
  int rc = plan(rows, head_dim, rows_per_group, 64, kDqTileUnits, &part, &ng);
  if (rc != KVFP4_OK) return rc;
  if (rows == 0) return KVFP4_OK;
  if (!codes || !scales || !group_amax || !y) return KVFP4_EINVAL;
  if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(group_amax, 4) || !aligned(y, 16))
    return KVFP4_EALIGN;
  const unsigned grid = (unsigned)(ng * part.slices_per_group);
  hipLaunchKernelGGL(dequant_kernel, dim3(grid), dim3(kDqThreads), 0, (hipStream_t)stream,
                     (const uint32_t*)codes, scales, group_amax, (uint4*)y, part);
  return launched();
}

extern "C" int kvfp4_packed_sizes(int64_t rows, int32_t head_dim, int64_t rows_per_group,
                                  int64_t* codes_bytes, int64_t* scales_bytes,
                                  int64_t* n_groups) {
  Part part;
  int64_t ng = 0;
  int rc = plan(rows, head_dim, rows_per_group, 64, 0, &part, &ng);
  if (rc != KVFP4_OK) return rc;
  if (codes_bytes) *codes_bytes = rows * (head_dim / 2);
  if (scales_bytes) *scales_bytes = rows * (head_dim / 16);
  if (n_groups) *n_groups = ng;
  return KVFP4_OK;
}

extern "C" const char* kvfp4_status_str(int status) {
  switch (status) {
    case KVFP4_OK: return "KVFP4_OK";
    case KVFP4_EINVAL: return "KVFP4_EINVAL: invalid argument (null pointer, negative size, rows_per_group <= 0, unknown rule or size overflow)";
    case KVFP4_EALIGN: return "KVFP4_EALIGN: misaligned pointer (bf16 and code buffers need 16 B, scales and amax 4 B)";
    case KVFP4_EUNSUPPORTED: return "KVFP4_EUNSUPPORTED: unsupported head_dim";
    case KVFP4_EHIP: return "KVFP4_EHIP: kernel launch failed (see kvfp4_last_hip_error)";
    default: return "KVFP4: unknown status";
  }
}

extern "C" int kvfp4_abi_version(void) { return KVFP4_ABI_VERSION; }

extern "C" int kvfp4_last_hip_error(void) { return g_last_hip_error; }
