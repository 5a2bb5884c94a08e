// kvfp4.hip -- libkvfp4: NVFP4 KV-cache quantize / dequantize kernels for MI355X (gfx950)
// and their C ABI (declared in include/kvfp4.h).
//
// Pages cited (titles as published):
//   [P-KV]    "How to Use KV Cache Quantization with LongLive's LongLiveQuantizationConfig"
//   [P-NVFP4] "How NVFP4 Quantization Works in LongLive 2.0 for Transformer Inference"
//   [P-SF]    "KV Cache Quantization for Self-Forcing Video Generation: A 33-Method
//              Empirical Study"
//
// Work decomposition.  The streaming kernels see a tensor as a flat sequence of 8-element
// "units" (16 B of bf16, 4 B of codes, half of a 16-element scale block).  A scale group
// (rows_per_group rows) is a contiguous run of units.  Each kernel cuts every group into
// fixed-size slices of its own tile size and launches one workgroup per (group, slice),
// in group-major order.  So a workgroup has a single group amax, read once into a
// uniform register, and never divides per lane to find its group; and because workgroups
// are dispatched in index order, the addresses in flight at any moment form a compact
// window of the tensor, which is what lets these kernels run near the HBM limit on
// MI355X (measured: persistent workgroups with long slices were 10-40% slower).
// Within a slice each wave takes 64*UNR consecutive units per step and its k-th load or
// store covers 64 consecutive units, so every wave instruction touches one contiguous
// span (1 KiB of bf16, 256 B of codes).  Index math is 64-bit.
//
// Quantize ([P-NVFP4] "Stage 1"): the group amax is a max over 15-bit bf16 magnitude
// patterns; the encode has the two lanes holding the halves of a 16-element block exchange
// half-block maxima through DPP, derive the same E4M3 scale, and each pack its 8 codes into
// one dword.  Two forms with identical output: one kernel that does both for a whole chunk
// (amax tiles hand each group's amax to its encode tiles through words in the group's own
// output; see "one-launch append" below), dense or paged, and three kernels (clear the amax
// words, amax pass with one atomicMax per workgroup, encode pass) for in-place fake
// quantization and for calls with a group (or page) of fewer than 66 units.
// Dequantize ([P-NVFP4] "Stage 3"): one pass; each lane turns one code dword and one scale
// byte into 8 bf16 (one 16 B non-temporal store).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvfp4.h"
#include "kvfp4_device.hpp"

namespace kvfp4 {
namespace {

// Launch shapes (threads per workgroup, units per lane per step, steps per workgroup),
// chosen by sweeping on MI355X over the 30-layer cache shapes.
constexpr int kAmaxThreads = 512, kAmaxUnroll = 4, kAmaxSteps = 4;
constexpr int kQuantThreads = 128, kQuantUnroll = 2, kQuantSteps = 1;  // static rules, RTN
constexpr int kMseThreads = 256, kMseUnroll = 2, kMseSteps = 4;        // mse rule
constexpr int kDqThreads = 128, kDqUnroll = 2;                         // one step
constexpr int kDqPagedThreads = 512;  // paged gather: one page lookup per 1024 units

constexpr int64_t tile_units(int threads, int unroll, int steps) {
  return (int64_t)threads * unroll * steps;
}

// Flat partition of a tensor into (group, slice) workgroups; sizes in 8-element units.
// With a block table (paged cache), dense group g lives in packed page table[g]; entries
// outside [0, n_pages) are skipped.  Without one, page = group.
struct Part {
  int64_t units_total;
  int64_t units_per_group;
  int64_t slice_units;
  uint32_t slices_per_group;
  const int32_t* table;
  int64_t n_pages;
};

struct Range {
  int64_t beg, end;  // dense-side units [beg, end)
  int64_t shift;     // packed-side unit = dense-side unit + shift
  int64_t page;      // packed-side group (index of its amax)
};

__device__ __forceinline__ Range wg_range(const Part& p) {
  Range r;
  const uint32_t g = blockIdx.x / p.slices_per_group;
  const uint32_t s = blockIdx.x - g * p.slices_per_group;
  const int64_t gbeg = (int64_t)g * p.units_per_group;
  const int64_t gend = min(gbeg + p.units_per_group, p.units_total);
  r.beg = gbeg + (int64_t)s * p.slice_units;
  r.end = min(r.beg + p.slice_units, gend);
  r.page = g;
  r.shift = 0;
  if (p.table) {
    r.page = p.table[g];
    if (r.page < 0 || r.page >= p.n_pages) r.end = r.beg;  // no such page: nothing to do
    r.shift = (r.page - (int64_t)g) * p.units_per_group;
  }
  return r;
}

// Value from the partner lane (lane ^ 1) through DPP quad_perm [1,0,3,2].
__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float swap_pair(float v) {
  return __uint_as_float(swap_pair(__float_as_uint(v)));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
  u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, (u32x4*)p);
}

// Streaming 16-byte load with the non-temporal hint (measured: faster for the group amax
// pass, slower for the encode passes, which read the same data right after).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// ---- kernel 1: clear group amax (through the block table when there is one) --------------
__global__ __launch_bounds__(256) void clear_kernel(uint32_t* __restrict__ p, int64_t n,
                                                    const int32_t* __restrict__ table,
                                                    int64_t n_pages) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t pg = table ? (int64_t)table[i] : i;
    if (pg >= 0 && pg < n_pages) p[pg] = 0u;
  }
}

// ---- kernel 2: group amax ([P-NVFP4] "Stage 1", global amax scalar) ---------------------
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const uint4* __restrict__ x,
                                                            uint32_t* __restrict__ amax_bits,
                                                            Part p) {
  constexpr int kW = kAmaxThreads / 64;
  const Range r = wg_range(p);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t mx = 0;
  for (int64_t base = r.beg + wave * 64 * kAmaxUnroll; base < r.end;
       base += kAmaxThreads * kAmaxUnroll) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int k = 0; k < kAmaxUnroll; ++k) {
      const int64_t u = base + k * 64 + lane;
      v[k] = (u < r.end) ? load_nt(x + u) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kAmaxUnroll; ++k) mx = max(mx, absmax8_bits(v[k]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  __shared__ uint32_t red[kW];
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0 && r.beg < r.end) {
    uint32_t m = red[0];
#pragma unroll
    for (int w = 1; w < kW; ++w) m = max(m, red[w]);
    // A non-negative binary32 orders like its bit pattern; bf16 -> fp32 is a 16-bit shift.
    atomicMax(&amax_bits[r.page], m << 16);
  }
}

// ---- kernel 3: encode ([P-NVFP4] "Stage 1"; [P-KV] scale rules) -------------------------

// Per-workgroup tables that replace the per-block divisions with lookups of values computed
// by the very same binary32 operations (so results are bit-identical):
//   t6[k]  = (128 + k) / 6          m/6 for a bf16 m with mantissa k, before the 2^e scaling
//   S[sf]  = E4M3(sf) * s_dec       decoded block scale
//   inv[sf] = S > 0 ? 1 / S : 0     its reciprocal
struct Tables {
  float t6[128], S[128], inv[128];
};

__device__ __forceinline__ void init_tables(Tables* tb, float s_dec, int nthreads) {
  for (int i = threadIdx.x; i < 128; i += nthreads) {
    tb->t6[i] = (float)(128 + i) / 6.0f;
    const float S = e4m3_decode((uint32_t)i) * s_dec;
    tb->S[i] = S;
    tb->inv[i] = (S > 0.0f) ? 1.0f / S : 0.0f;
  }
  __syncthreads();
}

// t = m / Dv for a block amax m given as its bf16 magnitude pattern mb.
// Dv = 4: m * 0.25 is the correctly rounded quotient.  Dv = 6: for a normal m with biased
// exponent e8 >= 4 the quotient is t6[mantissa] * 2^(e8 - 134) exactly (the power-of-two
// scaling is an exponent add that stays in the normal range); zero gives zero; the few
// remaining tiny values take a real division.
template <int DV>
__device__ __forceinline__ float block_t(uint32_t mb, const Tables* tb) {
  const float m = __uint_as_float(mb << 16);
  if constexpr (DV == 4) {
    return m * 0.25f;
  } else {
    const uint32_t e8 = mb >> 7;
    float t = __uint_as_float(__float_as_uint(tb->t6[mb & 127u]) + ((e8 - 134u) << 23));
    if (__builtin_expect(e8 < 4u, 0)) t = (mb == 0u) ? 0.0f : m / 6.0f;
    return t;
  }
}

// One candidate scaling of a block for this lane's 8 elements.
struct Cand {
  uint32_t sf;     // E4M3 byte
  float S;         // decoded block scale * s_dec
  uint32_t codes;  // 8 packed E2M1 codes
};

template <int DV>
__device__ __forceinline__ Cand make_cand(const float xf[8], uint32_t mb, float s_enc,
                                          const Tables* tb) {
  Cand c;
  // A product with a zero operand is zero, also where binary32 would form 0 * inf = NaN:
  // s_enc = +inf (group amax below 2688/FLT_MAX) meets an all-zero block, or inv = +inf
  // (S below 1/FLT_MAX, which needs S >= 2^-9 s_dec < 2^-128, i.e. s_enc > 2^119) meets a
  // zero element.  Both need s_enc > 2^100, a test that is uniform over the group, so
  // ordinary groups skip the fix-up.  Nonzero operands keep x * inf = +-inf (saturating).
  const bool tiny_group = s_enc > 0x1p100f;
  float u = block_t<DV>(mb, tb) * s_enc;
  if (__builtin_expect(tiny_group, 0)) u = (mb == 0u) ? 0.0f : u;
  c.sf = e4m3_encode(u);
  c.S = tb->S[c.sf];
  const float inv = tb->inv[c.sf];
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = xf[i] * inv;
  if (__builtin_expect(tiny_group, 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (xf[i] == 0.0f) ? xf[i] : y[i];
  }
  c.codes = e2m1_encode8(y);
  return c;
}

// Squared error of this lane's half block: fma chain in element order from +0.
__device__ __forceinline__ float half_err(const float xf[8], const Cand& c) {
  const f32x2 v[4] = {e2m1_decode2<0>(c.codes), e2m1_decode2<1>(c.codes),
                      e2m1_decode2<2>(c.codes), e2m1_decode2<3>(c.codes)};
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

// Encode one unit (8 elements, this lane) of a 16-element block whose other half is in the
// partner lane (lane ^ 1); both lanes must make the call.  Returns the chosen candidate.
template <int RULE>
__device__ __forceinline__ Cand encode_unit(uint4 v, float s_enc, const Tables* tb) {
  const float xf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                       bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  // Block amax: this lane's 8 elements, then the partner lane's.
  uint32_t mb = absmax8_bits(v);
  mb = max(mb, swap_pair(mb));
  if constexpr (RULE == KVFP4_RULE_STATIC6) {
    return make_cand<6>(xf, mb, s_enc, tb);
  } else if constexpr (RULE == KVFP4_RULE_STATIC4) {
    return make_cand<4>(xf, mb, s_enc, tb);
  } else {
    const Cand c6 = make_cand<6>(xf, mb, s_enc, tb);
    const Cand c4 = make_cand<4>(xf, mb, s_enc, tb);
    // err = (chain over elements 0..7) + (chain over 8..15); a sum of two values is the
    // same in either operand order, so both lanes of the pair agree.
    const float h6 = half_err(xf, c6), h4 = half_err(xf, c4);
    const float err6 = h6 + swap_pair(h6);
    const float err4 = h4 + swap_pair(h4);
    return (err4 < err6) ? c4 : c6;
  }
}

// FAKE: instead of storing codes and scale bytes, store the block dequantized to bf16
// (decode8 with the chosen candidate's S, which is E4M3(sf) * s_dec exactly as the
// dequantize kernel computes it), so the output equals dequantize(quantize(x)).
// x and fake_y are not restrict: fake quantization may run in place (each lane reads its
// unit before it writes the same unit, and no other lane touches it).
template <int RULE, int THREADS, int UNR, bool FAKE>
__global__ __launch_bounds__(THREADS) void quant_kernel(const uint4* x,
                                                        const float* __restrict__ amax,
                                                        uint32_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales,
                                                        uint4* fake_y, Part p) {
  const Range r = wg_range(p);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (r.beg >= r.end) return;  // uniform: skipped page or empty slice
  const float A = amax[r.page];
  const float s_enc = (A > 0.0f) ? kGlobalDiv / A : 0.0f;
  __shared__ Tables tabs;
  init_tables(&tabs, A / kGlobalDiv, THREADS);
  for (int64_t base = r.beg + wave * 64 * UNR; base < r.end; base += THREADS * UNR) {
    uint4 v[UNR];
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int64_t u = base + k * 64 + lane;
      v[k] = (u < r.end) ? x[u] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int64_t u = base + k * 64 + lane;
      const Cand pick = encode_unit<RULE>(v[k], s_enc, &tabs);
      if (u < r.end) {
        if constexpr (FAKE) {
          store_nt(fake_y + u, decode8(pick.codes, pick.S));
        } else {
          const int64_t pu = u + r.shift;
          __builtin_nontemporal_store(pick.codes, codes + pu);
          if ((lane & 1) == 0) scales[pu >> 1] = (uint8_t)pick.sf;
        }
      }
    }
  }
}

// ---- one-launch append: group amax and encode in a single kernel ------------------------
//
// The three-kernel form above reads the input twice from HBM (amax pass, then encode).  Here
// one launch does both.  Work items in workgroup index (= dispatch) order: the amax tiles of
// group g + L come before the encode tiles of group g, L = ceil(32 MiB / group input bytes)
// groups (at least 1, at most all), so an encode tile re-reads input that was read shortly
// before, a re-read that the 256 MB Infinity Cache partly serves (measured: the one launch
// beats amax pass + encode pass by about a fifth with the same bytes).
//
// Per group, three dwords inside the group's own output (the code dwords of its units 0, 32
// and 64, or the first dword of those units of the bf16 output for fake quantization: three
// different 128-byte lines), zeroed by append_clear_kernel before the launch, carry the
// hand-off from the amax tiles to the encode tiles:
//   count  (unit 0)   amax tiles done
//   max    (unit 32)  max over the done tiles of their 15-bit magnitude patterns << 16
//   ready  (unit 64)  final amax bits | 1, stored by the tile that completes the count
// An amax tile folds its max into `max`, then adds 1 to `count`; the add takes the returned
// old max as an operand, so it is issued only after the max has been performed.  The tile
// whose add completes the count reads `max` (now final), stores the group amax and sets
// `ready`.  All of these are device-scope atomics, coherent across the XCDs.
// An encode tile polls `ready` for at most `wait_ticks` wall-clock ticks (a short sleep
// between polls); past that it computes the group max from x itself -- the same value -- so
// the bound limits the wait and never changes a result.  Encode tiles skip the stores of
// units 0, 32 and 64 of their group; append_finish_kernel encodes those three units after the
// launch, overwriting the words.  Requires every group (the last included) to have at least
// 66 units.
constexpr int kAppendATile = 4096;  // units per amax tile
constexpr int kAppendETile = 2048;  // units per encode tile
constexpr int64_t kAppendLagUnits = (INT64_C(32) << 20) / 16;
constexpr int kAppendStaticThreads = 512, kAppendMseThreads = 256;  // measured

struct Append {
  int64_t units_total, units_per_group;
  uint32_t n_groups, lag;        // lag: groups, in [1, n_groups]
  uint32_t a_tiles, e_tiles;     // per group
  uint64_t wait_ticks;
  const int32_t* table;          // paged cache: dense group g lives in page table[g]; or null
  int64_t n_pages;
};

// Packed-side group of dense group g (itself without a table), or -1 for a table entry
// outside [0, n_pages): that block is skipped.
__device__ __forceinline__ int64_t append_page(const int32_t* table, int64_t n_pages, int64_t g) {
  if (!table) return g;
  const int64_t pg = table[g];
  return (pg >= 0 && pg < n_pages) ? pg : -1;
}

// Max of the 15-bit magnitude patterns over units [beg, end), per thread.
template <int THREADS>
__device__ __forceinline__ uint32_t thread_absmax(const uint4* x, int64_t beg, int64_t end) {
  constexpr int kU = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t mx = 0;
  for (int64_t base = beg + wave * 64 * kU; base < end; base += THREADS * kU) {
    uint4 v[kU];
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int64_t u = base + k * 64 + lane;
      v[k] = (u < end) ? x[u] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kU; ++k) mx = max(mx, absmax8_bits(v[k]));
  }
  return mx;
}

// Workgroup max; every thread gets it.  `red` must not be in use by another reduction.
template <int THREADS>
__device__ __forceinline__ uint32_t workgroup_max(uint32_t mx, uint32_t* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  uint32_t m = red[0];
#pragma unroll
  for (int w = 1; w < THREADS / 64; ++w) m = max(m, red[w]);
  return m;
}

// Dword of the hand-off word at unit `unit` of the output (codes: one dword per unit; fake
// bf16 output: four dwords per unit).
template <bool FAKE>
__device__ __forceinline__ uint32_t* handoff_word(uint32_t* out, int64_t unit) {
  return out + unit * (FAKE ? 4 : 1);
}

__global__ __launch_bounds__(256) void append_clear_kernel(uint32_t* __restrict__ out,
                                                           int64_t units_per_group,
                                                           int64_t n_groups, int stride,
                                                           const int32_t* __restrict__ table,
                                                           int64_t n_pages) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < 3 * n_groups;
       i += (int64_t)gridDim.x * 256) {
    const int64_t g = i / 3, k = i - g * 3;
    const int64_t pg = append_page(table, n_pages, g);
    if (pg >= 0) out[(pg * units_per_group + 32 * k) * stride] = 0u;
  }
}

template <int RULE, int THREADS, bool FAKE>
__global__ __launch_bounds__(THREADS) void append_kernel(const uint4* __restrict__ x,
                                                         uint32_t* __restrict__ amax_bits,
                                                         uint32_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales,
                                                         uint4* __restrict__ fake_y, Append f) {
  // work item of this workgroup
  const uint32_t b = blockIdx.x, per = f.a_tiles + f.e_tiles;
  const uint32_t head = f.lag * f.a_tiles, mid = (f.n_groups - f.lag) * per;
  uint32_t g, t;
  bool amax_tile;
  if (b < head) {
    g = b / f.a_tiles;
    t = b - g * f.a_tiles;
    amax_tile = true;
  } else if (b - head < mid) {
    const uint32_t k = b - head, j = k / per, o = k - j * per;
    amax_tile = o < f.a_tiles;
    g = amax_tile ? f.lag + j : j;
    t = amax_tile ? o : o - f.a_tiles;
  } else {
    const uint32_t k = b - head - mid, j = k / f.e_tiles;
    g = f.n_groups - f.lag + j;
    t = k - j * f.e_tiles;
    amax_tile = false;
  }
  const int64_t page = append_page(f.table, f.n_pages, g);
  if (page < 0) return;  // uniform: no such page, nothing to read or write
  const int64_t gbeg = (int64_t)g * f.units_per_group;
  const int64_t gend = min(gbeg + f.units_per_group, f.units_total);
  const int64_t shift = (page - (int64_t)g) * f.units_per_group;  // packed = dense + shift
  uint32_t* const out = FAKE ? (uint32_t*)fake_y : codes;
  uint32_t* const w_count = handoff_word<FAKE>(out, gbeg + shift);
  uint32_t* const w_max = handoff_word<FAKE>(out, gbeg + shift + 32);
  uint32_t* const w_ready = handoff_word<FAKE>(out, gbeg + shift + 64);
  __shared__ uint32_t red[THREADS / 64];
  __shared__ uint32_t ready_bits;

  if (amax_tile) {
    const int64_t beg = gbeg + (int64_t)t * kAppendATile;
    const int64_t end = min(beg + kAppendATile, gend);
    const uint32_t m = workgroup_max<THREADS>(thread_absmax<THREADS>(x, beg, end), red);
    if (threadIdx.x == 0) {
      const uint32_t old = __hip_atomic_fetch_max(w_max, m << 16, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      // old >> 31 is 0 (a magnitude pattern << 16); using it orders the add after the max
      const uint32_t done = __hip_atomic_fetch_add(w_count, 1u + (old >> 31), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      if (done + 1u == f.a_tiles) {
        const uint32_t fin = __hip_atomic_load(w_max, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        amax_bits[page] = fin;
        __hip_atomic_store(w_ready, fin | 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }

  if (threadIdx.x == 0) {
    uint32_t c = __hip_atomic_load(w_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!(c & 1u) && f.wait_ticks > 0) {
      const uint64_t t0 = wall_clock64();
      do {
        __builtin_amdgcn_s_sleep(8);
        c = __hip_atomic_load(w_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } while (!(c & 1u) && wall_clock64() - t0 < f.wait_ticks);
    }
    ready_bits = c;
  }
  __syncthreads();
  uint32_t abits = ready_bits;  // uniform
  if (abits & 1u)
    abits &= 0xFFFF0000u;
  else  // not published within the bound: the group max, computed here
    abits = workgroup_max<THREADS>(thread_absmax<THREADS>(x, gbeg, gend), red) << 16;

  const int64_t beg = gbeg + (int64_t)t * kAppendETile;
  const int64_t end = min(beg + kAppendETile, gend);
  const float A = __uint_as_float(abits);
  const float s_enc = (A > 0.0f) ? kGlobalDiv / A : 0.0f;
  __shared__ Tables tabs;
  init_tables(&tabs, A / kGlobalDiv, THREADS);
  constexpr int UNR = 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t base = beg + wave * 64 * UNR; base < end; base += THREADS * UNR) {
    uint4 v[UNR];
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int64_t u = base + k * 64 + lane;
      v[k] = (u < end) ? x[u] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int64_t u = base + k * 64 + lane;
      const Cand pick = encode_unit<RULE>(v[k], s_enc, &tabs);
      const int64_t rel = u - gbeg;
      const bool handoff = t == 0 && (rel == 0 || rel == 32 || rel == 64);
      if (u < end) {
        if constexpr (FAKE) {
          if (!handoff) store_nt(fake_y + u, decode8(pick.codes, pick.S));
        } else {
          if (!handoff) __builtin_nontemporal_store(pick.codes, codes + u + shift);
          if ((lane & 1) == 0) scales[(u + shift) >> 1] = (uint8_t)pick.sf;
        }
      }
    }
  }
}

// Units 0, 32 and 64 of each group (lanes 0..5 hold the blocks (0,1), (32,33), (64,65)),
// after append_kernel: the same encode, stored over the hand-off words.  One wave per group.
template <int RULE, bool FAKE>
__global__ __launch_bounds__(64) void append_finish_kernel(const uint4* __restrict__ x,
                                                           const float* __restrict__ amax,
                                                           uint32_t* __restrict__ codes,
                                                           uint4* __restrict__ fake_y,
                                                           int64_t units_per_group,
                                                           const int32_t* __restrict__ table,
                                                           int64_t n_pages) {
  const int64_t page = append_page(table, n_pages, blockIdx.x);
  if (page < 0) return;  // uniform
  const int lane = threadIdx.x;
  const int64_t rel = (lane >> 1) * 32 + (lane & 1);
  const int64_t u = (int64_t)blockIdx.x * units_per_group + rel;  // dense side (x)
  const int64_t pu = page * units_per_group + rel;                // packed side
  const bool active = lane < 6;
  const uint4 v = active ? x[u] : make_uint4(0, 0, 0, 0);
  const float A = amax[page];
  const float s_enc = (A > 0.0f) ? kGlobalDiv / A : 0.0f;
  __shared__ Tables tabs;
  init_tables(&tabs, A / kGlobalDiv, 64);
  const Cand pick = encode_unit<RULE>(v, s_enc, &tabs);
  if (active && (lane & 1) == 0) {
    if constexpr (FAKE)
      store_nt(fake_y + u, decode8(pick.codes, pick.S));
    else
      codes[pu] = pick.codes;
  }
}

// ---- dequantize ([P-NVFP4] "Stage 3"; [P-KV] "CUDA De-quantization Pipeline") -----------

// One step per workgroup: THREADS/64 waves, each writing one contiguous 2 KiB run of bf16.
// Dense reads use two-wave workgroups; the paged gather uses eight-wave ones, because each
// of its workgroups must look its page up before its loads can issue (measured: 5.85 ->
// 6.0 TB/s on random 16-token pages).
template <int THREADS>
__global__ __launch_bounds__(THREADS) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales,
                                                          const float* __restrict__ amax,
                                                          uint4* __restrict__ y, Part p) {
  const Range r = wg_range(p);
  if (r.beg >= r.end) return;  // uniform: skipped page or empty slice
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float s_dec = amax[r.page] / kGlobalDiv;
  const int64_t base = r.beg + wave * 64 * kDqUnroll;
  uint32_t c[kDqUnroll], sf[kDqUnroll];
#pragma unroll
  for (int k = 0; k < kDqUnroll; ++k) {
    const int64_t u = base + k * 64 + lane;
    const bool ok = u < r.end;
    c[k] = ok ? codes[u + r.shift] : 0u;
    sf[k] = ok ? (uint32_t)scales[(u + r.shift) >> 1] : 0u;
  }
#pragma unroll
  for (int k = 0; k < kDqUnroll; ++k) {
    const int64_t u = base + k * 64 + lane;
    if (u < r.end) store_nt(y + u, decode8(c[k], e4m3_decode(sf[k]) * s_dec));
  }
}

// float32 output ([P-NVFP4] "Stage 3": float32 or bf16).  A lane takes half a unit (4
// elements: one 16-bit code load, one 16 B store), so each wave store still covers one
// contiguous 1 KiB span; one step of 512 units per workgroup.
constexpr int kDqfThreads = 256, kDqfUnroll = 4;  // half units per lane (measured)

__global__ __launch_bounds__(kDqfThreads) void dequant_f32_kernel(const uint16_t* __restrict__ codes,
                                                                  const uint8_t* __restrict__ scales,
                                                                  const float* __restrict__ amax,
                                                                  float4* __restrict__ y, Part p) {
  const Range r = wg_range(p);
  if (r.beg >= r.end) return;  // uniform: skipped page or empty slice
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float s_dec = amax[r.page] / kGlobalDiv;
  const int64_t he = 2 * r.end, hs = 2 * r.shift;  // half units
  const int64_t base = 2 * r.beg + wave * 64 * kDqfUnroll;
  uint32_t c[kDqfUnroll], sf[kDqfUnroll];
#pragma unroll
  for (int k = 0; k < kDqfUnroll; ++k) {
    const int64_t h = min(base + k * 64 + lane, he - 1) + hs;  // clamped: always in range
    c[k] = codes[h];
    sf[k] = scales[h >> 2];
  }
#pragma unroll
  for (int k = 0; k < kDqfUnroll; ++k) {
    const int64_t h = base + k * 64 + lane;
    if (h < he) {
      const float S = e4m3_decode(sf[k]) * s_dec;
      const f32x2 a = e2m1_decode2<0>(c[k]), b = e2m1_decode2<1>(c[k]);
      float4 o;
      o.x = a.x * S;
      o.y = a.y * S;
      o.z = b.x * S;
      o.w = b.y * S;
      store_nt((uint4*)(y + h), __builtin_bit_cast(uint4, o));
    }
  }
}

// ---- RTN symmetric blockwise INT4 / INT2 ([P-SF] Table 3) --------------------------------
// Per 16-element block: s = bf16(m / qmax), inv = 1/s, q = clamp(rne(x * inv), +-qmax) in
// two's complement, lowest element in the lowest bits; dequant bf16(q * s).  Same lane-pair
// mapping as the NVFP4 encoder: a lane packs its 8 codes into 32 (INT4) or 16 (INT2) bits.
template <int BITS>
__global__ __launch_bounds__(kQuantThreads) void rtn_quant_kernel(const uint4* __restrict__ x,
                                                                  void* __restrict__ codes,
                                                                  uint16_t* __restrict__ scales,
                                                                  Part p) {
  constexpr float kQmax = (float)((1 << (BITS - 1)) - 1);
  const Range r = wg_range(p);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t base = r.beg + wave * 64 * kQuantUnroll; base < r.end;
       base += kQuantThreads * kQuantUnroll) {
    uint4 v[kQuantUnroll];
#pragma unroll
    for (int k = 0; k < kQuantUnroll; ++k) {
      const int64_t u = base + k * 64 + lane;
      v[k] = (u < r.end) ? x[u] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kQuantUnroll; ++k) {
      const int64_t u = base + k * 64 + lane;
      const float xf[8] = {bf16_lo(v[k].x), bf16_hi(v[k].x), bf16_lo(v[k].y), bf16_hi(v[k].y),
                           bf16_lo(v[k].z), bf16_hi(v[k].z), bf16_lo(v[k].w), bf16_hi(v[k].w)};
      uint32_t mb = absmax8_bits(v[k]);
      mb = max(mb, swap_pair(mb));
      const float m = __uint_as_float(mb << 16);
      const float sq = (BITS == 4) ? m / kQmax : m;  // IEEE division; m/1 is m
      const uint32_t sh = pack_bf16x2(sq, 0.0f) & 0xFFFFu;
      const float sv = __uint_as_float(sh << 16);
      const float inv = (sv > 0.0f) ? 1.0f / sv : 0.0f;
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = xf[i] * inv;
      // inv = +inf (s below 1/FLT_MAX): a zero element gives q = 0, not rint(0 * inf) = NaN.
      if (__builtin_expect(inv > 3.40282347e38f, 0)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = (xf[i] == 0.0f) ? 0.0f : p[i];
      }
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float qf = fminf(fmaxf(__builtin_rintf(p[i]), -kQmax), kQmax);
        w |= ((uint32_t)(int)qf & ((1u << BITS) - 1)) << (BITS * i);
      }
      if (u < r.end) {
        if constexpr (BITS == 4) ((uint32_t*)codes)[u] = w;
        else ((uint16_t*)codes)[u] = (uint16_t)w;
        if ((lane & 1) == 0) scales[u >> 1] = (uint16_t)sh;
      }
    }
  }
}

// Sign-extend the eight BITS-wide fields of w, scale by the block scale and round to bf16.
template <int BITS>
__device__ __forceinline__ uint4 rtn_decode8(uint32_t w, uint32_t scale_bits) {
  const float sv = __uint_as_float(scale_bits << 16);
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = (int)(w << (32 - BITS * (i + 1))) >> (32 - BITS);  // sign-extend field i
    f[i] = (float)q * sv;
  }
  uint4 o;
  o.x = pack_bf16x2(f[0], f[1]);
  o.y = pack_bf16x2(f[2], f[3]);
  o.z = pack_bf16x2(f[4], f[5]);
  o.w = pack_bf16x2(f[6], f[7]);
  return o;
}

template <int BITS>
__device__ __forceinline__ uint32_t rtn_word(const void* codes, int64_t u) {
  return (BITS == 4) ? ((const uint32_t*)codes)[u] : (uint32_t)((const uint16_t*)codes)[u];
}

// Dequantize a packed prefix of `prefix_units` units, then copy a bf16 tail (the recent,
// unquantized rows) behind it in the same launch.  Workgroups that lie wholly in the prefix
// or wholly in the tail load with indexes clamped into their own range, so every load is
// unconditional and all of them are in flight before the first use; only the one workgroup
// that straddles the boundary decides per lane.
template <int BITS>
__global__ __launch_bounds__(kDqThreads) void rtn_dequant_kernel(const void* __restrict__ codes,
                                                                 const uint16_t* __restrict__ scales,
                                                                 const uint4* __restrict__ tail,
                                                                 int64_t prefix_units,
                                                                 uint4* __restrict__ y, Part p) {
  const Range r = wg_range(p);  // never empty: one group, slices cover it
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = r.beg + wave * 64 * kDqUnroll;
  if (r.beg >= prefix_units) {  // uniform: tail only
    uint4 t[kDqUnroll];
#pragma unroll
    for (int k = 0; k < kDqUnroll; ++k)
      t[k] = tail[min(base + k * 64 + lane, r.end - 1) - prefix_units];
#pragma unroll
    for (int k = 0; k < kDqUnroll; ++k) {
      const int64_t u = base + k * 64 + lane;
      if (u < r.end) store_nt(y + u, t[k]);
    }
    return;
  }
  if (r.end <= prefix_units) {  // uniform: packed prefix only
    uint32_t w[kDqUnroll], sb[kDqUnroll];
#pragma unroll
    for (int k = 0; k < kDqUnroll; ++k) {
      const int64_t ui = min(base + k * 64 + lane, r.end - 1);
      w[k] = rtn_word<BITS>(codes, ui);
      sb[k] = scales[ui >> 1];
    }
#pragma unroll
    for (int k = 0; k < kDqUnroll; ++k) {
      const int64_t u = base + k * 64 + lane;
      if (u < r.end) store_nt(y + u, rtn_decode8<BITS>(w[k], sb[k]));
    }
    return;
  }
  // The boundary workgroup.
#pragma unroll
  for (int k = 0; k < kDqUnroll; ++k) {
    const int64_t u = base + k * 64 + lane;
    if (u >= r.end) continue;
    const uint4 o = (u < prefix_units) ? rtn_decode8<BITS>(rtn_word<BITS>(codes, u), scales[u >> 1])
                                       : tail[u - prefix_units];
    store_nt(y + u, o);
  }
}

// ---- host side ----------------------------------------------------------------------------

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shared argument checks.
int check_shape(int64_t rows, int32_t head_dim, int64_t rpg, int64_t* n_groups) {
  if (rows < 0 || rpg <= 0) return KVFP4_EINVAL;
  if (head_dim < 64 || head_dim > 1024 || head_dim % 64 != 0) return KVFP4_EUNSUPPORTED;
  if (rows > (INT64_C(1) << 52) / head_dim) return KVFP4_EINVAL;
  *n_groups = rows == 0 ? 0 : (rows - 1) / rpg + 1;
  return KVFP4_OK;
}

// Partition for a kernel whose workgroups each take `slice` units.  Fails (EINVAL) if the
// grid would not fit in 32 bits.
int plan(int64_t rows, int32_t head_dim, int64_t rpg, int64_t slice, Part* part,
         unsigned* grid) {
  int64_t ng = 0;
  int rc = check_shape(rows, head_dim, rpg, &ng);
  if (rc != KVFP4_OK) return rc;
  const int64_t upr = head_dim / 8;  // units per row (a multiple of 8)
  const int64_t upg = (rpg < rows ? rpg : (rows > 0 ? rows : 1)) * upr;
  const int64_t spg = (upg + slice - 1) / slice;
  if (ng * spg > INT32_MAX) return KVFP4_EINVAL;
  part->units_total = rows * upr;
  part->units_per_group = upg;
  part->slice_units = slice;
  part->slices_per_group = (uint32_t)spg;
  part->table = nullptr;
  part->n_pages = ng;
  *grid = (unsigned)(ng * spg);
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

template <int RULE, int THREADS, int UNR, int STEPS>
int launch_quant(const uint16_t* x, int64_t rows, int32_t head_dim, int64_t rpg,
                 const int32_t* table, int64_t n_pages, uint8_t* codes, uint8_t* scales,
                 const float* amax, uint16_t* fake_y, hipStream_t s) {
  Part part;
  unsigned grid = 0;
  int rc = plan(rows, head_dim, rpg, tile_units(THREADS, UNR, STEPS), &part, &grid);
  if (rc != KVFP4_OK) return rc;
  part.table = table;
  if (table) part.n_pages = n_pages;
  if (fake_y)
    hipLaunchKernelGGL((quant_kernel<RULE, THREADS, UNR, true>), dim3(grid), dim3(THREADS), 0, s,
                       (const uint4*)x, amax, nullptr, nullptr, (uint4*)fake_y, part);
  else
    hipLaunchKernelGGL((quant_kernel<RULE, THREADS, UNR, false>), dim3(grid), dim3(THREADS), 0,
                       s, (const uint4*)x, amax, (uint32_t*)codes, scales, nullptr, part);
  return launched();
}

// Wall-clock ticks in `us` microseconds on the current device (100 MHz if the runtime does
// not report the device's wall-clock rate).
uint64_t wall_ticks(int64_t us) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    khz = 100000;
  return (uint64_t)us * (uint64_t)khz / 1000u;
}

// Per-call quantize options, checked and defaulted (NULL = KVFP4_QUANTIZE_OPTS_DEFAULT).
constexpr int64_t kMaxWaitUs = INT64_C(60000000);

int read_opts(const kvfp4_quantize_opts* in, kvfp4_quantize_opts* out) {
  const kvfp4_quantize_opts def = KVFP4_QUANTIZE_OPTS_DEFAULT;
  *out = in ? *in : def;
  if (out->form != KVFP4_FORM_AUTO && out->form != KVFP4_FORM_THREE_KERNEL &&
      out->form != KVFP4_FORM_ONE_KERNEL)
    return KVFP4_EINVAL;
  if (out->wait_us < 0 || out->wait_us > kMaxWaitUs) return KVFP4_EINVAL;
  return KVFP4_OK;
}

// One-launch append (three launches: hand-off clear, append, finish) when it applies: not in
// place, every group at least 66 units, grid within 32 bits (with a block table, a group is
// a page).  Sets *used; returns the status of what it enqueued.
template <int RULE, int THREADS>
int launch_append(const uint16_t* x, int64_t rows, int32_t head_dim, int64_t rpg,
                  const int32_t* table, int64_t n_pages, uint8_t* codes, uint8_t* scales,
                  float* group_amax, uint16_t* fake_y, int64_t wait_us, hipStream_t s,
                  bool* used) {
  *used = false;
  const int64_t upr = head_dim / 8;
  const int64_t upg = (rpg < rows ? rpg : rows) * upr;
  const int64_t ng = (rows - 1) / rpg + 1;
  const int64_t total = rows * upr;
  if (total - (ng - 1) * upg < 66) return KVFP4_OK;
  const int64_t ta = (upg + kAppendATile - 1) / kAppendATile;
  const int64_t te = (upg + kAppendETile - 1) / kAppendETile;
  if (ng * (ta + te) > INT32_MAX) return KVFP4_OK;
  int64_t lag = (kAppendLagUnits + upg - 1) / upg;
  if (lag > ng) lag = ng;
  Append f;
  f.units_total = total;
  f.units_per_group = upg;
  f.n_groups = (uint32_t)ng;
  f.lag = (uint32_t)lag;
  f.a_tiles = (uint32_t)ta;
  f.e_tiles = (uint32_t)te;
  f.wait_ticks = wait_us > 0 ? wall_ticks(wait_us) : 0;
  f.table = table;
  f.n_pages = table ? n_pages : ng;
  *used = true;
  uint32_t* out = fake_y ? (uint32_t*)fake_y : (uint32_t*)codes;
  const int64_t cblocks = (3 * ng + 255) / 256;
  const unsigned cgrid = (unsigned)(cblocks < 1024 ? cblocks : 1024);
  hipLaunchKernelGGL(append_clear_kernel, dim3(cgrid), dim3(256), 0, s, out, upg, ng,
                     fake_y ? 4 : 1, table, f.n_pages);
  int rc = launched();
  if (rc != KVFP4_OK) return rc;
  const unsigned grid = (unsigned)(ng * (ta + te));
  if (fake_y) {
    hipLaunchKernelGGL((append_kernel<RULE, THREADS, true>), dim3(grid), dim3(THREADS), 0, s,
                       (const uint4*)x, (uint32_t*)group_amax, nullptr, nullptr, (uint4*)fake_y, f);
    if ((rc = launched()) != KVFP4_OK) return rc;
    hipLaunchKernelGGL((append_finish_kernel<RULE, true>), dim3((unsigned)ng), dim3(64), 0, s,
                       (const uint4*)x, group_amax, nullptr, (uint4*)fake_y, upg, table,
                       f.n_pages);
  } else {
    hipLaunchKernelGGL((append_kernel<RULE, THREADS, false>), dim3(grid), dim3(THREADS), 0, s,
                       (const uint4*)x, (uint32_t*)group_amax, (uint32_t*)codes, scales, nullptr,
                       f);
    if ((rc = launched()) != KVFP4_OK) return rc;
    hipLaunchKernelGGL((append_finish_kernel<RULE, false>), dim3((unsigned)ng), dim3(64), 0, s,
                       (const uint4*)x, group_amax, (uint32_t*)codes, nullptr, upg, table,
                       f.n_pages);
  }
  return launched();
}

// Shared body of the dense, paged and fake quantize entry points (arguments and options
// already checked).  With fake_y set, the encode pass writes bf16 there instead of
// codes/scales.  Not-in-place calls take the one-launch append where it applies and the
// options choose it; the rest take three kernels: clear, group amax, encode.
int quantize_impl(const uint16_t* x, int64_t rows, int32_t head_dim, int64_t rpg, int32_t rule,
                  const int32_t* table, int64_t n_pages, uint8_t* codes, uint8_t* scales,
                  float* group_amax, uint16_t* fake_y, const kvfp4_quantize_opts& o,
                  hipStream_t s) {
  // KVFP4_FORM_AUTO: the one-kernel form for inputs of at least 40 MiB (80 MiB under mse);
  // below those sizes the three-kernel form measured faster (a chunk that fits inside the
  // amax/encode lag leaves the one-kernel form's hand-off serialized, plus its finish kernel).
  const int64_t in_bytes = rows * (int64_t)head_dim * 2;
  const int64_t min_bytes = (rule == KVFP4_RULE_MSE ? INT64_C(80) : INT64_C(40)) << 20;
  const bool one = o.form == KVFP4_FORM_ONE_KERNEL ||
                   (o.form == KVFP4_FORM_AUTO && in_bytes >= min_bytes);
  if ((const void*)fake_y != (const void*)x && one) {
    bool used = false;
    int arc;
    switch (rule) {
      case KVFP4_RULE_STATIC6:
        arc = launch_append<KVFP4_RULE_STATIC6, kAppendStaticThreads>(
            x, rows, head_dim, rpg, table, n_pages, codes, scales, group_amax, fake_y, o.wait_us, s,
            &used);
        break;
      case KVFP4_RULE_STATIC4:
        arc = launch_append<KVFP4_RULE_STATIC4, kAppendStaticThreads>(
            x, rows, head_dim, rpg, table, n_pages, codes, scales, group_amax, fake_y, o.wait_us, s,
            &used);
        break;
      default:
        arc = launch_append<KVFP4_RULE_MSE, kAppendMseThreads>(
            x, rows, head_dim, rpg, table, n_pages, codes, scales, group_amax, fake_y, o.wait_us, s,
            &used);
        break;
    }
    if (used) return arc;
  }
  Part apart;
  unsigned agrid = 0;
  int rc = plan(rows, head_dim, rpg, tile_units(kAmaxThreads, kAmaxUnroll, kAmaxSteps), &apart,
                &agrid);
  if (rc != KVFP4_OK) return rc;
  apart.table = table;
  if (table) apart.n_pages = n_pages;
  const int64_t ng = (rows - 1) / rpg + 1;
  const int64_t cblocks = (ng + 255) / 256;
  const unsigned cgrid = (unsigned)(cblocks < 1024 ? cblocks : 1024);
  hipLaunchKernelGGL(clear_kernel, dim3(cgrid), dim3(256), 0, s, (uint32_t*)group_amax, ng, table,
                     table ? n_pages : ng);
  if ((rc = launched()) != KVFP4_OK) return rc;
  hipLaunchKernelGGL(amax_kernel, dim3(agrid), dim3(kAmaxThreads), 0, s, (const uint4*)x,
                     (uint32_t*)group_amax, apart);
  if ((rc = launched()) != KVFP4_OK) return rc;
  switch (rule) {
    case KVFP4_RULE_STATIC6:
      return launch_quant<KVFP4_RULE_STATIC6, kQuantThreads, kQuantUnroll, kQuantSteps>(
          x, rows, head_dim, rpg, table, n_pages, codes, scales, group_amax, fake_y, s);
    case KVFP4_RULE_STATIC4:
      return launch_quant<KVFP4_RULE_STATIC4, kQuantThreads, kQuantUnroll, kQuantSteps>(
          x, rows, head_dim, rpg, table, n_pages, codes, scales, group_amax, fake_y, s);
    default:
      return launch_quant<KVFP4_RULE_MSE, kMseThreads, kMseUnroll, kMseSteps>(
          x, rows, head_dim, rpg, table, n_pages, codes, scales, group_amax, fake_y, s);
  }
}

// Shared body of the dequantize entry points: bf16 output to y16, or float32 to y32.
int dequantize_impl(const uint8_t* codes, const uint8_t* scales, const float* group_amax,
                    int64_t rows, int32_t head_dim, int64_t rpg, const int32_t* table,
                    int64_t n_pages, uint16_t* y16, float* y32, hipStream_t s) {
  const int threads = (table && !y32) ? kDqPagedThreads : kDqThreads;
  Part part;
  unsigned grid = 0;
  const int64_t slice =
      y32 ? (int64_t)kDqfThreads * kDqfUnroll / 2 : tile_units(threads, kDqUnroll, 1);
  int rc = plan(rows, head_dim, rpg, slice, &part, &grid);
  if (rc != KVFP4_OK) return rc;
  part.table = table;
  if (table) part.n_pages = n_pages;
  if (y32)
    hipLaunchKernelGGL(dequant_f32_kernel, dim3(grid), dim3(kDqfThreads), 0, s,
                       (const uint16_t*)codes, scales, group_amax, (float4*)y32, part);
  else if (table)
    hipLaunchKernelGGL(dequant_kernel<kDqPagedThreads>, dim3(grid), dim3(kDqPagedThreads), 0, s,
                       (const uint32_t*)codes, scales, group_amax, (uint4*)y16, part);
  else
    hipLaunchKernelGGL(dequant_kernel<kDqThreads>, dim3(grid), dim3(kDqThreads), 0, s,
                       (const uint32_t*)codes, scales, group_amax, (uint4*)y16, part);
  return launched();
}

}  // namespace

// Records a failed launch for kvfp4_last_hip_error() (shared with kvfp4_attend.hip).
int set_last_hip_error(int e) {
  g_last_hip_error = e;
  return KVFP4_EHIP;
}

}  // namespace kvfp4

using namespace kvfp4;

static bool known_rule(int32_t rule) {
  return rule == KVFP4_RULE_STATIC6 || rule == KVFP4_RULE_STATIC4 || rule == KVFP4_RULE_MSE;
}

extern "C" int kvfp4_quantize_ex(const uint16_t* x, int64_t rows, int32_t head_dim,
                                 int64_t rows_per_group, int32_t rule, uint8_t* codes,
                                 uint8_t* scales, float* group_amax,
                                 const kvfp4_quantize_opts* opts, void* stream) {
  if (!known_rule(rule)) return KVFP4_EINVAL;
  kvfp4_quantize_opts o;
  int rc = read_opts(opts, &o);
  if (rc != KVFP4_OK) return rc;
  int64_t ng = 0;
  rc = check_shape(rows, head_dim, rows_per_group, &ng);
  if (rc != KVFP4_OK) return rc;
  if (rows == 0) return KVFP4_OK;
  if (!x || !codes || !scales || !group_amax) return KVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(group_amax, 4))
    return KVFP4_EALIGN;
  return quantize_impl(x, rows, head_dim, rows_per_group, rule, nullptr, 0, codes, scales,
                       group_amax, nullptr, o, (hipStream_t)stream);
}

extern "C" int kvfp4_quantize(const uint16_t* x, int64_t rows, int32_t head_dim,
                              int64_t rows_per_group, int32_t rule, uint8_t* codes,
                              uint8_t* scales, float* group_amax, void* stream) {
  return kvfp4_quantize_ex(x, rows, head_dim, rows_per_group, rule, codes, scales, group_amax,
                           nullptr, stream);
}

static int dequantize_entry(const uint8_t* codes, const uint8_t* scales, const float* group_amax,
                            int64_t rows, int32_t head_dim, int64_t rows_per_group, uint16_t* y16,
                            float* y32, void* stream) {
  int64_t ng = 0;
  int rc = check_shape(rows, head_dim, rows_per_group, &ng);
  if (rc != KVFP4_OK) return rc;
  if (rows == 0) return KVFP4_OK;
  const void* y = y32 ? (const void*)y32 : (const void*)y16;
  if (!codes || !scales || !group_amax || !y) return KVFP4_EINVAL;
  if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(group_amax, 4) || !aligned(y, 16))
    return KVFP4_EALIGN;
  return dequantize_impl(codes, scales, group_amax, rows, head_dim, rows_per_group, nullptr, 0,
                         y16, y32, (hipStream_t)stream);
}

extern "C" int kvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                                const float* group_amax, int64_t rows, int32_t head_dim,
                                int64_t rows_per_group, uint16_t* y, void* stream) {
  return dequantize_entry(codes, scales, group_amax, rows, head_dim, rows_per_group, y, nullptr,
                          stream);
}

extern "C" int kvfp4_dequantize_f32(const uint8_t* codes, const uint8_t* scales,
                                    const float* group_amax, int64_t rows, int32_t head_dim,
                                    int64_t rows_per_group, float* y, void* stream) {
  if (rows > 0 && !y) return KVFP4_EINVAL;  // a null y would otherwise select bf16 output
  return dequantize_entry(codes, scales, group_amax, rows, head_dim, rows_per_group, nullptr, y,
                          stream);
}

extern "C" int kvfp4_fake_quantize_ex(const uint16_t* x, int64_t rows, int32_t head_dim,
                                      int64_t rows_per_group, int32_t rule, float* group_amax,
                                      uint16_t* y, const kvfp4_quantize_opts* opts,
                                      void* stream) {
  if (!known_rule(rule)) return KVFP4_EINVAL;
  kvfp4_quantize_opts o;
  int rc = read_opts(opts, &o);
  if (rc != KVFP4_OK) return rc;
  int64_t ng = 0;
  rc = check_shape(rows, head_dim, rows_per_group, &ng);
  if (rc != KVFP4_OK) return rc;
  if (rows == 0) return KVFP4_OK;
  if (!x || !group_amax || !y) return KVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(group_amax, 4)) return KVFP4_EALIGN;
  return quantize_impl(x, rows, head_dim, rows_per_group, rule, nullptr, 0, nullptr, nullptr,
                       group_amax, y, o, (hipStream_t)stream);
}

extern "C" int kvfp4_fake_quantize(const uint16_t* x, int64_t rows, int32_t head_dim,
                                   int64_t rows_per_group, int32_t rule, float* group_amax,
                                   uint16_t* y, void* stream) {
  return kvfp4_fake_quantize_ex(x, rows, head_dim, rows_per_group, rule, group_amax, y, nullptr,
                                stream);
}

// Paged cache: shared checks of the two paged entry points.
static int check_paged(int64_t n_blocks, int64_t rows_per_page, int32_t head_dim, int64_t n_pages,
                       const int32_t* block_table) {
  if (n_blocks < 0 || rows_per_page <= 0 || n_pages < 0) return KVFP4_EINVAL;
  if (n_blocks > 0 && (rows_per_page > (INT64_C(1) << 52) / n_blocks)) return KVFP4_EINVAL;
  int64_t ng = 0;
  int rc = check_shape(n_blocks * rows_per_page, head_dim, rows_per_page, &ng);
  if (rc != KVFP4_OK) return rc;
  // the packed side (n_pages pages) obeys the same size limit as the dense side
  if (n_pages > 0 && rows_per_page > ((INT64_C(1) << 52) / head_dim) / n_pages) return KVFP4_EINVAL;
  if (n_blocks > 0 && !block_table) return KVFP4_EINVAL;
  if (n_blocks > 0 && !aligned(block_table, 4)) return KVFP4_EALIGN;
  return KVFP4_OK;
}

extern "C" int kvfp4_quantize_paged_ex(const uint16_t* x, int64_t n_blocks,
                                       int64_t rows_per_page, int32_t head_dim, int32_t rule,
                                       const int32_t* block_table, int64_t n_pages,
                                       uint8_t* codes, uint8_t* scales, float* page_amax,
                                       const kvfp4_quantize_opts* opts, void* stream) {
  if (!known_rule(rule)) return KVFP4_EINVAL;
  kvfp4_quantize_opts o;
  int rc = read_opts(opts, &o);
  if (rc != KVFP4_OK) return rc;
  rc = check_paged(n_blocks, rows_per_page, head_dim, n_pages, block_table);
  if (rc != KVFP4_OK) return rc;
  if (n_blocks == 0) return KVFP4_OK;
  if (!x || !codes || !scales || !page_amax) return KVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(page_amax, 4))
    return KVFP4_EALIGN;
  return quantize_impl(x, n_blocks * rows_per_page, head_dim, rows_per_page, rule, block_table,
                       n_pages, codes, scales, page_amax, nullptr, o, (hipStream_t)stream);
}

extern "C" int kvfp4_quantize_paged(const uint16_t* x, int64_t n_blocks, int64_t rows_per_page,
                                    int32_t head_dim, int32_t rule, const int32_t* block_table,
                                    int64_t n_pages, uint8_t* codes, uint8_t* scales,
                                    float* page_amax, void* stream) {
  return kvfp4_quantize_paged_ex(x, n_blocks, rows_per_page, head_dim, rule, block_table, n_pages,
                                 codes, scales, page_amax, nullptr, stream);
}

static int dequantize_paged_entry(const uint8_t* codes, const uint8_t* scales,
                                  const float* page_amax, const int32_t* block_table,
                                  int64_t n_blocks, int64_t rows_per_page, int32_t head_dim,
                                  int64_t n_pages, uint16_t* y16, float* y32, void* stream) {
  int rc = check_paged(n_blocks, rows_per_page, head_dim, n_pages, block_table);
  if (rc != KVFP4_OK) return rc;
  if (n_blocks == 0) return KVFP4_OK;
  const void* y = y32 ? (const void*)y32 : (const void*)y16;
  if (!codes || !scales || !page_amax || !y) return KVFP4_EINVAL;
  if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(page_amax, 4) || !aligned(y, 16))
    return KVFP4_EALIGN;
  return dequantize_impl(codes, scales, page_amax, n_blocks * rows_per_page, head_dim,
                         rows_per_page, block_table, n_pages, y16, y32, (hipStream_t)stream);
}

extern "C" int kvfp4_dequantize_paged(const uint8_t* codes, const uint8_t* scales,
                                      const float* page_amax, const int32_t* block_table,
                                      int64_t n_blocks, int64_t rows_per_page, int32_t head_dim,
                                      int64_t n_pages, uint16_t* y, void* stream) {
  return dequantize_paged_entry(codes, scales, page_amax, block_table, n_blocks, rows_per_page,
                                head_dim, n_pages, y, nullptr, stream);
}

extern "C" int kvfp4_dequantize_paged_f32(const uint8_t* codes, const uint8_t* scales,
                                          const float* page_amax, const int32_t* block_table,
                                          int64_t n_blocks, int64_t rows_per_page,
                                          int32_t head_dim, int64_t n_pages, float* y,
                                          void* stream) {
  if (n_blocks > 0 && !y) return KVFP4_EINVAL;  // a null y would otherwise select bf16 output
  return dequantize_paged_entry(codes, scales, page_amax, block_table, n_blocks, rows_per_page,
                                head_dim, n_pages, nullptr, y, stream);
}

extern "C" int kvfp4_rtn_quantize(const uint16_t* x, int64_t rows, int32_t head_dim, int32_t bits,
                                  uint8_t* codes, uint16_t* scales, void* stream) {
  if (bits != 2 && bits != 4) return KVFP4_EINVAL;
  Part part;
  unsigned grid = 0;
  int rc = plan(rows, head_dim, rows > 0 ? rows : 1, tile_units(kQuantThreads, kQuantUnroll, 1),
                &part, &grid);
  if (rc != KVFP4_OK) return rc;
  if (rows == 0) return KVFP4_OK;
  if (!x || !codes || !scales) return KVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return KVFP4_EALIGN;
  if (bits == 4)
    hipLaunchKernelGGL(rtn_quant_kernel<4>, dim3(grid), dim3(kQuantThreads), 0, (hipStream_t)stream,
                       (const uint4*)x, (void*)codes, scales, part);
  else
    hipLaunchKernelGGL(rtn_quant_kernel<2>, dim3(grid), dim3(kQuantThreads), 0, (hipStream_t)stream,
                       (const uint4*)x, (void*)codes, scales, part);
  return launched();
}

extern "C" int kvfp4_rtn_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t rows,
                                    int32_t head_dim, int32_t bits, const uint16_t* tail,
                                    int64_t tail_rows, uint16_t* y, void* stream) {
  if (bits != 2 && bits != 4) return KVFP4_EINVAL;
  if (rows < 0 || tail_rows < 0 || rows > INT64_MAX / 2 - tail_rows) return KVFP4_EINVAL;
  const int64_t total = rows + tail_rows;
  Part part;
  unsigned grid = 0;
  int rc = plan(total, head_dim, total > 0 ? total : 1, tile_units(kDqThreads, kDqUnroll, 1), &part,
                &grid);
  if (rc != KVFP4_OK) return rc;
  if (total == 0) return KVFP4_OK;
  if (!y || (rows > 0 && (!codes || !scales)) || (tail_rows > 0 && !tail)) return KVFP4_EINVAL;
  if (!aligned(y, 16) || (rows > 0 && (!aligned(codes, 16) || !aligned(scales, 4))) ||
      (tail_rows > 0 && !aligned(tail, 16)))
    return KVFP4_EALIGN;
  const int64_t prefix_units = rows * (head_dim / 8);
  if (bits == 4)
    hipLaunchKernelGGL(rtn_dequant_kernel<4>, dim3(grid), dim3(kDqThreads), 0, (hipStream_t)stream,
                       (const void*)codes, scales, (const uint4*)tail, prefix_units, (uint4*)y, part);
  else
    hipLaunchKernelGGL(rtn_dequant_kernel<2>, dim3(grid), dim3(kDqThreads), 0, (hipStream_t)stream,
                       (const void*)codes, scales, (const uint4*)tail, prefix_units, (uint4*)y, part);
  return launched();
}

extern "C" int kvfp4_packed_sizes(int64_t rows, int32_t head_dim, int64_t rows_per_group,
                                  int64_t* codes_bytes, int64_t* scales_bytes,
                                  int64_t* n_groups) {
  int64_t ng = 0;
  int rc = check_shape(rows, head_dim, rows_per_group, &ng);
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
