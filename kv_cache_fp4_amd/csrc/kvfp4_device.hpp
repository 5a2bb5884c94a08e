// kvfp4_device.hpp -- gfx950 device helpers for the NVFP4 KV-cache kernels: bf16 unpack,
// FP8 E4M3 block-scale encode/decode, E2M1 element encode/decode, bf16 packing.
//
// Pages cited (titles as published):
//   [P-NVFP4] "How NVFP4 Quantization Works in LongLive 2.0 for Transformer Inference"
//
// Formats ([P-NVFP4] "Understanding the NVFP4 Format and Architecture": 4-bit elements with
// block scale amax/6, FP8 per-block scales; "Stage 3": global scale amax/(e2m1_max*e4m3_max)):
//   E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit -> {0, .5, 1, 1.5, 2, 3, 4, 6}.
//   E4M3 (OCP): bias 7, subnormals m*2^-9, largest finite 0x7E = 448, 0x7F is NaN.
// Both conversions round to nearest, ties to even, and saturate at the largest finite value.
//
// gfx950 has single-instruction conversions between packed fp32 pairs and packed E2M1
// (v_cvt_scalef32_pk_fp4_f32 / v_cvt_scalef32_pk_f32_fp4), from an fp32 pair to OCP E4M3
// (v_cvt_pk_fp8_f32) and from an fp32 pair to a bf16 pair (v_cvt_pk_bf16_f32).  Their "scale" operand only carries a power of two in the fp32
// exponent, so the NVFP4 block scale cannot ride on it: it is always 1.0 here and the block
// scale is applied with an explicit binary32 multiply, which keeps the op order fixed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// e2m1_max * e4m3_max: A/2688 is the global decode scale, 2688/A the encode scale.
constexpr float kGlobalDiv = 2688.0f;

// ---- bf16 -------------------------------------------------------------------------------

// The two bf16 halves of a dword, widened exactly to binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round two binary32 values to bf16 (nearest even) and pack them, `a` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Largest |x| of the 8 bf16 values in a uint4, as a bf16 magnitude pattern (0..0x7F7F).
// For finite values the order of the 15-bit magnitude patterns is the order of |x|.
__device__ __forceinline__ uint32_t absmax8_bits(uint4 v) {
  uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu;
  uint32_t c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
  uint32_t ab = max(a & 0xFFFFu, a >> 16);
  uint32_t cd = max(b & 0xFFFFu, b >> 16);
  uint32_t ef = max(c & 0xFFFFu, c >> 16);
  uint32_t gh = max(d & 0xFFFFu, d >> 16);
  return max(max(ab, cd), max(ef, gh));
}

// ---- FP8 E4M3 block scales --------------------------------------------------------------

// u >= 0 and finite (NaN is outside the contract).  Nearest E4M3 byte, ties to even;
// u >= 448 gives 0x7E.  gfx950's fp32 -> fp8 conversion is OCP E4M3 (bias 7, subnormals,
// round to nearest even); clamping to 448 first keeps it away from its overflow handling.
__device__ __forceinline__ uint32_t e4m3_encode(float u) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(u, 448.0f), 0.0f, 0, false);
  return (uint32_t)w & 0xFFu;
}

// Value of a non-negative E4M3 byte (0..0x7E), exact in binary32.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  float normal = __uint_as_float((b + (120u << 3)) << 20);  // exp8 = e + 120, mant = m << 20
  float sub = (float)(b & 7u) * 0.001953125f;                // m * 2^-9
  return (b >> 3) ? normal : sub;
}

// ---- E2M1 elements ----------------------------------------------------------------------

// Encode 8 binary32 values into 8 E2M1 codes packed in a dword: value 2j in the low nibble
// of byte j, value 2j+1 in its high nibble.
__device__ __forceinline__ uint32_t e2m1_encode8(const float y[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// Decode the two codes of byte `sel` (0..3) of a dword: .x = low nibble, .y = high nibble.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1_decode2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Dequantize one code dword (8 elements) with block scale S (= E4M3(sf) * A/2688): each
// E2M1 value times S in binary32, rounded to bf16.  Output element i in bf16 lane i.
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

}  // namespace kvfp4
