// conv_probe.hip -- test-only kernels that apply the library's device conversion helpers
// (kvfp4_device.hpp) element-wise, so the GPU tests can sweep them against the oracle at
// arbitrary binary32 inputs (midpoints, neighbours, saturation), which the quantize path
// only reaches through bf16 inputs.  Each kernel is 1-D with an `i < n` bound.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvfp4_device.hpp"

using namespace kvfp4;

namespace {
constexpr int kT = 256;

// n8 groups of 8 values -> one code dword each
__global__ void e2m1_encode_k(const float* __restrict__ y, int64_t n8, uint32_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (i < n8) {
    float v[8];
    for (int j = 0; j < 8; ++j) v[j] = y[8 * i + j];
    out[i] = e2m1_encode8(v);
  }
}

__global__ void e2m1_decode_k(const uint32_t* __restrict__ w, int64_t n, float* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (i < n) {
    f32x2 a = e2m1_decode2<0>(w[i]), b = e2m1_decode2<1>(w[i]);
    f32x2 c = e2m1_decode2<2>(w[i]), d = e2m1_decode2<3>(w[i]);
    float* o = out + 8 * i;
    o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y; o[4] = c.x; o[5] = c.y; o[6] = d.x; o[7] = d.y;
  }
}

__global__ void e4m3_encode_k(const float* __restrict__ u, int64_t n, uint8_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (i < n) out[i] = (uint8_t)e4m3_encode(u[i]);
}

__global__ void e4m3_decode_k(const uint8_t* __restrict__ b, int64_t n, float* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (i < n) out[i] = e4m3_decode(b[i]);
}

__global__ void bf16_pack_k(const float* __restrict__ f, int64_t n2, uint32_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (i < n2) out[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
}

unsigned blocks(int64_t n) { return (unsigned)((n + kT - 1) / kT); }
int status() { return hipGetLastError() == hipSuccess ? 0 : 4; }
}  // namespace

extern "C" int probe_e2m1_encode(const float* y, int64_t n8, uint32_t* out, void* s) {
  if (n8 <= 0) return 0;
  hipLaunchKernelGGL(e2m1_encode_k, dim3(blocks(n8)), dim3(kT), 0, (hipStream_t)s, y, n8, out);
  return status();
}
extern "C" int probe_e2m1_decode(const uint32_t* w, int64_t n, float* out, void* s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(e2m1_decode_k, dim3(blocks(n)), dim3(kT), 0, (hipStream_t)s, w, n, out);
  return status();
}
extern "C" int probe_e4m3_encode(const float* u, int64_t n, uint8_t* out, void* s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(e4m3_encode_k, dim3(blocks(n)), dim3(kT), 0, (hipStream_t)s, u, n, out);
  return status();
}
extern "C" int probe_e4m3_decode(const uint8_t* b, int64_t n, float* out, void* s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(e4m3_decode_k, dim3(blocks(n)), dim3(kT), 0, (hipStream_t)s, b, n, out);
  return status();
}
extern "C" int probe_bf16_pack(const float* f, int64_t n2, uint32_t* out, void* s) {
  if (n2 <= 0) return 0;
  hipLaunchKernelGGL(bf16_pack_k, dim3(blocks(n2)), dim3(kT), 0, (hipStream_t)s, f, n2, out);
  return status();
}

// One 32x32x16 bf16 MFMA on one wave with the operand/result lane layout the attention
// kernel assumes: A[32x16] lane l holds row l%32, k = 8*(l/32)+i; B[16x32] lane l holds
// column l%32, k = 8*(l/32)+i; D[32x32] register j of lane l is row 8*(j/4)+4*(l/32)+j%4,
// column l%32.  a: row-major fp32 [32][16], b: row-major [16][32], d: row-major [32][32].
namespace {
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__global__ void mfma_layout_k(const float* __restrict__ a, const float* __restrict__ b,
                              float* __restrict__ d) {
  const int l = threadIdx.x;  // launched with exactly 64 threads
  const int col = l & 31, hi = l >> 5;
  bf16x8_t av, bv;
  for (int i = 0; i < 8; ++i) {
    av[i] = (__bf16)a[col * 16 + 8 * hi + i];   // row = l%32
    bv[i] = (__bf16)b[(8 * hi + i) * 32 + col]; // column = l%32
  }
  f32x16_t acc = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  for (int j = 0; j < 16; ++j) d[(8 * (j / 4) + 4 * hi + (j % 4)) * 32 + col] = acc[j];
}
}  // namespace
extern "C" int probe_mfma_32x32x16_bf16(const float* a, const float* b, float* d, void* s) {
  hipLaunchKernelGGL(mfma_layout_k, dim3(1), dim3(64), 0, (hipStream_t)s, a, b, d);
  return status();
}
