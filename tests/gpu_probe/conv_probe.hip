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
