// Measurement only: back-to-back bf16 matrix products with no memory traffic, the matrix-core
// rate the chip sustains (under its own clock and power limits) that the prefill kernel is
// measured against beside the 2.5 PFLOP/s specification.  Not part of the attention path.
//
// The rate depends on the operands: products of small integers (few mantissa bits toggling)
// run at the specification's rate, products of random bf16 values, like attention's, draw
// more power and the chip clocks down.  `data` picks one or the other.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;    // independent accumulators per wave

// 512 threads (two waves per SIMD, as the prefill kernel runs); every wave issues `iters`
// rounds of kChains independent 32x32x16 products.  The accumulators' sum is written only if
// it equals an unlikely value, which keeps the products alive.
__device__ __forceinline__ uint32_t mix(uint32_t x) {   // an integer hash (for operand bits)
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  return x ^ (x >> 16);
}

__global__ __launch_bounds__(512) void mfma_probe(int32_t iters, int32_t data, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (data == 0) {            // small integers 0 .. 7
      a[e] = (__bf16)(float)((lane + e) & 7);
      b[e] = (__bf16)(float)((lane * 3 + e) & 7);
    } else {                    // random values in [-2, 2), different in every lane and workgroup
      const uint32_t h = mix((uint32_t)(threadIdx.x * 131 + e * 7) ^ mix((uint32_t)blockIdx.x));
      a[e] = (__bf16)((float)(h & 0xffffu) * (1.f / 16384.f) - 2.f);
      b[e] = (__bf16)((float)(h >> 16) * (1.f / 16384.f) - 2.f);
    }
  }
  f32x16 c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = f32x16{};
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) {
#pragma unroll
    for (int r = 0; r < 16; ++r) t += c[k][r];
  }
  if (__float_as_uint(t) == 0x9e3779b9u) sink[0] = __float_as_uint(t);
}

}  // namespace

int64_t mfma_probe_flops(int32_t iters, int32_t grid) {
  return (int64_t)grid * 8 * iters * kChains * (2LL * 32 * 32 * 16);
}

hipError_t launch_mfma_probe(int32_t iters, int32_t data, uint32_t* sink, int32_t grid, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe, dim3((unsigned)grid), dim3(512), 0, s, iters, data, sink);
  return hipGetLastError();
}

}  // namespace pa
