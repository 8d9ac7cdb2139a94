// KV write: the slot_mapping scatter of a step's new K/V rows into the block pool
// (write_kv of "Engine v2: one core for every request", section "Attention over the pool").
//
// The pool is slot-major ([blocks, block_size, Hkv, D]), so one token's Hkv*D row is
// contiguous both in the input and in the pool: the scatter is a copy of N contiguous rows
// to N row addresses.  Each thread moves 16-byte pieces (8 elements) and consecutive
// threads cover consecutive pieces of a row, so every wave reads and writes whole cache
// lines.  Negative slots (padding rows) go to the pool's last slot.
#include "pa_internal.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t dest_slot(const int64_t* slots, int64_t i, int64_t num_slots) {
  const int64_t s = slots[i];
  return s >= 0 ? s : num_slots - 1;
}

// Same dtype in and out: a bit copy in 16-byte pieces.  pieces = row bytes / 16.
__global__ __launch_bounds__(256) void kv_copy16(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                 const int64_t* __restrict__ slots, u32x4* __restrict__ kc,
                                                 u32x4* __restrict__ vc, int64_t n, int32_t pieces,
                                                 int64_t num_slots) {
  const int64_t total = n * pieces;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / pieces;
    const int32_t e = (int32_t)(idx - i * pieces);
    const int64_t s = dest_slot(slots, i, num_slots);
    const u32x4 kk = __builtin_nontemporal_load(&k[idx]);
    const u32x4 vv = __builtin_nontemporal_load(&v[idx]);
    kc[s * pieces + e] = kk;
    vc[s * pieces + e] = vv;
  }
}

// Any dtype pair, element by element (also the path for rows that are not 16-byte pieces).
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void kv_convert(const TI* __restrict__ k, const TI* __restrict__ v,
                                                  const int64_t* __restrict__ slots, TO* __restrict__ kc,
                                                  TO* __restrict__ vc, int64_t n, int32_t row,
                                                  int64_t num_slots) {
  const int64_t total = n * row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / row;
    const int32_t e = (int32_t)(idx - i * row);
    const int64_t s = dest_slot(slots, i, num_slots);
    Elem<TO>::store(&kc[s * row + e], Elem<TI>::load(&k[idx]));
    Elem<TO>::store(&vc[s * row + e], Elem<TI>::load(&v[idx]));
  }
}

// Nearest fp8 E4M3 (OCP FN: bias 7, 3 mantissa bits, no infinities, largest finite 448) of a
// float, ties to even; magnitudes of 448 and above give 448 (values in [448, 464) round there,
// larger ones saturate); NaN gives the NaN code.  The value is rounded on its binade's grid
// (2^(E-3) for |y| in [2^E, 2^(E+1)), E >= -6; 2^-9 below 2^-6); a rounding that reaches the
// next binade lands on its code because codes of one sign increase with the value.
__device__ __forceinline__ uint32_t fp8_e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a < 448.f)) return a != a ? 0x7Fu : (sign | 0x7Eu);
  const int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // floor(log2 a); -127 for 0 and subnormals
  if (E < -6) return sign | (uint32_t)rintf(a * 512.f);
  return sign | (uint32_t)((E + 7) * 8 + (int)rintf(ldexpf(a, 3 - E)) - 8);
}

// KV write into fp8 pools: one wave per (token, KV head) row of D values.  scale = max|x| /
// 448 (1 for an all-zero row), codes = nearest fp8 of x / scale; both divisions are IEEE
// float32 divisions.  Codes go to the row's slot in the byte pools, the scale to
// scales[slot * Hkv + head].
template <typename TI>
__global__ __launch_bounds__(256) void kv_quant_fp8(const TI* __restrict__ k, const TI* __restrict__ v,
                                                    const int64_t* __restrict__ slots, uint8_t* __restrict__ kc,
                                                    uint8_t* __restrict__ vc, float* __restrict__ ks,
                                                    float* __restrict__ vs, int64_t n, int32_t hkv, int32_t d,
                                                    int64_t num_slots) {
  const int lane = threadIdx.x & 63;
  const int64_t rowid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rowid >= n * hkv) return;                              // whole waves exit together
  const int64_t i = rowid / hkv;
  const int32_t h = (int32_t)(rowid - i * hkv);
  const int64_t slot = dest_slot(slots, i, num_slots);
  const int64_t src = rowid * d, dst = (slot * hkv + h) * d;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const TI* x = which == 0 ? k : v;
    uint8_t* out = which == 0 ? kc : vc;
    float* sc = which == 0 ? ks : vs;
    float val[4];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = lane + 64 * e;
      val[e] = col < d ? Elem<TI>::load(&x[src + col]) : 0.f;
      amax = fmaxf(amax, fabsf(val[e]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = lane + 64 * e;
      if (col < d) out[dst + col] = (uint8_t)fp8_e4m3_code(val[e] / scale);
    }
    if (lane == 0) sc[slot * hkv + h] = scale;
  }
}

int grid_for(int64_t work) {
  int64_t blocks = (work + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return (int)(blocks < 1 ? 1 : blocks);
}

}  // namespace

hipError_t launch_kv_write(const void* k, const void* v, const int64_t* slots, void* kc, void* vc,
                           int64_t n, int32_t row, int64_t num_slots, int32_t in_dtype,
                           int32_t cache_dtype, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int esize_in = in_dtype == 0 ? 4 : 2;
  const bool aligned = ((uintptr_t)k | (uintptr_t)v | (uintptr_t)kc | (uintptr_t)vc) % 16 == 0;
  if (in_dtype == cache_dtype && aligned && ((int64_t)row * esize_in) % 16 == 0) {
    const int32_t pieces = (int32_t)((int64_t)row * esize_in / 16);
    hipLaunchKernelGGL(kv_copy16, dim3(grid_for(n * pieces)), dim3(256), 0, s, (const u32x4*)k,
                       (const u32x4*)v, slots, (u32x4*)kc, (u32x4*)vc, n, pieces, num_slots);
  } else if (in_dtype == 0 && cache_dtype == 0) {
    hipLaunchKernelGGL((kv_convert<float, float>), dim3(grid_for(n * row)), dim3(256), 0, s,
                       (const float*)k, (const float*)v, slots, (float*)kc, (float*)vc, n, row, num_slots);
  } else if (in_dtype == 0 && cache_dtype == 1) {
    hipLaunchKernelGGL((kv_convert<float, uint16_t>), dim3(grid_for(n * row)), dim3(256), 0, s,
                       (const float*)k, (const float*)v, slots, (uint16_t*)kc, (uint16_t*)vc, n, row,
                       num_slots);
  } else if (in_dtype == 1 && cache_dtype == 0) {
    hipLaunchKernelGGL((kv_convert<uint16_t, float>), dim3(grid_for(n * row)), dim3(256), 0, s,
                       (const uint16_t*)k, (const uint16_t*)v, slots, (float*)kc, (float*)vc, n, row,
                       num_slots);
  } else {
    hipLaunchKernelGGL((kv_convert<uint16_t, uint16_t>), dim3(grid_for(n * row)), dim3(256), 0, s,
                       (const uint16_t*)k, (const uint16_t*)v, slots, (uint16_t*)kc, (uint16_t*)vc, n,
                       row, num_slots);
  }
  return hipGetLastError();
}

hipError_t launch_kv_write_fp8(const void* k, const void* v, const int64_t* slots, void* kc, void* vc, float* ks,
                               float* vs, int64_t n, int32_t hkv, int32_t d, int64_t num_slots, int32_t in_dtype,
                               hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t rows = n * hkv;
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (in_dtype == 0)
    hipLaunchKernelGGL((kv_quant_fp8<float>), dim3((unsigned)blocks), dim3(256), 0, s, (const float*)k,
                       (const float*)v, slots, (uint8_t*)kc, (uint8_t*)vc, ks, vs, n, hkv, d, num_slots);
  else
    hipLaunchKernelGGL((kv_quant_fp8<uint16_t>), dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t*)k,
                       (const uint16_t*)v, slots, (uint8_t*)kc, (uint8_t*)vc, ks, vs, n, hkv, d, num_slots);
  return hipGetLastError();
}

}  // namespace pa
