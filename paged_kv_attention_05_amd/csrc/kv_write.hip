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

}  // namespace pa
