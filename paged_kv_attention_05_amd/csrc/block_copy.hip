// Block copies between pools and staging buffers: swap_out (a preempted request's blocks to
// a host copy), swap_in (a saved copy into newly allocated blocks) and copy-on-write (a
// shared block into a private one before the step), from "Engine v2: one core for every
// request" (section "Preemption": swap_out / swap_in over the pool's blocks) and the
// vllm-lite README (copy-on-write of reference-counted blocks).
//
// One rule covers the three: for every pair i, block dst_block[i] of dst becomes block
// src_block[i] of src.  A block is block_bytes contiguous bytes (for a pool tensor
// [blocks, block_size, Hkv, D]: block_size * Hkv * D * element size).  Workgroup (i, c)
// copies chunk c of pair i, 256 threads x 16 bytes x kPer; src or dst may be host memory
// pinned with hipHostMalloc, which the kernel reads or writes over PCIe.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPer = 4;                                   // 16-byte pieces per thread and chunk
constexpr int64_t kChunkBytes = (int64_t)kThreads * 16 * kPer;

__global__ __launch_bounds__(kThreads) void copy_blocks16(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          const int64_t* __restrict__ src_block,
                                                          const int64_t* __restrict__ dst_block,
                                                          int64_t block_pieces) {
  const int64_t pair = blockIdx.x;
  const int64_t s = src_block[pair], d = dst_block[pair];
  const int64_t base = (int64_t)blockIdx.y * (kChunkBytes / 16);
  u32x4 x[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t e = base + threadIdx.x + (int64_t)k * kThreads;
    if (e < block_pieces) x[k] = __builtin_nontemporal_load(&src[s * block_pieces + e]);
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t e = base + threadIdx.x + (int64_t)k * kThreads;
    if (e < block_pieces) __builtin_nontemporal_store(x[k], &dst[d * block_pieces + e]);
  }
}

}  // namespace

hipError_t launch_copy_blocks(const void* src, void* dst, const int64_t* src_block, const int64_t* dst_block,
                              int64_t num_pairs, int64_t block_bytes, hipStream_t s) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = (block_bytes + kChunkBytes - 1) / kChunkBytes;
  if (num_pairs > INT32_MAX || chunks > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks16, dim3((unsigned)num_pairs, (unsigned)chunks), dim3(kThreads), 0, s,
                     (const u32x4*)src, (u32x4*)dst, src_block, dst_block, block_bytes / 16);
  return hipGetLastError();
}

}  // namespace pa
