// Measurement only: a streaming read of a device buffer, the achievable HBM read rate that
// the decode kernels (which read each live K/V row once) are measured against beside the
// 8 TB/s specification.  Not part of the attention path.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// grid-stride over 16-byte words with nontemporal loads; the xor of everything read is
// written only if it equals an unlikely value, which keeps the loads alive
__global__ __launch_bounds__(256) void read_probe(const u32x4* __restrict__ p, int64_t n, uint32_t* sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, hipStream_t s) {
  hipLaunchKernelGGL(read_probe, dim3((unsigned)grid), dim3(256), 0, s, (const u32x4*)buf, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pa
