// Varlen work decomposition, computed on the device from query_start_loc and seq_lens.
//
// The batch layout of "Engine v2: one core for every request" (section "Flattened ragged
// batches") gives each request's rows and context length; the host copies exist so that
// launches need no device sync.  The host sizes the grids from those copies with the same
// per-request formula (request_counts), and this one-workgroup kernel writes the item lists
// the attention kernels read: no host-to-device copy, so the whole step stays on the stream.
//
// Requests are processed in chunks of 1024: a block scan gives each request's offsets in
// the three lists, then every thread expands items of the chunk, finding the owning request
// by binary search over the chunk's offsets in LDS.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int block_scan_inclusive(int32_t* buf, int32_t v) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int32_t add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  return buf[tid];
}

// largest i in [0, n) with off[i] <= idx (off non-decreasing, off[0] <= idx)
__device__ __forceinline__ int find_owner(const int32_t* off, int n, int32_t idx) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= idx) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Plan p, const int32_t* __restrict__ qsl,
                                                            const int32_t* __restrict__ seq_lens,
                                                            ReqOffsets* __restrict__ req,
                                                            SmallItem* __restrict__ small,
                                                            MergeItem* __restrict__ merge,
                                                            PfItem* __restrict__ pf,
                                                            int32_t* __restrict__ pf_wide) {
  __shared__ int32_t scan[kPlanThreads];
  __shared__ int32_t o_small[kPlanThreads], o_merge[kPlanThreads], o_pf[kPlanThreads];
  __shared__ int32_t c_t[kPlanThreads], c_ns[kPlanThreads];
  __shared__ int32_t carry[4];
  const int tid = threadIdx.x;
  // the prefill kernel's per-workgroup "redo in bf16" flags start cleared every call
  for (int64_t i = tid; i < p.n_pf * p.Hkv; i += kPlanThreads) pf_wide[i] = 0;
  if (tid == 0) carry[0] = carry[1] = carry[2] = carry[3] = 0;
  __syncthreads();

  for (int base = 0; base < p.R; base += kPlanThreads) {
    const int r = base + tid;
    const int n = min(kPlanThreads, p.R - base);
    int32_t ns_small = 0, ns_merge = 0, ns_pf = 0, nsplit = 1, t = 0, ns_stage = 0;
    if (r < p.R) {
      t = qsl[r + 1] - qsl[r];
      request_counts(p, t, seq_lens[r], &ns_small, &ns_merge, &ns_pf, &nsplit);
      ns_stage = staged_blocks(p, t, seq_lens[r]);
    }
    const int32_t cs = carry[0], cm = carry[1], cp = carry[2], cg = carry[3];
    const int32_t inc_s = block_scan_inclusive(scan, ns_small);
    const int32_t tot_s = scan[kPlanThreads - 1];
    __syncthreads();
    const int32_t inc_m = block_scan_inclusive(scan, ns_merge);
    const int32_t tot_m = scan[kPlanThreads - 1];
    __syncthreads();
    const int32_t inc_p = block_scan_inclusive(scan, ns_pf);
    const int32_t tot_p = scan[kPlanThreads - 1];
    __syncthreads();
    const int32_t inc_g = block_scan_inclusive(scan, ns_stage);
    const int32_t tot_g = scan[kPlanThreads - 1];
    o_small[tid] = cs + inc_s - ns_small;
    o_merge[tid] = cm + inc_m - ns_merge;
    o_pf[tid] = cp + inc_p - ns_pf;
    c_t[tid] = t;
    c_ns[tid] = nsplit;
    if (r < p.R) req[r] = ReqOffsets{o_small[tid], o_merge[tid], o_pf[tid], nsplit, cg + inc_g - ns_stage, 0, 0, 0};
    __syncthreads();
    if (tid == 0) {
      carry[0] = cs + tot_s;
      carry[1] = cm + tot_m;
      carry[2] = cp + tot_p;
      carry[3] = cg + tot_g;
    }
    __syncthreads();

    // expand this chunk's items
    for (int32_t idx = cs + tid; idx < cs + tot_s; idx += kPlanThreads) {
      const int i = find_owner(o_small, n, idx);
      const int32_t li = idx - o_small[i];
      const int32_t ns = c_ns[i];
      const int32_t tile = li / ns;
      SmallItem it;
      it.r = base + i;
      it.tok0 = (tile / p.hsubs) * p.tile_tokens;
      it.hsub = tile % p.hsubs;
      it.split = li - tile * ns;
      it.nsplit = ns;
      it.first = o_small[i] + tile * ns;
      it.pad0 = it.pad1 = 0;
      small[idx] = it;
    }
    for (int32_t idx = cm + tid; idx < cm + tot_m; idx += kPlanThreads) {
      const int i = find_owner(o_merge, n, idx);
      const int32_t tile = idx - o_merge[i];
      MergeItem it;
      it.r = base + i;
      it.tok0 = (tile / p.hsubs) * p.tile_tokens;
      it.hsub = tile % p.hsubs;
      it.first = o_small[i] + tile * c_ns[i];
      it.nsplit = c_ns[i];
      it.pad0 = it.pad1 = it.pad2 = 0;
      merge[idx] = it;
    }
    for (int32_t idx = cp + tid; idx < cp + tot_p; idx += kPlanThreads) {
      const int i = find_owner(o_pf, n, idx);
      const int32_t li = idx - o_pf[i];
      const int32_t tiles = (c_t[i] + p.pf_tokens - 1) / p.pf_tokens;
      PfItem it;
      it.r = base + i;
      it.tok0 = (tiles - 1 - li) * p.pf_tokens;      // longest (latest) tiles first
      pf[idx] = it;
    }
    __syncthreads();
  }
  if (tid == 0) req[p.R] = ReqOffsets{carry[0], carry[1], carry[2], 0, carry[3], 0, 0, 0};
}

}  // namespace

hipError_t launch_plan(const Plan& p, const int32_t* qsl, const int32_t* seq_lens, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, p, qsl, seq_lens,
                     (ReqOffsets*)(w + p.off_req), (SmallItem*)(w + p.off_small),
                     (MergeItem*)(w + p.off_merge), (PfItem*)(w + p.off_pf), (int32_t*)(w + p.off_pf_wide));
  return hipGetLastError();
}

}  // namespace pa
