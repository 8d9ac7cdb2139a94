// Varlen work decomposition, computed on the device from query_start_loc and seq_lens.
//
// The batch layout of "Engine v2: one core for every request" (section "Flattened ragged
// batches") gives each request's rows and context length; the host copies exist so that
// launches need no device sync.  The host sizes the grids from those copies with the same
// per-request formula (request_counts), and this one-workgroup kernel writes the item lists
// the attention kernels read: no host-to-device copy, so the whole step stays on the stream.
//
// Requests are processed in chunks of 512: a block scan gives each request's offsets in
// the three lists, then every thread expands items of the chunk, finding the owning request
// by binary search over the chunk's offsets in LDS.
#include "pa_internal.h"

namespace pa {
namespace {

// 512 threads: at 1024 the kernel's registers spill to scratch and it takes twice as long
constexpr int kPlanThreads = 512;

// Inclusive scans of K counts per thread over the workgroup at once: within each wave by
// shuffles, then across the 8 waves through LDS (two barriers in all).  tot gets the
// workgroup totals.
template <int K>
__device__ __forceinline__ void block_scan_multi(int32_t (&v)[K], int32_t (&tot)[K], int32_t* wave_tot) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int32_t y = __shfl_up(v[k], off);
      if (lane >= off) v[k] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < K; ++k) wave_tot[wv * K + k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    int32_t pre = 0, all = 0;
    for (int j = 0; j < kPlanThreads / 64; ++j) {
      const int32_t x = wave_tot[j * K + k];
      pre += j < wv ? x : 0;
      all += x;
    }
    v[k] += pre;
    tot[k] = all;
  }
  __syncthreads();   // wave_tot is reused by the next chunk
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
                                                            int32_t* __restrict__ pf_wide,
                                                            SmallItem* __restrict__ g1,
                                                            SmallItem* __restrict__ g3) {
  __shared__ int32_t wave_tot[(kPlanThreads / 64) * 6];
  __shared__ int32_t o_small[kPlanThreads], o_merge[kPlanThreads], o_pf[kPlanThreads];
  __shared__ int32_t o_g1[kPlanThreads], o_g3[kPlanThreads];
  __shared__ int32_t c_t[kPlanThreads], c_ns[kPlanThreads], c_q0[kPlanThreads];
  __shared__ int32_t carry[6];
  const int tid = threadIdx.x;
  // the prefill kernel's per-workgroup "redo in bf16" flags start cleared every call
  for (int64_t i = tid; i < p.n_pf * p.Hkv; i += kPlanThreads) pf_wide[i] = 0;
  if (tid == 0) carry[0] = carry[1] = carry[2] = carry[3] = carry[4] = carry[5] = 0;
  __syncthreads();

  for (int base = 0; base < p.R; base += kPlanThreads) {
    const int r = base + tid;
    const int n = min(kPlanThreads, p.R - base);
    int32_t ns_small = 0, ns_merge = 0, ns_pf = 0, nsplit = 1, t = 0, ns_stage = 0, n_g1 = 0, n_g3 = 0, q0 = 0;
    if (r < p.R) {
      q0 = qsl[r];
      t = qsl[r + 1] - q0;
      // a call sized for a capacity: lengths past it (a caller's precondition violation)
      // are counted at the capacity, so the lists never outgrow what the host sized
      const int32_t L = p.graph_max > 0 ? min(seq_lens[r], p.graph_max) : seq_lens[r];
      request_counts(p, t, L, &ns_small, &ns_merge, &ns_pf, &nsplit);
      ns_stage = staged_blocks(p, t, L);
      small_groups(p, t, L, &n_g1, &n_g3);
    }
    const int32_t cs = carry[0], cm = carry[1], cp = carry[2], cg = carry[3], c1 = carry[4], c3 = carry[5];
    int32_t inc[6] = {ns_small, ns_merge, ns_pf, ns_stage, n_g1, n_g3}, tot[6];
    block_scan_multi<6>(inc, tot, wave_tot);
    const int32_t inc_s = inc[0], inc_m = inc[1], inc_p = inc[2], inc_g = inc[3], inc_1 = inc[4], inc_3 = inc[5];
    const int32_t tot_s = tot[0], tot_m = tot[1], tot_p = tot[2], tot_g = tot[3], tot_1 = tot[4], tot_3 = tot[5];
    o_g1[tid] = c1 + inc_1 - n_g1;
    o_g3[tid] = c3 + inc_3 - n_g3;
    o_small[tid] = cs + inc_s - ns_small;
    o_merge[tid] = cm + inc_m - ns_merge;
    o_pf[tid] = cp + inc_p - ns_pf;
    c_t[tid] = t;
    c_q0[tid] = q0;
    c_ns[tid] = nsplit;
    if (r < p.R) req[r] = ReqOffsets{o_small[tid], o_merge[tid], o_pf[tid], nsplit, cg + inc_g - ns_stage,
                                     o_g1[tid], o_g3[tid], 0};
    __syncthreads();
    if (tid == 0) {
      carry[0] = cs + tot_s;
      carry[1] = cm + tot_m;
      carry[2] = cp + tot_p;
      carry[3] = cg + tot_g;
      carry[4] = c1 + tot_1;
      carry[5] = c3 + tot_3;
    }
    __syncthreads();

    // expand this chunk's items (the per-tile list only for the vector kernel; the matrix-core
    // kernel reads the two lists below)
    for (int32_t idx = cs + tid; p.decode_kind != 1 && idx < cs + tot_s; idx += kPlanThreads) {
      const int i = find_owner(o_small, n, idx);
      small[idx] = single_item(p, base + i, idx - o_small[i], c_ns[i], o_small[i]);
    }
    // matrix-core lists: single tiles (one item per tile and split) ...
    for (int32_t idx = c1 + tid; p.decode_kind == 1 && idx < c1 + tot_1; idx += kPlanThreads) {
      const int i = find_owner(o_g1, n, idx);
      g1[idx] = single_item(p, base + i, idx - o_g1[i], c_ns[i], o_small[i]);
    }
    // ... and groups of up to kGroupTiles consecutive tiles (one item per group and split)
    for (int32_t idx = c3 + tid; p.decode_kind == 1 && idx < c3 + tot_3; idx += kPlanThreads) {
      const int i = find_owner(o_g3, n, idx);
      g3[idx] = group_item(p, base + i, idx - o_g3[i], c_ns[i], o_small[i], c_t[i]);
    }
    for (int32_t idx = cm + tid; idx < cm + tot_m; idx += kPlanThreads) {
      const int i = find_owner(o_merge, n, idx);
      merge[idx] = merge_item(p, base + i, idx - o_merge[i], c_ns[i], o_small[i], c_t[i], c_q0[i]);
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
  if (tid == 0) req[p.R] = ReqOffsets{carry[0], carry[1], carry[2], 0, carry[3], carry[4], carry[5], 0};
}

}  // namespace

hipError_t launch_plan(const Plan& p, const int32_t* qsl, const int32_t* seq_lens, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, p, qsl, seq_lens,
                     (ReqOffsets*)(w + p.off_req), (SmallItem*)(w + p.off_small),
                     (MergeItem*)(w + p.off_merge), (PfItem*)(w + p.off_pf), (int32_t*)(w + p.off_pf_wide),
                     (SmallItem*)(w + p.off_g1), (SmallItem*)(w + p.off_g3));
  return hipGetLastError();
}

}  // namespace pa
