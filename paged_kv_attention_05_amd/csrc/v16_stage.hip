// bf16 pools, prefill requests: a transposed fp16 copy of V for the prefill kernel.
//
// The prefill kernel's PV product runs on fp16 matrix cores, with V^T as the A operand: a
// lane holds 8 keys of one head dim.  V as the pool holds it is bf16, one row of D dims per
// key ("Attention over the pool" in "Engine v2: one core for every request" reads the
// pool's rows as they are), and every bf16 value with |v| <= 65504 converts to fp16
// exactly, except below 2^-14, where fp16 is subnormal and the value moves by at most
// 2^-25.  This kernel makes that conversion once per call, for the blocks of every
// prefill-path request that its 64-key tiles read (from v16_first_block on), into a
// contiguous staging area, transposed: request r's block j lands at staged block
// req[r].stage + j - first as [Hkv][D][16], each row holding the block's 16 keys in the
// order kperm, which is the order the kernel's P^T fragments hold them.  A lane's operand
// is then one 16-byte read.  Keys at or past the request's seq_len (the last tile's tail)
// are staged as zeros, so the kernel reads whole tiles and no unwritten slot reaches it.
//
// A block with a V value out of fp16's range (|v| > 65504, or an infinity) flags every
// prefill item of its request for that KV head; the bf16 prefill kernel, launched after the
// fp16 one, recomputes those items from the pool.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kStageD = 128;    // head dim of the prefill path

struct V16Args {
  const ReqOffsets* req;        // [R + 1]: .stage (first staged block), .pf (first item)
  const int32_t* table;         // the requests' pool block tables
  const int32_t* qsl;           // query_start_loc [R + 1]
  const int32_t* seq_lens;      // [R]
  int32_t R, stride, Hkv, window;
  int32_t n_pf;                 // prefill items (the flag array is [Hkv][n_pf])
  const uint16_t* vc;           // bf16 V pool [num_slots, Hkv, D]
  uint16_t* v16;                // transposed fp16 copy [n_stage][Hkv][D][16]
  int32_t* wide;                // per (KV head, item): 1 = recompute in bf16
};

// one workgroup (256 threads) per staged block, one KV head at a time: the head's 16 x 128
// values go through LDS (thread i loads 16 bytes of key i/16), then thread i writes dim i/2,
// positions 8(i%2) .. 8(i%2)+7 of the transposed row
__global__ __launch_bounds__(256) void stage_v16(V16Args s) {
  constexpr int D = kStageD;
  __shared__ float vals[16][D + 1];                          // one head: [key][dim], padded
  const int32_t b = blockIdx.x;
  if (b >= __builtin_amdgcn_readfirstlane(s.req[s.R].stage)) return;
  // owning request: the largest r with req[r].stage <= b (requests with no staged blocks
  // share their successor's offset, so the largest one is the owner)
  int lo = 0, hi = s.R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s.req[mid].stage <= b) lo = mid;
    else hi = mid - 1;
  }
  const int32_t r = __builtin_amdgcn_readfirstlane(lo);
  const int32_t t = s.qsl[r + 1] - s.qsl[r], L = s.seq_lens[r];
  const int32_t j = b - s.req[r].stage + v16_first_block(s.window, t, L);   // the request's block
  const int32_t nkeys = min(16, L - 16 * j);                 // keys of this block (<= 0: padding)
  const int32_t src = nkeys > 0 ? __builtin_amdgcn_readfirstlane(s.table[(int64_t)r * s.stride + j]) : 0;

  const int64_t row = (int64_t)s.Hkv * D;                   // elements per pool slot
  const int tid = threadIdx.x;
  const int lk = tid >> 4, lc = tid & 15;                    // load: key, 8-dim chunk
  const int od = tid >> 1, oh = tid & 1;                     // store: dim, half row
  for (int head = 0; head < s.Hkv; ++head) {
    float amax = 0.f;
    {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (lk < nkeys) w = *(const u32x4*)(s.vc + ((int64_t)src * 16 + lk) * row + (int64_t)head * D + 8 * lc);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo_f = __uint_as_float(w[k] << 16), hi_f = __uint_as_float(w[k] & 0xffff0000u);
        amax = fmaxf(amax, fmaxf(fabsf(lo_f), fabsf(hi_f)));
        vals[lk][8 * lc + 2 * k] = lo_f;
        vals[lk][8 * lc + 2 * k + 1] = hi_f;
      }
    }
    if (amax > 65504.f) {                                     // rare: flag the request's items
      for (int32_t it = s.req[r].pf; it < s.req[r + 1].pf; ++it) s.wide[(int64_t)head * s.n_pf + it] = 1;
    }
    __syncthreads();
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (_Float16)vals[kperm(8 * oh + e)][od];
    *(u32x4*)(s.v16 + (((int64_t)b * s.Hkv + head) * D + od) * 16 + 8 * oh) = __builtin_bit_cast(u32x4, o);
    __syncthreads();                                          // vals is refilled for the next head
  }
}

}  // namespace

hipError_t launch_stage_v16(const Plan& p, const AttnArgs& a, void* ws, hipStream_t st) {
  if (p.n_stage == 0) return hipSuccess;
  if (p.D != kStageD || p.bs != 16) return hipErrorInvalidValue;
  char* w = (char*)ws;
  V16Args s{};
  s.req = (const ReqOffsets*)(w + p.off_req);
  s.table = a.block_table;
  s.qsl = a.qsl;
  s.seq_lens = a.seq_lens;
  s.R = p.R; s.stride = a.stride; s.Hkv = p.Hkv; s.window = p.window;
  s.n_pf = (int32_t)p.n_pf;
  s.vc = (const uint16_t*)a.v_cache;
  s.v16 = (uint16_t*)(w + p.off_v16);
  s.wide = (int32_t*)(w + p.off_pf_wide);
  hipLaunchKernelGGL(stage_v16, dim3((unsigned)p.n_stage), dim3(256), 0, st, s);
  return hipGetLastError();
}

}  // namespace pa
