// bf16 pools, prefill requests: an fp16 copy of V for the prefill kernel.
//
// The prefill kernel's PV product runs on fp16 matrix cores: V in fp16, P rounded to fp16.
// V as the pool holds it is bf16 ("Attention over the pool" in "Engine v2: one core for
// every request" reads the pool's rows as they are), and every bf16 value with
// |v| <= 65504 converts to fp16 exactly, except below 2^-14, where fp16 is subnormal and the
// value moves by at most 2^-25.  This kernel makes that conversion once per call for the
// blocks of every prefill-path request that its tiles read (all of them, or under a sliding
// window those from v16_first_block on), into a contiguous staging area: request r's block
// j lands at staged block req[r].stage + j - first (the planner's offsets), in the pool's
// own [block][16][Hkv][D] layout.  The prefill kernel then loads the fp16 rows straight
// into LDS and converts nothing itself.
//
// A block with a V value out of fp16's range (|v| > 65504, or an infinity) flags every
// prefill item of its request for that KV head; the bf16 prefill kernel, launched after the
// fp16 one, recomputes those items from the pool.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct V16Args {
  const ReqOffsets* req;        // [R + 1]: .stage (first staged block), .pf (first item)
  const int32_t* table;         // the requests' pool block tables
  const int32_t* qsl;           // query_start_loc [R + 1]
  const int32_t* seq_lens;      // [R]
  int32_t R, stride, Hkv, D, window;
  int32_t n_pf;                 // prefill items (the flag array is [Hkv][n_pf])
  const uint16_t* vc;           // bf16 V pool [num_slots, Hkv, D]
  uint16_t* v16;                // fp16 copy [n_stage * 16, Hkv, D]
  int32_t* wide;                // per (KV head, item): 1 = recompute in bf16
};

// one workgroup per staged block
__global__ __launch_bounds__(256) void stage_v16(V16Args s) {
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
  const int32_t j = b - s.req[r].stage + v16_first_block(s.window, t, L);
  const int32_t src = __builtin_amdgcn_readfirstlane(s.table[(int64_t)r * s.stride + j]);

  const int64_t row = (int64_t)s.Hkv * s.D;                 // elements per slot
  const int32_t chunks = 16 * (int32_t)(row / 8);           // 8-element chunks of the block
  const uint16_t* vsrc = s.vc + (int64_t)src * 16 * row;
  uint16_t* vdst = s.v16 + (int64_t)b * 16 * row;
  for (int32_t c = threadIdx.x; c < chunks; c += 256) {
    const u32x4 w = *(const u32x4*)(vsrc + 8 * (int64_t)c);
    u32x4 o;
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo_f = __uint_as_float(w[k] << 16), hi_f = __uint_as_float(w[k] & 0xffff0000u);
      amax = fmaxf(amax, fmaxf(fabsf(lo_f), fabsf(hi_f)));
      const f16x2 h2 = {(_Float16)lo_f, (_Float16)hi_f};
      o[k] = __builtin_bit_cast(uint32_t, h2);
    }
    *(u32x4*)(vdst + 8 * (int64_t)c) = o;
    if (amax > 65504.f) {                                   // rare: flag the request's items
      const int32_t head = (int32_t)((8 * (int64_t)c % row) / s.D);
      for (int32_t it = s.req[r].pf; it < s.req[r + 1].pf; ++it) s.wide[(int64_t)head * s.n_pf + it] = 1;
    }
  }
}

}  // namespace

hipError_t launch_stage_v16(const Plan& p, const AttnArgs& a, void* ws, hipStream_t st) {
  if (p.n_stage == 0) return hipSuccess;
  if ((int64_t)p.Hkv * p.D % 8 != 0) return hipErrorInvalidValue;
  char* w = (char*)ws;
  V16Args s{};
  s.req = (const ReqOffsets*)(w + p.off_req);
  s.table = a.block_table;
  s.qsl = a.qsl;
  s.seq_lens = a.seq_lens;
  s.R = p.R; s.stride = a.stride; s.Hkv = p.Hkv; s.D = p.D; s.window = p.window;
  s.n_pf = (int32_t)p.n_pf;
  s.vc = (const uint16_t*)a.v_cache;
  s.v16 = (uint16_t*)(w + p.off_v16);
  s.wide = (int32_t*)(w + p.off_pf_wide);
  hipLaunchKernelGGL(stage_v16, dim3((unsigned)p.n_stage), dim3(256), 0, st, s);
  return hipGetLastError();
}

}  // namespace pa
