// fp8 pools, prefill requests: staged copies for the prefill kernels.
//
// A quantized pool holds K/V as fp8 E4M3 codes with a float32 scale per (slot, KV head), the
// `cache[2:]` scales that "ReferenceBackend.dequantize" of "Engine v2: one core for every
// request" multiplies into the gathered rows.  For every staged block of a prefill-path
// request (the blocks of each 64-key tile from v16_first_block on, zeros past seq_len:
// staged_blocks in pa_internal.h) one workgroup writes, per KV head:
//   - the K codes as bf16 rows, [staged block][16][Hkv][D] (exact: every E4M3 value is a
//     bf16 value), and the K scales times |softmax scale| * log2(e), the factor the prefill
//     kernel applies to every score, into [staged block][2][Hkv][16] (first half);
//   - V dequantized, code times scale rounded to fp16, into the transposed fp16 copy that
//     the fast prefill kernel reads for bf16 pools too ([staged block][Hkv][D][16], keys in
//     kperm order).  The float32 product and the rounding to fp16 move each value by at
//     most 2^-11 of itself plus 2^-24 (2^-25 below 2^-14);
//   - the V codes as bf16 rows and the V scales (second half of the scales), which only the
//     bf16 kernel reads: it redoes the items of a request whose dequantized V leaves fp16's
//     range (|v| > 65504), flagged here per request and KV head.
// Request r's block j is staged block req[r].stage + j - first (first = v16_first_block), so
// the kernels address staged blocks directly, with no table.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kStageD = 128;    // head dim of the prefill path

struct StageArgs {
  const ReqOffsets* req;        // [R + 1]: .stage (first staged block), .pf (first item)
  const int32_t* table;         // the requests' pool block tables
  const int32_t* qsl;           // query_start_loc [R + 1]
  const int32_t* seq_lens;      // [R]
  int32_t R, stride, Hkv, window;
  int32_t n_pf;                 // prefill items (the flag array is [Hkv][n_pf])
  const uint8_t* kc;            // codes [num_slots, Hkv, D]
  const uint8_t* vc;
  const float* ks;              // scales [num_slots, Hkv]
  const float* vs;
  float kmul;                   // |scale| * log2(e), folded into the staged K scales
  uint16_t* k16;                // staged bf16 K codes [n_stage * 16, Hkv, D]
  uint16_t* v16r;               // staged bf16 V codes, same layout
  float* sc;                    // staged scales [n_stage][2][Hkv][16]
  uint16_t* v16t;               // transposed fp16 V (codes times scales) [n_stage][Hkv][D][16]
  int32_t* wide;                // per (KV head, item): 1 = redo in bf16
};

// one workgroup (256 threads) per staged block, one KV head at a time: thread i handles key
// i/16, codes 8(i%16) .. 8(i%16)+7 of the row, then writes dim i/2, positions 8(i%2) ..
// 8(i%2)+7 of the transposed row
__global__ __launch_bounds__(256) void stage_fp8(StageArgs s) {
  constexpr int D = kStageD;
  __shared__ float vals[16][D + 1];                          // one head's dequantized V, padded
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

  const int64_t row = (int64_t)s.Hkv * D;                   // elements per slot
  const int tid = threadIdx.x;
  const int lk = tid >> 4, lc = tid & 15;                    // load: key, 8-code chunk
  const int od = tid >> 1, oh = tid & 1;                     // store: dim, half row
  for (int head = 0; head < s.Hkv; ++head) {
    u32x2 kw = {0u, 0u}, vw = {0u, 0u};
    float vsc = 0.f;
    const int64_t slot = (int64_t)src * 16 + lk;
    if (lk < nkeys) {
      kw = *(const u32x2*)(s.kc + slot * row + (int64_t)head * D + 8 * lc);
      vw = *(const u32x2*)(s.vc + slot * row + (int64_t)head * D + 8 * lc);
      vsc = s.vs[slot * s.Hkv + head];
    }
    const int64_t dst = ((int64_t)b * 16 + lk) * row + (int64_t)head * D + 8 * lc;
    const pa_u32x2 k0 = fp8x4_to_bf16x4(kw[0]), k1 = fp8x4_to_bf16x4(kw[1]);
    const pa_u32x2 v0 = fp8x4_to_bf16x4(vw[0]), v1 = fp8x4_to_bf16x4(vw[1]);
    *(u32x4*)(s.k16 + dst) = u32x4{k0[0], k0[1], k1[0], k1[1]};
    *(u32x4*)(s.v16r + dst) = u32x4{v0[0], v0[1], v1[0], v1[1]};
    // dequantized V: the float32 product of code and scale, rounded to fp16 below
    const uint32_t vb[4] = {v0[0], v0[1], v1[0], v1[1]};
    bool out_of_range = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo_f = __uint_as_float(vb[k] << 16) * vsc, hi_f = __uint_as_float(vb[k] & 0xffff0000u) * vsc;
      out_of_range |= !(fabsf(lo_f) <= 65504.f) || !(fabsf(hi_f) <= 65504.f);   // also catches NaN
      vals[lk][8 * lc + 2 * k] = lo_f;
      vals[lk][8 * lc + 2 * k + 1] = hi_f;
    }
    if (out_of_range) {                                       // rare: flag the request's items
      for (int32_t it = s.req[r].pf; it < s.req[r + 1].pf; ++it) s.wide[(int64_t)head * s.n_pf + it] = 1;
    }
    if (tid < 32) {                                           // K scales (tid < 16), then V
      const int key = tid & 15, which = tid >> 4;
      const int64_t si = ((int64_t)src * 16 + key) * s.Hkv + head;
      const float x = key < nkeys ? (which == 0 ? s.ks[si] * s.kmul : s.vs[si]) : 0.f;
      s.sc[(((int64_t)b * 2 + which) * s.Hkv + head) * 16 + key] = x;
    }
    __syncthreads();
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (_Float16)vals[kperm(8 * oh + e)][od];
    *(u32x4*)(s.v16t + (((int64_t)b * s.Hkv + head) * D + od) * 16 + 8 * oh) = __builtin_bit_cast(u32x4, o);
    __syncthreads();                                          // vals is refilled for the next head
  }
}

}  // namespace

hipError_t launch_stage_fp8(const Plan& p, const AttnArgs& a, float scale_abs_log2e, void* ws, hipStream_t st) {
  if (p.n_stage == 0) return hipSuccess;
  if (p.D != kStageD || p.bs != 16) return hipErrorInvalidValue;
  char* w = (char*)ws;
  StageArgs s{};
  s.req = (const ReqOffsets*)(w + p.off_req);
  s.table = a.block_table;
  s.qsl = a.qsl;
  s.seq_lens = a.seq_lens;
  s.R = p.R; s.stride = a.stride; s.Hkv = p.Hkv; s.window = p.window;
  s.n_pf = (int32_t)p.n_pf;
  s.kc = (const uint8_t*)a.k_cache; s.vc = (const uint8_t*)a.v_cache;
  s.ks = a.k_scale; s.vs = a.v_scale;
  s.kmul = scale_abs_log2e;
  s.k16 = (uint16_t*)(w + p.off_f8_k);
  s.v16r = (uint16_t*)(w + p.off_f8_v);
  s.sc = (float*)(w + p.off_f8_s);
  s.v16t = (uint16_t*)(w + p.off_v16);
  s.wide = (int32_t*)(w + p.off_pf_wide);
  hipLaunchKernelGGL(stage_fp8, dim3((unsigned)p.n_stage), dim3(256), 0, st, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the prefill kernels on the staged copies: bf16 K codes, scales, the fp16 V copy (and the
  // bf16 V codes for the redo kernel), all at staged block numbers
  AttnArgs a8 = a;
  a8.k_cache = s.k16;
  a8.v_cache = s.v16r;
  a8.v_staged = s.v16t;
  a8.k_scale = s.sc;
  a8.v_scale = nullptr;
  a8.req = (const ReqOffsets*)(w + p.off_req);
  return launch_prefill_mfma(p, a8, ws, st);
}

}  // namespace pa
