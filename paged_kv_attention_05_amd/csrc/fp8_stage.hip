// fp8 pools, prefill requests: a staged bf16 copy for the prefill kernel.
//
// A quantized pool holds K/V as fp8 E4M3 codes with a float32 scale per (slot, KV head), the
// `cache[2:]` scales that "ReferenceBackend.dequantize" of "Engine v2: one core for every
// request" multiplies into the gathered rows.  The prefill kernel reads bf16 tiles; every
// E4M3 code is exactly a bf16 value (4 significant bits fit in 8), so each block of a
// prefill-path request is copied once per call into a contiguous staging area as bf16 codes
// (no scale applied: the copy is exact), and its scales are copied beside it, transposed to
// [block][K or V][KV head][slot] so that a tile's 64 scales of one head are four runs of 16
// floats.  The K scales are stored multiplied by |softmax scale| * log2(e), the factor the
// prefill kernel applies to every score; the attention arithmetic itself stays exact up to
// that float32 product.  The copy of request r starts at staged block req[r].stage (written
// by the planner) and a staged block table (row r: stage, stage + 1, ...) addresses it.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct StageArgs {
  const ReqOffsets* req;        // [R + 1], .stage: first staged block of each request
  const int32_t* table;         // the request's pool block table
  int32_t R, stride, W, Hkv, D;
  const uint8_t* kc;            // codes [num_slots, Hkv, D]
  const uint8_t* vc;
  const float* ks;              // scales [num_slots, Hkv]
  const float* vs;
  float kmul;                   // |scale| * log2(e), folded into the staged K scales
  uint16_t* k16;                // staged bf16 codes [n_stage * 16, Hkv, D]
  uint16_t* v16;
  float* sc;                    // staged scales [n_stage][2][Hkv][16]
  int32_t* tab;                 // staged block table [R, W]
};

// one workgroup per staged block
__global__ __launch_bounds__(256) void stage_fp8(StageArgs s) {
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
  const int32_t r = lo;
  const int32_t j = b - s.req[r].stage;
  const int32_t src = __builtin_amdgcn_readfirstlane(s.table[(int64_t)r * s.stride + j]);
  if (threadIdx.x == 0) s.tab[(int64_t)r * s.W + j] = b;

  const int64_t row = (int64_t)s.Hkv * s.D;                 // elements per slot
  const int32_t chunks = 16 * (int32_t)(row / 16);          // 16-code chunks of the block
  const uint8_t* ksrc = s.kc + (int64_t)src * 16 * row;
  const uint8_t* vsrc = s.vc + (int64_t)src * 16 * row;
  uint16_t* kdst = s.k16 + (int64_t)b * 16 * row;
  uint16_t* vdst = s.v16 + (int64_t)b * 16 * row;
  for (int32_t c = threadIdx.x; c < chunks; c += 256) {
    const u32x4 kw = *(const u32x4*)(ksrc + 16 * (int64_t)c);
    const u32x4 vw = *(const u32x4*)(vsrc + 16 * (int64_t)c);
    u32x4 ko[2], vo[2];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const pa_u32x2 k2 = fp8x4_to_bf16x4(kw[x]), v2 = fp8x4_to_bf16x4(vw[x]);
      ko[x >> 1][2 * (x & 1)] = k2[0];
      ko[x >> 1][2 * (x & 1) + 1] = k2[1];
      vo[x >> 1][2 * (x & 1)] = v2[0];
      vo[x >> 1][2 * (x & 1) + 1] = v2[1];
    }
    *(u32x4*)(kdst + 16 * (int64_t)c) = ko[0];
    *(u32x4*)(kdst + 16 * (int64_t)c + 8) = ko[1];
    *(u32x4*)(vdst + 16 * (int64_t)c) = vo[0];
    *(u32x4*)(vdst + 16 * (int64_t)c + 8) = vo[1];
  }
  const int32_t nsc = 2 * s.Hkv * 16;
  for (int32_t e = threadIdx.x; e < nsc; e += 256) {
    const int which = e / (s.Hkv * 16), h = (e / 16) % s.Hkv, i = e % 16;
    const int64_t si = ((int64_t)src * 16 + i) * s.Hkv + h;
    s.sc[(int64_t)b * nsc + e] = which == 0 ? s.ks[si] * s.kmul : s.vs[si];
  }
}

}  // namespace

hipError_t launch_stage_fp8(const Plan& p, const AttnArgs& a, float scale_abs_log2e, void* ws, hipStream_t st) {
  if (p.n_stage == 0) return hipSuccess;
  if ((int64_t)p.Hkv * p.D % 16 != 0) return hipErrorInvalidValue;
  char* w = (char*)ws;
  StageArgs s{};
  s.req = (const ReqOffsets*)(w + p.off_req);
  s.table = a.block_table;
  s.R = p.R; s.stride = a.stride; s.W = p.stage_w; s.Hkv = p.Hkv; s.D = p.D;
  s.kc = (const uint8_t*)a.k_cache; s.vc = (const uint8_t*)a.v_cache;
  s.ks = a.k_scale; s.vs = a.v_scale;
  s.kmul = scale_abs_log2e;
  s.k16 = (uint16_t*)(w + p.off_f8_k); s.v16 = (uint16_t*)(w + p.off_f8_v);
  s.sc = (float*)(w + p.off_f8_s);
  s.tab = (int32_t*)(w + p.off_f8_tab);
  hipLaunchKernelGGL(stage_fp8, dim3((unsigned)p.n_stage), dim3(256), 0, st, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the prefill kernel on the staged copy: bf16 codes, staged table, staged scales
  AttnArgs a8 = a;
  a8.k_cache = s.k16;
  a8.v_cache = s.v16;
  a8.block_table = s.tab;
  a8.stride = p.stage_w;
  a8.k_scale = s.sc;
  a8.v_scale = nullptr;
  return launch_prefill_mfma(p, a8, ws, st);
}

}  // namespace pa
