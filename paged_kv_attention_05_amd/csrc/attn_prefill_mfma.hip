// Prefill-chunk paged attention on bf16 matrix cores.
//
// A request whose rows times grouped heads exceed 16 query columns (a prefill chunk) is cut
// into tiles of 32 * WAVES query rows: (32 * WAVES) / g consecutive tokens times the g query
// heads of one KV head.  Packing the group's heads into one tile means every K/V tile brought
// on chip serves all g heads (grouped-query attention without repeating K/V, as the
// vllm-lite README's fold does for its CPU path).  The causal mask is offset by the request's
// computed tokens: row i of a request with seq_len L and t rows sits at position L - t + i
// ("Attention over the pool" in "Engine v2: one core for every request").  K/V are read in
// place through the block table, 64 keys (four 16-token blocks) at a time; the online
// softmax keeps exact attention without a score matrix in memory (the FlashAttention section
// of the tensorsofthewall.com post).
//
// Data movement: each 64-key K and V tile goes from HBM straight into LDS with the gfx950
// direct loads (global_load_lds_dwordx4, 16 bytes per lane, no register staging), into
// double buffers, so the next tiles stream in while the current one is computed (one
// workgroup barrier per tile).  An LDS row is one key's 256 bytes; its sixteen 16-byte
// chunks are stored XOR-swizzled (chunk c of row r at slot c ^ f(r), f(r) = 4*(r%4) +
// (r/4)%4), which makes both the K reads (16 consecutive rows, one chunk) and the V transpose
// reads (4 rows x 4 chunks) free of bank conflicts.
//
// Compute: wave w owns tile rows 32w .. 32w+31, one row per lane column.
//   S^T[key][row] = K[key][:] . Q[row][:]     mfma_f32_32x32x16_bf16, K from LDS (A operand,
//                                             one 16-byte read per lane), Q^T in registers.
//   O^T[d][row]  += V^T[d][key] P^T[key][row]  mfma_f32_32x32x16_bf16; P^T is the S^T
//                                             accumulator layout with the key index
//                                             bit-permuted (bits 2 and 3 swapped in each
//                                             16-key chunk); V^T comes from LDS with the same
//                                             permutation through two ds_read_tr16_b64.
// The loop is software-pipelined: the QK^T products of tile j+1 are issued before the softmax
// of tile j, so the matrix cores and the vector ALUs work at the same time.
// Softmax per row in base 2: one FMA and one v_exp_f32 per score; the running max is only
// moved (and O rescaled) when a row's max grows by more than 8 (a factor 256), so rescaling
// is rare; the sum uses the same reference, so the result is exact either way.
// P is carried as a bf16 pair (truncated high part plus the bf16 rounding of the exact
// remainder), two products per chunk: ~16 significant bits, where a single bf16 P loses up
// to 2^-9 of a weight, which against ~10x outlier values exceeds 2e-2.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kBK = 64;          // keys per K/V tile
constexpr int kBlk = 16;         // block_size
constexpr float kLazy = 8.0f;    // base-2 headroom before the running max is moved

template <int D>
struct PrefillCfg {
  static constexpr int ROW = D * 2;                 // bytes per key row in LDS
  static constexpr int CHUNKS = ROW / 16;           // 16-byte chunks per row
  static constexpr int TILE = kBK * ROW;            // bytes of one K (or V) tile
  static constexpr int KC = D / 16;                 // k-chunks of QK^T
  static constexpr int DT = D / 32;                 // 32-wide d tiles of PV
};

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ bf16x4 tr_read(const unsigned char* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) void*)p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ void load_lds16(const void* g, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void prefill_tile_mfma(AttnArgs a, const PfItem* __restrict__ items,
                                                                            int32_t n_items) {
  using C = PrefillCfg<D>;
  constexpr int ROWS = 32 * WAVES;
  constexpr int NT = 64 * WAVES;
  // two K tiles and two V tiles; the output staging reuses the same bytes
  constexpr int OUT_BYTES = ROWS * C::ROW;
  constexpr int SMEM = (4 * C::TILE) > OUT_BYTES ? (4 * C::TILE) : OUT_BYTES;
  __shared__ __align__(1024) unsigned char smem[SMEM];

  // workgroup -> (item, KV head): consecutive items of one head on one XCD (workgroups are
  // dealt round-robin over the 8 XCDs), so tiles sweeping the same K/V share its L2
  const int32_t total = n_items * a.Hkv;
  const int32_t per_xcd = (total + 7) / 8;
  const int32_t lin = (int32_t)(blockIdx.x % 8) * per_xcd + (int32_t)(blockIdx.x / 8);
  if (lin >= total) return;
  const int hkv = lin / n_items;
  const PfItem it = items[lin - hkv * n_items];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave id: uniform
  const int n = lane & 31, h = lane >> 5;
  const int BQ = ROWS / a.g;                                  // tokens per tile
  // request metadata is the same for the whole workgroup: keep it in scalar registers so
  // every tile bound and branch below is scalar
  const int32_t r_id = __builtin_amdgcn_readfirstlane(it.r);
  const int32_t b = __builtin_amdgcn_readfirstlane(a.qsl[r_id]);
  const int32_t t = __builtin_amdgcn_readfirstlane(a.qsl[r_id + 1]) - b;
  const int32_t L = __builtin_amdgcn_readfirstlane(a.seq_lens[r_id]);
  const int32_t c = L - t;
  const int32_t tok0 = __builtin_amdgcn_readfirstlane(it.tok0);
  const int32_t Tn = min(BQ, t - tok0);
  const int32_t kend = c + tok0 + Tn;                         // one past the last visible key
  const int32_t* table_row = a.block_table + (int64_t)r_id * a.stride;
  const int64_t row_elems = (int64_t)a.Hkv * D;
  const __bf16* kc = (const __bf16*)a.k_cache + (int64_t)hkv * D;
  const __bf16* vc = (const __bf16*)a.v_cache + (int64_t)hkv * D;

  // this lane's query row; a negative scale is applied as |scale| on -q
  const int m_row = 32 * w + n;
  const int head_l = m_row / BQ, token = m_row - head_l * BQ;
  const bool row_ok = token < Tn;
  const int32_t pos = c + tok0 + token;
  const float sl = fmaxf(fabsf(a.scale_log2e), 1e-30f);
  const uint32_t qsign = a.scale_log2e < 0.f ? 0x80008000u : 0u;
  bf16x8 qf[C::KC];
  {
    const __bf16* qp = (const __bf16*)a.q + ((int64_t)(b + tok0 + token) * a.H + hkv * a.g + head_l) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < C::KC; ++kk) {
      u32x4 v = row_ok ? *(const u32x4*)(qp + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
      v ^= qsign;
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // direct loads of one tile: instruction u of wave w fills LDS rows 4I .. 4I+3 (I = w +
  // WAVES*u) of the K and V tiles; lane l takes row r = 4I + l/16, slot l%16, which holds
  // chunk (l%16) ^ swz(r).  A lane's row within its 16-key block and its chunk are the same
  // for every instruction, so a full tile costs one table lookup per block.  Keys at or past
  // kend (last tile only) read key kend-1 instead: finite data, masked out.
  constexpr int UK = kBK / 4 / WAVES;                         // instructions per wave per tile
  const int32_t ntiles = (kend + kBK - 1) / kBK;
  const int rowoff = (4 * w + (lane >> 4)) & 15;
  const int chunk_sw = (lane & 15) ^ swz(rowoff);
  const int64_t lane_off = (int64_t)rowoff * row_elems + 8 * chunk_sw;
  const int64_t blk_stride = (int64_t)kBlk * row_elems;
  // Block ids of a full tile (4 consecutive table entries, wave-uniform) are fetched one
  // iteration before they are needed, so no load waits on a table lookup; only the last,
  // partial tile computes clamped per-lane keys.
  struct Blocks { int32_t b0, b1, b2, b3; };
  auto fetch_blocks = [&](int32_t j) -> Blocks {
    if (j * kBK + kBK > kend) return Blocks{0, 0, 0, 0};     // partial tile: not used
    const int32_t* e = table_row + 4 * j;
    return Blocks{e[0], e[1], e[2], e[3]};
  };
  // block of instruction u within the tile: wave-uniform ((w + WAVES*u) / 4)
  auto pick = [&](const Blocks& bl, int u) -> int32_t {
    const int bi = WAVES == 4 ? u : ((w >> 2) + (WAVES / 4) * u);
    return bi == 0 ? bl.b0 : bi == 1 ? bl.b1 : bi == 2 ? bl.b2 : bl.b3;
  };
  auto issue = [&](const __bf16* base, int32_t j, const Blocks& bl, unsigned char* dst) {
    if (j * kBK + kBK <= kend) {
#pragma unroll
      for (int u = 0; u < UK; ++u)
        load_lds16(base + ((int64_t)pick(bl, u) * blk_stride + lane_off), dst + (w + WAVES * u) * 1024);
    } else {
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        const int32_t kg = min(j * kBK + 4 * (w + WAVES * u) + (lane >> 4), kend - 1);
        const int64_t off = ((int64_t)table_row[kg >> 4] * kBlk + (kg & 15)) * row_elems + 8 * chunk_sw;
        load_lds16(base + off, dst + (w + WAVES * u) * 1024);
      }
    }
  };
  auto issue_k = [&](int32_t j, const Blocks& bl, unsigned char* dst) { issue(kc, j, bl, dst); };
  auto issue_v = [&](int32_t j, const Blocks& bl, unsigned char* dst) { issue(vc, j, bl, dst); };

  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x16{};
  float m = kNegInf, lsum = 0.f;
  const int G = lane >> 4, i16 = lane & 15;

  // S^T of one K tile (keys 64j .. 64j+63, two halves of 32 keys)
  // (the two halves alternate, so consecutive matrix instructions are independent)
  auto qk = [&](const unsigned char* Ks, f32x16* s) {
    const int sw = swz(n);                                  // swz(32 + n) == swz(n)
#pragma unroll
    for (int kk = 0; kk < C::KC; ++kk) {
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const bf16x8 ka = *(const bf16x8*)(Ks + (32 * sh + n) * C::ROW + 16 * ((2 * kk + h) ^ sw));
        s[sh] = kk == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], f32x16{}, 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[sh], 0, 0, 0);
      }
    }
  };

  // Software pipeline: K runs one tile ahead of V.  Iteration j holds K(j+1) and V(j) in LDS,
  // starts the loads of K(j+2) and V(j+1), computes S(j+1) on the matrix cores while the
  // vector ALUs turn S(j) into probabilities, then accumulates V(j) P(j).  Buffers: K tile
  // j in kbuf(j % 2), V tile j in vbuf(j % 2); one barrier per iteration.
  auto kbuf = [&](int i) { return smem + i * C::TILE; };
  auto vbuf = [&](int i) { return smem + (2 + i) * C::TILE; };
  Blocks bl0 = fetch_blocks(0), bl1 = fetch_blocks(1);
  issue_k(0, bl0, kbuf(0));
  issue_v(0, bl0, vbuf(0));
  if (ntiles > 1) issue_k(1, bl1, kbuf(1));
  Blocks blV = bl1;                                        // blocks of V(j+1)
  Blocks blK = fetch_blocks(2);                            // blocks of K(j+2)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 s_cur[2];
  qk(kbuf(0), s_cur);
  __syncthreads();                                          // K(0) read by all before K(2) lands there

  for (int32_t j = 0; j < ntiles; ++j) {
    if (j + 2 < ntiles) issue_k(j + 2, blK, kbuf(j & 1));
    if (j + 1 < ntiles) issue_v(j + 1, blV, vbuf((j + 1) & 1));
    blV = blK;
    blK = fetch_blocks(j + 3);
    f32x16 s_next[2];
    if (j + 1 < ntiles) qk(kbuf((j + 1) & 1), s_next);

    // causal mask on the diagonal tiles only; masked scores are -inf before the max
    if (j * kBK + kBK - 1 > c + tok0 || Tn < BQ) {
      const int32_t lim = row_ok ? pos - j * kBK - 4 * h : -1000000;
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * sh + 8 * (r >> 2) + (r & 3);
          s_cur[sh][r] = off > lim ? kNegInf : s_cur[sh][r];
        }
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s_cur[sh][r], s_cur[sh][r + 1]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxs = mx * sl;                              // mx is finite or -inf, sl > 0
    // move the reference only when the row max grew by more than kLazy (or it is unset)
    if (__builtin_amdgcn_ballot_w64(mxs > m + kLazy) != 0) {
      const float m_new = mxs > m + kLazy ? mxs : m;
      const float alpha = m_new > m ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;   // m may be -inf
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
    }
    const float m_use = m == kNegInf ? 0.f : m;

    u32x4 pb[4], pl[4];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[sh][8 * kh + jj], sl, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[sh][8 * kh + jj + 1], sl, -m_use));
          lsum += p0 + p1;
          const uint32_t h0 = __float_as_uint(p0) & 0xffff0000u, h1 = __float_as_uint(p1) & 0xffff0000u;
          const float r0 = p0 - __uint_as_float(h0), r1 = p1 - __uint_as_float(h1);
          pb[2 * sh + kh][jj >> 1] = __builtin_amdgcn_perm(h1, h0, 0x07060302u);   // {h0.hi16, h1.hi16}
          const bf16x2 lo = {(__bf16)r0, (__bf16)r1};
          pl[2 * sh + kh][jj >> 1] = __builtin_bit_cast(uint32_t, lo);
        }
      }
    }

    // O^T += V^T P^T over the four 16-key chunks
    const unsigned char* Vs = vbuf(j & 1);
    // (per 16-key chunk: the four d tiles' high-part products, then their low-part products,
    // so consecutive matrix instructions accumulate into different tiles)
    const int sub = 8 * (i16 & 1);
#pragma unroll
    for (int qc = 0; qc < 4; ++qc) {
      const int r0 = 16 * qc + 4 * h + (i16 >> 2);
      const int r1 = r0 + 8;
      bf16x8 va[C::DT];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const int chunk = 4 * dt + 2 * (G & 1) + ((i16 & 3) >> 1);
        const bf16x4 v0 = tr_read(Vs + r0 * C::ROW + 16 * (chunk ^ swz(r0)) + sub);
        const bf16x4 v1 = tr_read(Vs + r1 * C::ROW + 16 * (chunk ^ swz(r1)) + sub);
        va[dt] = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], __builtin_bit_cast(bf16x8, pb[qc]), o[dt], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], __builtin_bit_cast(bf16x8, pl[qc]), o[dt], 0, 0, 0);
    }
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // K(j+2), V(j+1) have landed
    __syncthreads();                                        // ... for every thread; tile j consumed
  }

  // normalise and stage the tile's output rows in LDS, then write them out coalesced
  lsum += __shfl_xor(lsum, 32);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  __syncthreads();                                          // all waves done with the K/V tiles
  __bf16* Os = (__bf16*)smem;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * dt + 8 * (r >> 2) + 4 * h + (r & 3);
      // same chunk swizzle on the staging rows keeps these 2-byte stores spread over banks
      const int chunk = (d >> 3) ^ (m_row & 15);
      Os[m_row * D + 8 * chunk + (d & 7)] = (__bf16)(o[dt][r] * inv);
    }
  }
  __syncthreads();
  __bf16* out = (__bf16*)a.out;
  for (int ci = tid; ci < ROWS * C::CHUNKS; ci += NT) {
    const int mr = ci / C::CHUNKS, chunk = ci - mr * C::CHUNKS;
    const int hl = mr / BQ, tk = mr - hl * BQ;
    if (tk >= Tn) continue;
    *(u32x4*)(out + ((int64_t)(b + tok0 + tk) * a.H + hkv * a.g + hl) * D + 8 * chunk) =
        *(const u32x4*)(Os + mr * D + 8 * (chunk ^ (mr & 15)));
  }
}

constexpr int kWaves = 8;

}  // namespace

// The LDS row layout (one 256-byte key row, sixteen swizzled chunks) is built for head_dim
// 128; other head sizes take the small-tile kernels.
bool prefill_mfma_supported(int32_t D, int32_t bs, int32_t g) {
  return bs == kBlk && D == 128 && g >= 1 && g <= 32 * kWaves && (32 * kWaves) % g == 0;
}

int32_t prefill_tile_tokens(int32_t g) { return 32 * kWaves / g; }

hipError_t launch_prefill_mfma(const Plan& p, const AttnArgs& a, void* ws, hipStream_t s) {
  if (p.n_pf == 0) return hipSuccess;
  const PfItem* items = (const PfItem*)((char*)ws + p.off_pf);
  const int64_t total = p.n_pf * p.Hkv;
  const dim3 grid((unsigned)((total + 7) / 8 * 8));
  if (p.D != 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_tile_mfma<128, kWaves>), grid, dim3(64 * kWaves), 0, s, a, items, (int32_t)p.n_pf);
  return hipGetLastError();
}

}  // namespace pa
