// Prefill-chunk paged attention on bf16 matrix cores.
//
// A request whose rows times grouped heads exceed 16 query columns (a prefill chunk) is cut
// into tiles of 128 query rows: 128 / g consecutive tokens times the g query heads of one KV
// head.  Packing the group's heads into one tile means every K/V tile brought on chip serves
// all g heads (grouped-query attention without repeating K/V, as the vllm-lite README's fold
// does for its CPU path).  The causal mask is offset by the request's computed tokens: row i
// of a request with seq_len L and t rows sits at position L - t + i ("Attention over the
// pool" in "Engine v2: one core for every request").  K/V are read in place through the block
// table, 64 keys (four 16-token blocks) at a time, staged in LDS; the online softmax keeps
// exact attention without a score matrix in memory (the FlashAttention section of the
// tensorsofthewall.com post).
//
// Workgroup: 4 waves, wave w owns tile rows 32w .. 32w+31 (one row per lane column).
//   S^T[key][row] = K[key][:] . Q[row][:]    mfma_f32_32x32x16_bf16, K from LDS (A operand,
//                                            one 16-byte read per lane), Q^T in registers.
//   O^T[d][row]  += V^T[d][key] P^T[key][row] mfma_f32_32x32x16_bf16; P^T is taken from the S^T
//                                            accumulators with the key index bit-permuted
//                                            (bits 2 and 3 swapped inside each 16-key chunk),
//                                            and V^T is read from LDS with the same permutation
//                                            by two gfx950 transpose reads (ds_read_tr16_b64).
// The next K/V tile is loaded into registers while the current one is computed.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kBK = 64;          // keys per K/V tile
constexpr int kRows = 128;       // query rows per workgroup
constexpr int kBlk = 16;         // block_size

template <int D>
struct PrefillCfg {
  static constexpr int PK = D + 8;            // K row pitch (elements): conflict-free 16-byte reads
  static constexpr int PV = D + 32;           // V row pitch: conflict-free transpose reads
  static constexpr int PO = D + 8;            // output staging pitch
  static constexpr int KC = D / 16;           // k-chunks of QK^T
  static constexpr int DT = D / 32;           // 32-wide d tiles of PV
  static constexpr int PIECES = D / 8;        // 16-byte pieces per row
  static constexpr int LOADS = kBK * PIECES / 256;   // 16-byte loads per thread per K (or V) tile
  static constexpr int K_BYTES = kBK * PK * 2;
  static constexpr int V_BYTES = kBK * PV * 2;
  static constexpr int O_BYTES = kRows * PO * 2;
  static constexpr int SMEM = (K_BYTES + V_BYTES) > O_BYTES ? (K_BYTES + V_BYTES) : O_BYTES;
};

__device__ __forceinline__ bf16x4 tr_read(const __bf16* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) void*)p));
  return __builtin_bit_cast(bf16x4, r);
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_tile_mfma(AttnArgs a, const PfItem* __restrict__ items) {
  using C = PrefillCfg<D>;
  __shared__ __align__(16) unsigned char smem[C::SMEM];
  __bf16* Ks = (__bf16*)smem;
  __bf16* Vs = (__bf16*)(smem + C::K_BYTES);

  const PfItem it = items[blockIdx.x];
  const int hkv = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int BQ = kRows / a.g;                                 // tokens per tile
  const int32_t b = a.qsl[it.r], t = a.qsl[it.r + 1] - b, L = a.seq_lens[it.r], c = L - t;
  const int32_t tok0 = it.tok0;
  const int32_t Tn = min(BQ, t - tok0);
  const int32_t kend = c + tok0 + Tn;                         // one past the last visible key
  const int32_t* table_row = a.block_table + (int64_t)it.r * a.stride;
  const int64_t row_elems = (int64_t)a.Hkv * D;
  const __bf16* kc = (const __bf16*)a.k_cache + (int64_t)hkv * D;
  const __bf16* vc = (const __bf16*)a.v_cache + (int64_t)hkv * D;

  // this lane's query row
  const int m_row = 32 * w + n;
  const int head_l = m_row / BQ, token = m_row - head_l * BQ;
  const bool row_ok = token < Tn;
  const int32_t pos = c + tok0 + token;
  bf16x8 qf[C::KC];
  {
    const __bf16* qp = (const __bf16*)a.q + ((int64_t)(b + tok0 + token) * a.H + hkv * a.g + head_l) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < C::KC; ++kk) qf[kk] = row_ok ? *(const bf16x8*)(qp + 16 * kk) : bf16x8{};
  }

  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x16{};
  float m = kNegInf, lsum = 0.f;
  const float sl = a.scale_log2e;

  const int32_t ntiles = (kend + kBK - 1) / kBK;
  u32x4 kr[C::LOADS], vr[C::LOADS];
  auto load_tile = [&](int32_t j) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int ci = tid + 256 * u;
      const int key = ci / C::PIECES, piece = ci - key * C::PIECES;
      const int32_t kg = j * kBK + key;
      if (kg < kend) {
        const int64_t slot = (int64_t)table_row[kg / kBlk] * kBlk + (kg % kBlk);
        kr[u] = *(const u32x4*)(kc + slot * row_elems + 8 * piece);
        vr[u] = *(const u32x4*)(vc + slot * row_elems + 8 * piece);
      } else {
        kr[u] = u32x4{0u, 0u, 0u, 0u};   // past the visible keys: zero (pool tails may hold NaN)
        vr[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int ci = tid + 256 * u;
      const int key = ci / C::PIECES, piece = ci - key * C::PIECES;
      *(u32x4*)(Ks + key * C::PK + 8 * piece) = kr[u];
      *(u32x4*)(Vs + key * C::PV + 8 * piece) = vr[u];
    }
  };

  load_tile(0);
  store_tile();
  __syncthreads();

  for (int32_t j = 0; j < ntiles; ++j) {
    if (j + 1 < ntiles) load_tile(j + 1);

    // S^T for keys 64j .. 64j+63 in two halves of 32
    f32x16 s[2];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      s[sh] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C::KC; ++kk) {
        const bf16x8 ka = *(const bf16x8*)(Ks + (32 * sh + n) * C::PK + 16 * kk + 8 * h);
        s[sh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[sh], 0, 0, 0);
      }
    }

    // scale (base 2), causal mask near the diagonal, running max
    const bool need_mask = (j * kBK + kBK - 1 > c + tok0) || (Tn < BQ);
    float mx = kNegInf;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[sh][r] * sl;
        if (need_mask) {
          const int32_t key = j * kBK + 32 * sh + 8 * (r >> 2) + 4 * h + (r & 3);
          if (!row_ok || key > pos) x = kNegInf;
        }
        s[sh][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    m = m_new;
    bf16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = exp2f(s[sh][8 * kh + jj] - m_use);
          psum += p;
          pb[2 * sh + kh][jj] = (__bf16)p;
        }
      }
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;

    // O^T += V^T P^T over the four 16-key chunks
    const int G = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int col = 32 * dt + 16 * (G & 1) + 4 * (i16 & 3);
#pragma unroll
      for (int qc = 0; qc < 4; ++qc) {
        const int row = 16 * qc + 4 * h + (i16 >> 2);
        const bf16x4 v0 = tr_read(Vs + row * C::PV + col);
        const bf16x4 v1 = tr_read(Vs + (row + 8) * C::PV + col);
        const bf16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qc], o[dt], 0, 0, 0);
      }
    }

    __syncthreads();                 // every wave is done with this tile
    if (j + 1 < ntiles) {
      store_tile();
      __syncthreads();
    }
  }

  // normalise and stage the tile's output rows in LDS, then write them out coalesced
  lsum += __shfl_xor(lsum, 32);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  __bf16* Os = (__bf16*)smem;
  __syncthreads();
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * dt + 8 * (r >> 2) + 4 * h + (r & 3);
      Os[m_row * C::PO + d] = (__bf16)(o[dt][r] * inv);
    }
  }
  __syncthreads();
  __bf16* out = (__bf16*)a.out;
  for (int ci = tid; ci < kRows * C::PIECES; ci += 256) {
    const int mr = ci / C::PIECES, piece = ci - mr * C::PIECES;
    const int hl = mr / BQ, tk = mr - hl * BQ;
    if (tk >= Tn) continue;
    *(u32x4*)(out + ((int64_t)(b + tok0 + tk) * a.H + hkv * a.g + hl) * D + 8 * piece) =
        *(const u32x4*)(Os + mr * C::PO + 8 * piece);
  }
}

}  // namespace

bool prefill_mfma_supported(int32_t D, int32_t bs, int32_t g) {
  return bs == kBlk && (D == 64 || D == 128) && g >= 1 && g <= kRows && kRows % g == 0;
}

int32_t prefill_tile_tokens(int32_t g) { return kRows / g; }

hipError_t launch_prefill_mfma(const Plan& p, const AttnArgs& a, void* ws, hipStream_t s) {
  if (p.n_pf == 0) return hipSuccess;
  const PfItem* items = (const PfItem*)((char*)ws + p.off_pf);
  const dim3 grid((unsigned)p.n_pf, (unsigned)p.Hkv);
  if (p.D == 128) hipLaunchKernelGGL(prefill_tile_mfma<128>, grid, dim3(256), 0, s, a, items);
  else if (p.D == 64) hipLaunchKernelGGL(prefill_tile_mfma<64>, grid, dim3(256), 0, s, a, items);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
