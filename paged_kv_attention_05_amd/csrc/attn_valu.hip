// Paged varlen attention on the vector ALUs: the path for float32 pools and for shapes the
// bf16 matrix-core kernels do not take, and the split-K merge shared by every small tile.
//
// Computes ReferenceBackend.forward of "Engine v2: one core for every request" (section
// "Attention over the pool"): row i of request r is at position seq_len - t + i and attends
// keys 0 .. that position, read in place through the block table (slot = table[p / bs] * bs
// + p % bs), with query heads grouped contiguously onto KV heads.  Softmax is the online
// (rescaled running max) form, so no score matrix is ever stored ("FlashAttention is not
// PagedAttention" in the tensorsofthewall.com post: exact attention without materialising
// the attention matrix).
//
// One workgroup (4 waves) takes one small tile: up to 16 query columns (token, head) of one
// request and one KV head, over one split of the keys.  Wave w takes 16-key chunks w, w+4,
// ...; lane (G = lane / 16, n = lane % 16) scores keys 4G..4G+3 of the chunk against column
// n and accumulates column n's output for head_dim slice G.  The four waves' running
// (max, sum, output) are combined in LDS; a tile with several splits writes partials that
// the merge kernel combines with the log-sum-exp rule.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
    const float4 v = *(const float4*)p;
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct Vec4<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* o) {
    const uint2 v = *(const uint2*)p;
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};

__device__ __forceinline__ int64_t slot_of(const int32_t* table_row, int32_t key, int32_t bs) {
  return (int64_t)table_row[key / bs] * bs + key % bs;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void small_tile_valu(AttnArgs a, const SmallItem* __restrict__ items,
                                                       Partials part) {
  constexpr int DQ = D / 4;
  __shared__ float sQ[kCols][D + 4];       // Q of the 16 columns; later the combined output
  __shared__ float sP[4][16][kCols + 1];   // per wave: P[key][column]
  __shared__ float sM[4][kCols], sL[4][kCols], sTot[kCols], sMax[kCols];

  if ((int32_t)blockIdx.x >= __builtin_amdgcn_readfirstlane(a.totals[0])) return;
  const SmallItem it = items[blockIdx.x];
  const int hkv = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int32_t b = a.qsl[it.r], t = a.qsl[it.r + 1] - b, L = a.seq_lens[it.r], c = L - t;
  const int32_t Tn = min(a.tile_tokens, t - it.tok0);
  const int32_t h0 = it.hsub * a.tile_heads;
  const int32_t HGn = min(a.tile_heads, a.g - h0);
  const T* q = (const T*)a.q;
  T* out = (T*)a.out;

  for (int e = threadIdx.x; e < kCols * D; e += 256) {
    const int col = e / D, d = e - col * D;
    const int i = col / a.tile_heads, j = col - i * a.tile_heads;
    float x = 0.f;
    if (i < Tn && j < HGn)
      x = Elem<T>::load(q + ((int64_t)(b + it.tok0 + i) * a.H + hkv * a.g + h0 + j) * D + d);
    sQ[col][d] = x;
  }
  __syncthreads();

  if (L <= 0) {   // padding request: its rows are zero
    for (int e = threadIdx.x; e < kCols * D; e += 256) {
      const int col = e / D, d = e - col * D;
      const int i = col / a.tile_heads, j = col - i * a.tile_heads;
      if (i < Tn && j < HGn)
        Elem<T>::store(out + ((int64_t)(b + it.tok0 + i) * a.H + hkv * a.g + h0 + j) * D + d, 0.f);
    }
    return;
  }

  const int ni = n / a.tile_heads, nj = n - ni * a.tile_heads;
  const bool col_ok = ni < Tn && nj < HGn;
  const int32_t pos = c + it.tok0 + ni;                      // this column's position
  const int32_t lo = a.window > 0 ? pos - a.window : -1;      // keys <= lo are outside the window
  const int32_t kb = small_key_base(a.window, c + it.tok0) + it.split * a.split_keys;
  const int32_t ke = min(c + it.tok0 + Tn, kb + a.split_keys);
  const int32_t* table_row = a.block_table + (int64_t)it.r * a.stride;
  const T* kc = (const T*)a.k_cache;
  const T* vc = (const T*)a.v_cache;
  const int64_t row_elems = (int64_t)a.Hkv * D;

  float m = kNegInf, lsum = 0.f;
  float acc[DQ];
#pragma unroll
  for (int dd = 0; dd < DQ; ++dd) acc[dd] = 0.f;

  for (int32_t k0 = kb + 16 * w; k0 < ke; k0 += 64) {
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t key = k0 + 4 * G + i;
      s[i] = kNegInf;
      if (key < ke && col_ok && key <= pos && key > lo) {
        const T* kp = kc + slot_of(table_row, key, a.bs) * row_elems + (int64_t)hkv * D;
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; d += 4) {
          float kv4[4];
          Vec4<T>::load(kp + d, kv4);
          dot += kv4[0] * sQ[n][d] + kv4[1] * sQ[n][d + 1] + kv4[2] * sQ[n][d + 2] + kv4[3] * sQ[n][d + 3];
        }
        s[i] = dot * a.scale_log2e;
      }
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2f(s[i] - m_use);
      psum += p;
      sP[w][4 * G + i][n] = p;
    }
    lsum = lsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int dd = 0; dd < DQ; ++dd) acc[dd] *= alpha;
    const int kmax = min(16, ke - k0);
    for (int j = 0; j < kmax; ++j) {
      const float p = sP[w][j][n];
      const T* vp = vc + slot_of(table_row, k0 + j, a.bs) * row_elems + (int64_t)hkv * D + G * DQ;
      if constexpr (DQ % 4 == 0) {
#pragma unroll
        for (int dd = 0; dd < DQ; dd += 4) {
          float v4[4];
          Vec4<T>::load(vp + dd, v4);
          acc[dd] += p * v4[0];
          acc[dd + 1] += p * v4[1];
          acc[dd + 2] += p * v4[2];
          acc[dd + 3] += p * v4[3];
        }
      } else {
#pragma unroll
        for (int dd = 0; dd < DQ; ++dd) acc[dd] += p * Elem<T>::load(vp + dd);
      }
    }
  }

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (G == 0) {
    sM[w][n] = m;
    sL[w][n] = lsum;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sM[ww][n]);
  const float M_use = M == kNegInf ? 0.f : M;
  const float f_own = exp2f(m - M_use);
  if (w == 0 && G == 0) {
    float tot = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) tot += sL[ww][n] * exp2f(sM[ww][n] - M_use);
    sTot[n] = tot;
    sMax[n] = M;
  }
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int dd = 0; dd < DQ; ++dd) {
        const float prev = ww == 0 ? 0.f : sQ[n][G * DQ + dd];
        sQ[n][G * DQ + dd] = prev + acc[dd] * f_own;
      }
    }
    __syncthreads();
  }

  if (it.nsplit == 1) {
    for (int e = threadIdx.x; e < kCols * D; e += 256) {
      const int col = e / D, d = e - col * D;
      const int i = col / a.tile_heads, j = col - i * a.tile_heads;
      if (i < Tn && j < HGn)
        Elem<T>::store(out + ((int64_t)(b + it.tok0 + i) * a.H + hkv * a.g + h0 + j) * D + d,
                       sQ[col][d] / sTot[col]);
    }
  } else {
    const int64_t pbase = ((int64_t)blockIdx.x * a.Hkv + hkv) * kCols;
    if (threadIdx.x < kCols) {
      part.m[pbase + threadIdx.x] = sMax[threadIdx.x];
      part.l[pbase + threadIdx.x] = sTot[threadIdx.x];
    }
    for (int e = threadIdx.x; e < kCols * D; e += 256) {
      const int col = e / D, d = e - col * D;
      part.acc[(pbase + col) * D + d] = sQ[col][d];
    }
  }
}

// Combine the splits of a small tile: M = max m_s, out = sum 2^(m_s - M) acc_s / sum 2^(m_s - M) l_s.
// One thread per (column, dim) output; a workgroup takes 256 / D columns of one tile and KV
// head (blockIdx.y picks the column group), so even a handful of long decodes spreads over
// many compute units.  The kernel is a chain of dependent loads (item, then partials): the
// item carries the tile's output row and row count, and the splits are read kMergeBatch at a
// time, all loads of a batch in flight together, folded into a running maximum (the sums
// rescaled when it grows).  A small batch's tiles have at most 8 splits: one round trip.
constexpr int kMergeBatch = 8;
template <typename T>
__global__ __launch_bounds__(256) void merge_splits(AttnArgs a, Plan pl, const MergeItem* __restrict__ items,
                                                    Partials part) {
  const int D = a.D;
  const int cols_per_wg = 256 / D;
  const int32_t idx = blockIdx.x / a.Hkv;
  MergeItem it;
  if (pl.inline_items) {       // no planner launch: the item from the batch metadata itself
    const InlineOwner o = inline_owner(pl, a.qsl, a.seq_lens, kListMerge, idx);
    if (__builtin_amdgcn_readfirstlane(o.r) < 0) return;
    it = merge_item(pl, o.r, o.li, o.ns, o.o_small, o.t, o.q0);
    it.row0 = __builtin_amdgcn_readfirstlane(it.row0);
    it.ntok = __builtin_amdgcn_readfirstlane(it.ntok);
    it.hsub = __builtin_amdgcn_readfirstlane(it.hsub);
    it.first = __builtin_amdgcn_readfirstlane(it.first);
    it.nsplit = __builtin_amdgcn_readfirstlane(it.nsplit);
    asm volatile("" ::"s"(it.row0), "s"(it.ntok), "s"(it.hsub), "s"(it.first), "s"(it.nsplit), "s"(a.g),
                 "s"(a.tile_heads), "s"(a.H), "s"(part.m), "s"(part.l), "s"(part.acc), "s"(a.out));
  } else {
    // the item is read together with the count: a workgroup past the count (a graph replayed
    // with fewer items than its grid) reads a stale item inside the list and exits unused
    const int32_t total = __builtin_amdgcn_readfirstlane(a.totals[1]);
    it = items[idx];
    asm volatile("" ::"s"(total), "s"(it.row0), "s"(it.ntok), "s"(it.hsub), "s"(it.first), "s"(it.nsplit),
                 "s"(a.g), "s"(a.tile_heads), "s"(a.H), "s"(part.m), "s"(part.l), "s"(part.acc), "s"(a.out));
    if (idx >= total) return;
  }
  const int hkv = blockIdx.x % a.Hkv;
  const int col = blockIdx.y * cols_per_wg + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (col >= kCols || threadIdx.x >= cols_per_wg * D) return;
  const int32_t h0 = it.hsub * a.tile_heads;
  const int32_t HGn = min(a.tile_heads, a.g - h0);
  const int i = col / a.tile_heads, j = col - i * a.tile_heads;
  if (i >= it.ntok || j >= HGn) return;
  const int64_t base = ((int64_t)it.first * a.Hkv + hkv) * kCols + col;
  const int64_t step = (int64_t)a.Hkv * kCols;                  // next split of the same column
  float M = kNegInf, lt = 0.f, o = 0.f;
  for (int s0 = 0; s0 < it.nsplit; s0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch], av[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const bool in = s0 + k < it.nsplit;
      const int64_t pi = base + (int64_t)(s0 + k) * step;
      mv[k] = in ? part.m[pi] : kNegInf;
      lv[k] = in ? part.l[pi] : 0.f;
      av[k] = in ? part.acc[pi * D + d] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) Mn = fmaxf(Mn, mv[k]);
    if (Mn == kNegInf) continue;                                 // no key seen yet
    const float c = exp2f(M - Mn);                               // 0 while M is -inf
    lt *= c;
    o *= c;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float f = exp2f(mv[k] - Mn);
      lt += f * lv[k];
      o += f * av[k];
    }
    M = Mn;
  }
  T* out = (T*)a.out;
  Elem<T>::store(out + ((int64_t)(it.row0 + i) * a.H + hkv * a.g + h0 + j) * D + d, o / lt);
}

template <typename T>
hipError_t launch_small_valu_t(const Plan& p, const AttnArgs& a, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  const SmallItem* items = (const SmallItem*)(w + p.off_small);
  Partials part{(float*)(w + p.off_pm), (float*)(w + p.off_pl), (float*)(w + p.off_pacc)};
  const dim3 grid((unsigned)p.n_small, (unsigned)p.Hkv);
  switch (p.D) {
#define PA_CASE(DD) \
  case DD: hipLaunchKernelGGL((small_tile_valu<T, DD>), grid, dim3(256), 0, s, a, items, part); break;
    PA_CASE(8) PA_CASE(16) PA_CASE(32) PA_CASE(48) PA_CASE(64) PA_CASE(96) PA_CASE(128) PA_CASE(256)
#undef PA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool valu_head_dim_supported(int32_t D) {
  switch (D) {
    case 8: case 16: case 32: case 48: case 64: case 96: case 128: case 256: return true;
    default: return false;
  }
}

hipError_t launch_small_valu(const Plan& p, const AttnArgs& a, void* ws, int32_t dtype, hipStream_t s) {
  if (p.n_small == 0) return hipSuccess;
  return dtype == 0 ? launch_small_valu_t<float>(p, a, ws, s) : launch_small_valu_t<uint16_t>(p, a, ws, s);
}

hipError_t launch_merge(const Plan& p, const AttnArgs& a, void* ws, int32_t dtype, hipStream_t s) {
  if (p.n_merge == 0) return hipSuccess;
  char* w = (char*)ws;
  const MergeItem* items = (const MergeItem*)(w + p.off_merge);
  Partials part{(float*)(w + p.off_pm), (float*)(w + p.off_pl), (float*)(w + p.off_pacc)};
  const int cols_per_wg = 256 / p.D;
  const dim3 grid((unsigned)(p.n_merge * p.Hkv), (unsigned)((kCols + cols_per_wg - 1) / cols_per_wg));
  if (dtype == 0) hipLaunchKernelGGL(merge_splits<float>, grid, dim3(256), 0, s, a, p, items, part);
  else hipLaunchKernelGGL(merge_splits<uint16_t>, grid, dim3(256), 0, s, a, p, items, part);
  return hipGetLastError();
}

}  // namespace pa
