// Small-tile paged attention on bf16 matrix cores: the decode path (and any request whose
// rows times grouped heads fit 16 query columns: decodes, speculative-verification rows).
//
// Same contract and work items as the vector kernel (attn_valu.hip): one workgroup of four
// waves takes up to 16 query columns (token, head) of one request and one KV head over one
// split of the keys; the split-K partials are combined by the shared merge kernel.  Decode
// reads the whole history once per step, so this kernel is built to stream K/V: every
// key's row of one KV head is read exactly once per tile, with the query heads of the
// group as the 16 columns (grouped-query attention folds heads instead of repeating K, as
// in the vllm-lite README's note), and the blocks of a table are read in place (slot-major
// pool: a 16-token block of one KV head is 16 rows of D contiguous elements).
//
// Per wave and 16-key block (one pool block at block_size 16):
//   S^T[key][col] = K[key][:] . Q[col][:]   mfma_f32_16x16x32_bf16, K as the A operand
//                                           (lane: key = lane%16, 8 dims), Q^T held in
//                                           registers as the B operand.
//   online softmax per column               the lane owning column n keeps its running max;
//                                           the 4 lane groups share it with two xor shuffles.
//   O^T[d][col] += V^T[d][key] P^T[key][col] mfma_f32_16x16x16 bf16: P^T is the S^T
//                                           accumulator layout itself; V^T is read from a
//                                           padded LDS copy of the block with the gfx950
//                                           LDS transpose read (ds_read_tr16_b64).
// P is split into bf16 high and low parts (two products) so the probabilities keep ~16
// bits: cheap here, since the path is bound by HBM, not by the matrix cores.
// bf16 pools: K and V go from HBM straight into two per-wave LDS buffers (gfx950 direct
// loads of whole rows), are read into registers as soon as they land, and the next block's
// loads are in flight while the current one is computed.  fp8 pools: the codes of K and V
// go into two register sets (ping-pong) and V is converted into the LDS buffer.  The block
// table is read with scalar loads (one entry per block), so no wait on a table entry drains
// the vector loads in flight.  Keys past the split end are read from the last visible key
// instead (finite data, masked), so no NaN from an unwritten slot enters.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kBlk = 16;                      // keys per block (block_size)

// head_dim 48 runs padded to 64: its rows take 128 bytes in LDS (the two padding chunks of a
// row hold copies of real chunks and are never used), the QK^T contraction runs over 64 dims
// with Q and K zero in dims 48..63 (set in registers), and the PV product takes 3 d tiles.
template <int D>
struct DecodeCfg {
  static constexpr int DP = D == 48 ? 64 : D; // contraction width and LDS row length
  static constexpr int KC = DP / 32;          // k-chunks of the QK^T product
  static constexpr int DT = D / 16;           // 16-wide d tiles of the PV product
  static constexpr int ROW = DP * 2;          // bytes of one key row in LDS
  static constexpr int CHUNKS = ROW / 16;     // 16-byte chunks per LDS row
  static constexpr int GCHUNKS = D / 8;       // 16-byte chunks per row in the pool
  static constexpr int RPI = 1024 / ROW;      // rows one direct-load instruction fills
  static constexpr int VLOADS = kBlk / RPI;   // direct-load instructions per wave per block
  static constexpr int VBUF = kBlk * ROW;     // bytes of one wave's V buffer
};

// Chunk swizzle of a V row in LDS (chunk c of row r sits at slot c ^ vswz(r)): makes the
// transpose reads of a 16-key block (rows 0..7 x two adjacent chunks per half-wave) hit
// 16 distinct 16-byte slots of the 256-byte bank window.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

// Chunk swizzle of a K row in LDS (chunk c of row r at slot c ^ kswz(r)): the A-operand
// reads (16 rows x one chunk per lane group) hit 16 distinct 16-byte slots of the 256-byte
// bank window.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

__device__ __forceinline__ bf16x4 tr_read(const unsigned char* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) void*)p));
  return __builtin_bit_cast(bf16x4, r);
}

// (nontemporal: the rows are streamed rather than kept in the caches; the cache-policy
// operand 2 is the instruction's nt bit.  Measured against cached loads: 256 decodes 5.72 ->
// 6.23 TB/s, speculative verification 4.72 -> 5.20, the long-context decodes 5.63 -> 6.22,
// even the shared-prefix decodes, which re-read the prefix blocks, 4.43 -> 5.16.)
__device__ __forceinline__ void load_lds16(const void* g, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 2);
}

// v of lane i of the lane's quad, for i = 0..3 (DPP quad permutes)
__device__ __forceinline__ void quad_bcast4(float v, float* r) {
  const int x = __builtin_bit_cast(int, v);
  r[0] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x00, 0xf, 0xf, false));
  r[1] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x55, 0xf, 0xf, false));
  r[2] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xaa, 0xf, 0xf, false));
  r[3] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xff, 0xf, 0xf, false));
}

// F8: the pools hold fp8 E4M3 codes with a float32 scale per (slot, KV head) (a.k_scale,
// a.v_scale).  K codes convert exactly to bf16 for the QK^T product and each score is then
// multiplied by its key's scale; V codes convert exactly to bf16 into the wave's LDS buffer,
// and each probability is multiplied by its key's V scale before the PV product (the row sum
// takes the probabilities alone), so sum_j p_j (s_j v8_j) = sum_j (p_j s_j) v8_j.
//
// NC > 1: the workgroup takes up to NC consecutive 16-column tiles of one request (a request
// with more than 16 query columns per KV head: speculative-verification rows, short chunks)
// over one key split, and every K/V block it reads serves all of them: each tile keeps its
// own Q^T, running max, sum and O^T, and the V^T transpose reads are shared.  Tiles of one
// item share the split's key range, which holds without a sliding window.
template <int D, bool F8, int NC>
__global__ __launch_bounds__(256, NC == 1 ? 3 : 2) void small_tile_mfma(AttnArgs a, Plan pl,
                                                                       const SmallItem* __restrict__ items,
                                                                       int32_t total_idx, Partials part) {
  using C = DecodeCfg<D>;
  // per wave two block buffers (bf16: V and K; fp8: two V); after the key loop the same
  // bytes hold the per-wave output slabs
  constexpr int kVBytes = 4 * 2 * C::VBUF;
  constexpr int kSlabBytes = 4 * kCols * D * 4;
  __shared__ __align__(1024) unsigned char smem[kVBytes > kSlabBytes ? kVBytes : kSlabBytes];
  __shared__ float sM[4][kCols], sL[4][kCols], sTot[kCols], sMax[kCols];

  const int32_t item = blockIdx.x;
  const int hkv = blockIdx.y;
  SmallItem it;
  int32_t b, t, L;             // the request's first row, rows and seq_len
  if (pl.inline_items) {       // no planner launch: the item from the batch metadata itself
    const InlineOwner o = inline_owner(pl, a.qsl, a.seq_lens, NC == 1 ? kListSingle : kListGroup, item);
    if (__builtin_amdgcn_readfirstlane(o.r) < 0) return;
    it = NC == 1 ? single_item(pl, o.r, o.li, o.ns, o.o_small) : group_item(pl, o.r, o.li, o.ns, o.o_small, o.t);
    b = __builtin_amdgcn_readfirstlane(o.q0);
    t = __builtin_amdgcn_readfirstlane(o.t);
    L = __builtin_amdgcn_readfirstlane(o.L);
  } else {
    if (item >= __builtin_amdgcn_readfirstlane(a.totals[total_idx])) return;
    it = items[item];
    const int32_t r = __builtin_amdgcn_readfirstlane(it.r);
    b = __builtin_amdgcn_readfirstlane(a.qsl[r]);
    t = __builtin_amdgcn_readfirstlane(a.qsl[r + 1]) - b;
    L = __builtin_amdgcn_readfirstlane(a.seq_lens[r]);
  }
  // the item is the same for the whole workgroup: scalar registers, scalar loop bounds
  it.r = __builtin_amdgcn_readfirstlane(it.r);
  it.split = __builtin_amdgcn_readfirstlane(it.split);
  it.nsplit = __builtin_amdgcn_readfirstlane(it.nsplit);
  it.first = __builtin_amdgcn_readfirstlane(it.first);
  const int32_t tile0 = __builtin_amdgcn_readfirstlane(it.tile0);
  const int32_t ntile = NC == 1 ? 1 : __builtin_amdgcn_readfirstlane(it.ntile);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave id: uniform
  const int n = lane & 15, G = lane >> 4;
  const int32_t c = L - t;
  const __bf16* q = (const __bf16*)a.q;
  __bf16* out = (__bf16*)a.out;
  // tile u of the item: its first token, head subset, token and head counts
  const int hsubs = (a.g + a.tile_heads - 1) / a.tile_heads;
  int32_t tok0[NC], h0[NC], Tn[NC], HGn[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int32_t tl = tile0 + u;
    tok0[u] = (tl / hsubs) * a.tile_tokens;
    h0[u] = (tl % hsubs) * a.tile_heads;
    Tn[u] = u < ntile ? min(a.tile_tokens, t - tok0[u]) : 0;
    HGn[u] = min(a.tile_heads, a.g - h0[u]);
  }

  if (L <= 0) {   // padding request: zero rows
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      for (int e = threadIdx.x; e < kCols * D; e += 256) {
        const int col = e / D, d = e - col * D;
        const int i = col / a.tile_heads, j = col - i * a.tile_heads;
        if (i < Tn[u] && j < HGn[u]) out[((int64_t)(b + tok0[u] + i) * a.H + hkv * a.g + h0[u] + j) * D + d] = (__bf16)0.f;
      }
    }
    return;
  }

  const int ni = n / a.tile_heads, nj = n - ni * a.tile_heads;
  bool col_ok[NC];
  int32_t pos[NC], ke_u[NC];
  const int32_t kb = small_key_base(a.window, c + tok0[0]) + it.split * a.split_keys;   // multiple of 64
  int32_t ke = 0;                                               // one past the last key of any tile
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    col_ok[u] = ni < Tn[u] && nj < HGn[u];
    pos[u] = c + tok0[u] + ni;
    ke_u[u] = u < ntile ? min(c + tok0[u] + Tn[u], kb + a.split_keys) : 0;
    ke = max(ke, ke_u[u]);
  }
  const int32_t lo = a.window > 0 ? pos[0] - a.window : -1;     // keys <= lo are outside the window (NC == 1)
  const int32_t* table_row = a.block_table + (int64_t)it.r * a.stride;
  const int64_t row_elems = (int64_t)a.Hkv * D;
  const __bf16* kc = (const __bf16*)a.k_cache + (int64_t)hkv * D;
  const __bf16* vc = (const __bf16*)a.v_cache + (int64_t)hkv * D;
  const uint8_t* kc8 = (const uint8_t*)a.k_cache + (int64_t)hkv * D;   // F8: bytes
  const uint8_t* vc8 = (const uint8_t*)a.v_cache + (int64_t)hkv * D;

  // Q^T as the B operand: column n, dims 32*kk + 8*G .. +7; a negative scale becomes -q
  const float sl = fmaxf(fabsf(a.scale_log2e), 1e-30f);
  const uint32_t qsign = a.scale_log2e < 0.f ? 0x80008000u : 0u;
  // dims of k-chunk kk in lane group G (Q and K take the same permutation of the contraction
  // dim): fp8 lanes hold D/4 contiguous dims, so a lane's K codes are one contiguous run
  auto kdim = [](int kk, int g4) { return F8 ? (D / 4) * g4 + 8 * kk : 32 * kk + 8 * g4; };
  bf16x8 qf[NC][C::KC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const __bf16* qrow = q + ((int64_t)(b + tok0[u] + ni) * a.H + hkv * a.g + h0[u] + nj) * D;
#pragma unroll
    for (int kk = 0; kk < C::KC; ++kk) {
      u32x4 v = col_ok[u] && kdim(kk, G) < D ? *(const u32x4*)(qrow + kdim(kk, G)) : u32x4{0u, 0u, 0u, 0u};
      v ^= qsign;
      qf[u][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  unsigned char* vbuf0 = smem + w * 2 * C::VBUF;
  f32x4 o[NC][C::DT];
  float m[NC], lsum[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[u] = kNegInf;
    lsum[u] = 0.f;
  }

  const int32_t nblk_end = (ke + kBlk - 1) / kBlk;               // one past the last block
  const int32_t blk0 = kb / kBlk + w;
  // A block's keys share one table entry: one scalar load per block, read through the
  // constant address space so that it waits behind no vector load in flight.
  const __attribute__((address_space(4))) int32_t* trow =
      (const __attribute__((address_space(4))) int32_t*)table_row;
  // slot of key j of block lb; keys past the split end read key ke-1 instead (finite data,
  // masked), which lies in the same block since lb*16 <= ke-1 for every block in the loop
  auto slot = [&](int32_t tb, int32_t lb, int j) -> int64_t {
    return (int64_t)tb * kBlk + (min(lb * kBlk + j, ke - 1) & (kBlk - 1));
  };

  // F8: one block of codes in registers.  K: key n, the lane's D/4 contiguous dims (kdim).
  // V: row lane/4, quarter lane%4 of the row.  Scales: K and V scale of key 4G + n%4 (the
  // lane's quad broadcasts them to the four keys of its S^T rows).  Every load is an
  // ordinary vector load, so the compiler waits for exactly the block it is about to use.
  // (Unlike the bf16 rows, these stay cached loads: nontemporal ones measured slower here,
  // 6% on 256 decodes and 27% on speculative verification, whose tiles re-read each block.)
  constexpr int VX = D / 64;                                   // 16-byte pieces of V codes per lane
  constexpr int KX = D / 64;                                   // 16-byte pieces of K codes per lane
  struct Blk { u32x4 k[KX]; u32x4 v[VX]; float ks, vs; };
  auto load_f8 = [&](int32_t lb, Blk& f) {
    const int32_t tb = trow[lb];
    const uint8_t* kp = kc8 + slot(tb, lb, n) * row_elems + (D / 4) * G;
#pragma unroll
    for (int x = 0; x < KX; ++x) f.k[x] = *(const u32x4*)(kp + 16 * x);
    const uint8_t* vp = vc8 + slot(tb, lb, lane >> 2) * row_elems + (D / 4) * (lane & 3);
#pragma unroll
    for (int x = 0; x < VX; ++x) f.v[x] = *(const u32x4*)(vp + 16 * x);
    const int64_t si = slot(tb, lb, 4 * G + (n & 3)) * a.Hkv + hkv;
    f.ks = a.k_scale[si];
    f.vs = a.v_scale[si];
  };
  // V codes of one block as bf16 rows in the wave's LDS buffer (16-byte chunk c of row r at
  // slot c ^ vswz(r), as the direct loads of the bf16 path place them)
  auto stage_v = [&](const Blk& f, unsigned char* dst) {
    const int r = lane >> 2;
#pragma unroll
    for (int x = 0; x < VX; ++x) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int chunk = (D / 32) * (lane & 3) + 2 * x + hf;
        const u32x2 a0 = fp8x4_to_bf16x4(f.v[x][2 * hf]), a1 = fp8x4_to_bf16x4(f.v[x][2 * hf + 1]);
        *(u32x4*)(dst + r * C::ROW + 16 * (chunk ^ vswz<D>(r))) = u32x4{a0[0], a0[1], a1[0], a1[1]};
      }
    }
  };

  // V^T operand of d tile dt (keys 4G + n/4 .. as the S^T accumulator holds them) from a
  // wave's V buffer
  auto vt_read = [&](const unsigned char* vb, int dt) -> bf16x4 {
    const int r = 4 * G + (n >> 2);
    const int chunk = 2 * dt + ((n & 3) >> 1);
    return tr_read(vb + r * C::ROW + 16 * (chunk ^ vswz<D>(r)) + 8 * (n & 1));
  };
  auto compute = [&](int32_t lb, const bf16x8* kcur, auto&& vfrag, const float* ks, const float* vs) {
    const int32_t key0 = lb * kBlk + 4 * G;
    float alpha[NC];
    bf16x4 phi[NC], plo[NC];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      if (u >= ntile) break;
      // S^T = K Q^T
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::KC; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kcur[kk], qf[u][kk], s, 0, 0, 0);
      if constexpr (F8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] *= ks[i];
      }
      // masked scores, running max (base 2)
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sv[i] = (col_ok[u] && key0 + i < ke_u[u] && key0 + i <= pos[u] && key0 + i > lo) ? s[i] : kNegInf;
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m[u], mx * sl);
      alpha[u] = m_new > m[u] ? __builtin_amdgcn_exp2f(m[u] - m_new) : 1.f;   // m may be -inf
      m[u] = m_new;
      const float m_use = m[u] == kNegInf ? 0.f : m[u];
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], sl, -m_use));
      lsum[u] = lsum[u] * alpha[u] + (p[0] + p[1]) + (p[2] + p[3]);
      if constexpr (F8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] *= vs[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        phi[u][i] = (__bf16)p[i];
        plo[u][i] = (__bf16)(p[i] - (float)phi[u][i]);
      }
    }
    // O^T = alpha * O^T + V^T P^T (one transpose read per d tile serves every tile)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const bf16x4 vt = vfrag(dt);
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        if (u >= ntile) break;
        o[u][dt] *= alpha[u];
        o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, phi[u], o[u][dt], 0, 0, 0);
        o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, plo[u], o[u][dt], 0, 0, 0);
      }
    }
  };

  if constexpr (F8) {
    auto run = [&](int32_t lb, const Blk& f, unsigned char* vb) {
      stage_v(f, vb);
      bf16x8 kr[C::KC];
#pragma unroll
      for (int kk = 0; kk < C::KC; ++kk) {
        const u32x4 w4 = f.k[kk / 2];
        const u32x2 a0 = fp8x4_to_bf16x4(w4[2 * (kk & 1)]), a1 = fp8x4_to_bf16x4(w4[2 * (kk & 1) + 1]);
        kr[kk] = __builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]});
      }
      float ks[4], vs[4];
      quad_bcast4(f.ks, ks);
      quad_bcast4(f.vs, vs);
      compute(lb, kr, [&](int dt) { return vt_read(vb, dt); }, ks, vs);
    };
    // this wave's blocks blk0, blk0 + 4, ... through two register sets: the loads of the next
    // block are issued before each block is computed (a third set measured slower).  They are
    // unconditional (past the wave's last block they re-read it, from cache), so that every
    // path through the loop has the same loads in flight and the compiler's waits stay partial.
    constexpr int NSET = 2;
    if (blk0 < nblk_end) {
      const int32_t last = blk0 + 4 * ((nblk_end - 1 - blk0) / 4);   // this wave's last block
      Blk f[NSET];
#pragma unroll
      for (int s = 0; s < NSET - 1; ++s) load_f8(min(blk0 + 4 * s, last), f[s]);
      bool more = true;
      for (int32_t lb = blk0; more; lb += 4 * NSET) {
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
          const int32_t cur = lb + 4 * s;
          load_f8(min(cur + 4 * (NSET - 1), last), f[(s + NSET - 1) % NSET]);
          run(cur, f[s], vbuf0 + (s & 1) * C::VBUF);
          if (cur >= last) {
            more = false;
            break;
          }
        }
      }
    }
  } else {
    // K and V of a block go straight into this wave's two LDS buffers (gfx950 direct loads),
    // every load instruction covering whole rows (RPI rows of D contiguous elements): a K
    // read in the A-operand layout straight from HBM covers 16 rows x 64 bytes per
    // instruction, which streams measurably slower than whole rows.  Each block is read
    // out of LDS into registers (K operand, V^T operand) as soon as it has landed, and the
    // next block's loads go out into the same buffers before the block is computed.
    unsigned char* kbufw = vbuf0 + C::VBUF;
    auto issue = [&](int32_t lb) {
      const int32_t tb = trow[lb];
#pragma unroll
      for (int u = 0; u < C::VLOADS; ++u) {
        const int r = C::RPI * u + lane / C::CHUNKS;
        const int64_t src = slot(tb, lb, r) * row_elems;
        // the chunk each lane's LDS slot holds; a padding slot (head_dim 48) gets a real chunk
        // of the same row, so every read stays inside the row
        int ck = (lane % C::CHUNKS) ^ kswz<D>(r), cv = (lane % C::CHUNKS) ^ vswz<D>(r);
        if constexpr (C::GCHUNKS < C::CHUNKS) {
          ck = ck < C::GCHUNKS ? ck : ck - (C::CHUNKS - C::GCHUNKS);
          cv = cv < C::GCHUNKS ? cv : cv - (C::CHUNKS - C::GCHUNKS);
        }
        load_lds16(kc + src + 8 * ck, kbufw + u * 1024);
        load_lds16(vc + src + 8 * cv, vbuf0 + u * 1024);
      }
    };
    const float ones[4] = {1.f, 1.f, 1.f, 1.f};
    if (blk0 < nblk_end) issue(blk0);
    for (int32_t lb = blk0; lb < nblk_end; lb += 4) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");            // block lb landed
      bf16x8 kr[C::KC];
      bf16x4 vt[C::DT];
#pragma unroll
      for (int kk = 0; kk < C::KC; ++kk) {
        kr[kk] = *(const bf16x8*)(kbufw + n * C::ROW + 16 * ((4 * kk + G) ^ kswz<D>(n)));
        if (4 * kk + G >= C::GCHUNKS) kr[kk] = bf16x8{};             // head_dim 48: padding dims
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) vt[dt] = vt_read(vbuf0, dt);
      // the reads are done before the buffers are reloaded
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lb + 4 < nblk_end) issue(lb + 4);
      compute(lb, kr, [&](int dt) { return vt[dt]; }, ones, ones);
    }
  }

  // combine the four waves, one tile after another: per column max, sum and output
  float* slab = (float*)smem;                 // [4][16 cols][D]
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    if (u >= ntile) break;
    float ls = lsum[u];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if (G == 0) {
      sM[w][n] = m[u];
      sL[w][n] = ls;
    }
    __syncthreads();   // also: every wave is done with its V buffers (tile 0) or with the
                       // previous tile's slab (later tiles)
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sM[ww][n]);
    const float M_use = M == kNegInf ? 0.f : M;
    const float f_own = __builtin_amdgcn_exp2f(m[u] - M_use);
    if (w == 0 && G == 0) {
      float tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) tot += sL[ww][n] * __builtin_amdgcn_exp2f(sM[ww][n] - M_use);
      sTot[n] = tot;
      sMax[n] = M;
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) slab[(w * kCols + n) * D + 16 * dt + 4 * G + i] = o[u][dt][i] * f_own;
    }
    __syncthreads();

    // each thread finishes 8 consecutive dims of one column; split-K partials go to the
    // tile's own slot (tile-split index first + u * nsplit + split), which the merge reads
    const int64_t ts = (int64_t)it.first + (int64_t)u * it.nsplit + it.split;
    constexpr int kPer = 8;
    for (int e = threadIdx.x * kPer; e < kCols * D; e += 256 * kPer) {
      const int col = e / D, d = e - col * D;
      const int i = col / a.tile_heads, j = col - i * a.tile_heads;
      if (i >= Tn[u] || j >= HGn[u]) continue;
      float acc[kPer];
#pragma unroll
      for (int x = 0; x < kPer; ++x)
        acc[x] = slab[(0 * kCols + col) * D + d + x] + slab[(1 * kCols + col) * D + d + x] +
                 slab[(2 * kCols + col) * D + d + x] + slab[(3 * kCols + col) * D + d + x];
      if (it.nsplit == 1) {
        const float inv = 1.f / sTot[col];
        bf16x8 r;
#pragma unroll
        for (int x = 0; x < kPer; ++x) r[x] = (__bf16)(acc[x] * inv);
        *(bf16x8*)(out + ((int64_t)(b + tok0[u] + i) * a.H + hkv * a.g + h0[u] + j) * D + d) = r;
      } else {
        const int64_t pi = (ts * a.Hkv + hkv) * kCols + col;
        float4* dst = (float4*)(part.acc + pi * D + d);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if (d == 0) {
          part.m[pi] = sMax[col];
          part.l[pi] = sTot[col];
        }
      }
    }
    if (u + 1 < ntile) __syncthreads();   // the next tile reuses sM, sTot and the slab
  }
}

template <int NC, bool F8>
hipError_t launch_small_nc(const Plan& p, const AttnArgs& a, const SmallItem* items, int64_t n_items, int32_t total_idx,
                           Partials part, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid((unsigned)n_items, (unsigned)p.Hkv);
  if (p.D == 128) hipLaunchKernelGGL((small_tile_mfma<128, F8, NC>), grid, dim3(256), 0, s, a, p, items, total_idx, part);
  else if (p.D == 64) hipLaunchKernelGGL((small_tile_mfma<64, F8, NC>), grid, dim3(256), 0, s, a, p, items, total_idx, part);
  else if (p.D != 48) return hipErrorInvalidValue;
  else if constexpr (F8) return hipErrorInvalidValue;     // fp8 codes: head_dim 64 or 128 only
  else hipLaunchKernelGGL((small_tile_mfma<48, false, NC>), grid, dim3(256), 0, s, a, p, items, total_idx, part);
  return hipGetLastError();
}

}  // namespace

bool small_mfma_supported(int32_t D, int32_t bs, bool fp8) {
  return bs == kBlk && (D == 64 || D == 128 || (D == 48 && !fp8));
}

hipError_t launch_small_mfma(const Plan& p, const AttnArgs& a, void* ws, hipStream_t s) {
  if (p.n_small == 0) return hipSuccess;
  char* w = (char*)ws;
  Partials part{(float*)(w + p.off_pm), (float*)(w + p.off_pl), (float*)(w + p.off_pacc)};
  // single tiles (decodes), then the groups of tiles of wider requests
  const SmallItem* single = (const SmallItem*)(w + p.off_g1);
  const SmallItem* grouped = (const SmallItem*)(w + p.off_g3);
  if (a.k_scale != nullptr) {   // fp8 pools: single tiles only
    if (p.n_g3 != 0) return hipErrorInvalidValue;
    return launch_small_nc<1, true>(p, a, single, p.n_g1, kTotalG1, part, s);
  }
  if (group_tiles(p) != kGroupTiles) return hipErrorInvalidValue;
  hipError_t e = launch_small_nc<1, false>(p, a, single, p.n_g1, kTotalG1, part, s);
  if (e != hipSuccess) return e;
  return launch_small_nc<kGroupTiles, false>(p, a, grouped, p.n_g3, kTotalG3, part, s);
}

}  // namespace pa
