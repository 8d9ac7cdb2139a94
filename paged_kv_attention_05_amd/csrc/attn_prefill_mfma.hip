// Prefill-chunk paged attention on the matrix cores.
//
// A request whose rows times grouped heads exceed 16 query columns (a prefill chunk) is cut
// into tiles of 32 * WAVES query rows: (32 * WAVES) / g consecutive tokens times the g query
// heads of one KV head.  Packing the group's heads into one tile means every K/V tile brought
// on chip serves all g heads (grouped-query attention without repeating K/V, as the
// vllm-lite README's fold does for its CPU path).  The causal mask is offset by the request's
// computed tokens: row i of a request with seq_len L and t rows sits at position L - t + i
// ("Attention over the pool" in "Engine v2: one core for every request").  Keys come 64
// (four 16-token blocks) at a time; the online softmax keeps exact attention without a score
// matrix in memory (the FlashAttention section of the tensorsofthewall.com post).
//
// Data movement: each 64-key K and V tile goes from HBM straight into LDS with the gfx950
// direct loads (global_load_lds_dwordx4, 16 bytes per lane, no register staging), into rings
// of three tiles, so later tiles stream in while the current one is computed.  A load's
// block address (base + block number x block bytes) is formed on the scalar unit.
//   - bf16 pools: K is read in place, through the wave's two block-table entries per tile;
//     V from the fp16 copy of the request's blocks that stage_v16 (v16_stage.hip) made just
//     before, at staged block numbers.
//   - fp8 pools: stage_fp8 (fp8_stage.hip) made bf16 copies of the K (and V) codes, their
//     scales, and an fp16 copy of V dequantized; all are read at staged block numbers.
// An LDS row of K is one key's 256 bytes; its sixteen 16-byte chunks are stored XOR-swizzled
// (chunk c of row r at slot c ^ f(r), f(r) = 4*(r%4) + (r/4)%4), which makes the K reads (16
// consecutive rows, one chunk) and the bf16 kernels' V transpose reads (4 rows x 4 chunks)
// free of bank conflicts.
//
// Compute: wave w owns tile rows 32w .. 32w+31, one row per lane column.
//   S^T[key][row] = K[key][:] . Q[row][:]     mfma_f32_32x32x16_bf16, K from LDS (A operand,
//                                             one 16-byte read per lane), Q^T in registers.
//   O^T[d][row]  += V^T[d][key] P^T[key][row]  mfma_f32_32x32x16_f16 (the fp16 kernels); P^T
//                                             is the S^T accumulator layout with the key
//                                             index bit-permuted (bits 2 and 3 swapped in
//                                             each 16-key chunk), and the staged fp16 copy
//                                             holds V^T in that order, so a lane's operand is
//                                             one 16-byte read.  The bf16 kernels read V^T
//                                             from key rows with two ds_read_tr16_b64.
// Two groups of four waves run in ping-pong (one wave of each per SIMD), so one wave's
// exponentials overlap the other's matrix products (see the loop below).
// Softmax per row in base 2: one FMA and one v_exp_f32 per score; the running max is only
// moved (and O rescaled) when a row's max grows by more than 8 (a factor 256), so rescaling
// is rare; the sum uses the same reference, so the result is exact either way.
//
// Precision of PV: in the fp16 kernels V is fp16 (bf16 pools: converted, exact for
// 2^-14 <= |v| <= 65504 and off by at most 2^-25 below; fp8 pools: code times scale, off by
// at most 2^-11 relative), and P is rounded to nearest fp16 (p <= 256 here), with the row sum
// taken over the same rounded values.  The output is then a convex combination of V rows
// whose weights are off by at most 2^-12 relative: a single bf16 P (2^-9) would use most of
// the 2e-2 budget against ~10x outlier values.  An item that meets |v| > 65504 is redone by
// the bf16 kernel of its pool kind, which keeps V in bf16 and carries P as a bf16 pair
// (truncated high part plus the bf16 rounding of the remainder, two products per chunk,
// ~16 significant bits).
#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// LDS reads at a byte address
__device__ __forceinline__ bf16x4 tr_read(uint32_t addr) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)addr);
  return __builtin_bit_cast(bf16x4, r);
}
// max of x over lanes l and l ^ 32, with one swap of the wave's halves (a vector-ALU
// instruction: unlike a shuffle through the LDS crossbar, it does not queue behind the other
// waves' LDS reads)
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr;
}

// 16 bytes per lane from global memory straight into LDS at lds_wave_base + 16 * lane.  Issued
// as inline assembly on purpose: the compiler then does not know that the load writes LDS and
// does not wait for it before every later LDS read (it cannot tell the ring slots apart); the
// kernel waits for these loads itself (vmcnt before the barrier that publishes them).
// M0 holds the LDS base of the load.  The compiler treats M0 as reserved and does not accept
// it as a clobber; nothing else in this file uses M0 (no LDS-DMA builtins, no M0-indexed
// moves), so setting it here disturbs no compiler-held value.
__device__ __forceinline__ uint32_t lds_addr(unsigned char* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)p;
}
// per-lane 64-bit address
__device__ __forceinline__ void load_lds16(const void* g, unsigned char* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr(lds_wave_base)), "v"(g)
               : "memory");
}
// wave-uniform base plus a per-lane 32-bit byte offset
__device__ __forceinline__ void load_lds16(const void* base, uint32_t voff, unsigned char* lds_wave_base) {
  const uint64_t b64 = (uint64_t)(uintptr_t)base;
  // (readfirstlane returns int: go through uint32_t so the low word is not sign-extended)
  const uint64_t sbase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32)) << 32) |
                         (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr(lds_wave_base)), "v"(voff),
               "s"(sbase)
               : "memory");
}

// The same load from base + idx * stride (bytes; base as two 32-bit halves, idx and stride
// wave-uniform): the block address is formed by the scalar unit, with no vector round trip.
__device__ __forceinline__ void load_lds16_at(uint32_t base_lo, uint32_t base_hi, uint32_t idx, uint32_t stride,
                                              uint32_t voff, unsigned char* lds_wave_base) {
  // (readfirstlane: the operands are wave-uniform; it makes sure they sit in scalar registers)
  uint32_t lo, hi;
  asm volatile("s_mul_i32 %0, %2, %3\n\ts_mul_hi_u32 %1, %2, %3\n\ts_add_u32 %0, %0, %4\n\ts_addc_u32 %1, %1, %5"
               : "=&s"(lo), "=&s"(hi)
               : "s"(__builtin_amdgcn_readfirstlane(idx)), "s"(__builtin_amdgcn_readfirstlane(stride)),
                 "s"(__builtin_amdgcn_readfirstlane(base_lo)), "s"(__builtin_amdgcn_readfirstlane(base_hi))
               : "scc");
  const uint64_t sbase = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr(lds_wave_base)), "v"(voff),
               "s"(sbase)
               : "memory");
}

// 4 bytes per lane from global memory straight into LDS at lds_wave_base + 4 * lane (the
// same conventions as load_lds16)
__device__ __forceinline__ void load_lds4(const void* g, unsigned char* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_addr(lds_wave_base)), "v"(g) : "memory");
}

// F16 = true: the fast kernels.  V comes already in fp16, from the copy that the staging
// kernel made of the request's blocks (v16_stage.hip for bf16 pools, fp8_stage.hip for fp8
// pools): request r's block j is staged block req[r].stage + j - first, so V needs no table
// lookup.  P goes to the matrix cores as fp16.  An item whose V leaves fp16's range
// (|v| > 65504) was flagged by the staging kernel (wide[lin] = 1); its output is rewritten
// by the F16 = false kernel of the same pool kind, launched right after on the same stream,
// which reads V in bf16 and carries P as a bf16 pair; its other workgroups exit at once.
//
// F8 = true: fp8 pools.  K comes from the staged bf16 copy of the codes (exact), at staged
// block numbers (no table), and each score is multiplied by its key's staged K scale (which
// carries |scale| log2 e), as the gathered rows of "ReferenceBackend.dequantize" are the
// codes times their scales.  The fast kernel's fp16 V already holds codes times scales; the
// bf16 redo kernel reads the staged bf16 V codes and multiplies each probability by its
// key's V scale before the PV product (the row sum takes the probabilities alone).  Scales
// of a tile come into LDS with its V loads (wave 0 the K scales, wave 1 the V scales).
template <int D, int WAVES, bool F16, bool F8>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void prefill_tile_mfma(AttnArgs a, const PfItem* __restrict__ items,
                                                                            int32_t n_items, int32_t* __restrict__ wide) {
  using C = PrefillCfg<D>;
  constexpr int ROWS = 32 * WAVES;
  constexpr int NT = 64 * WAVES;
  // Rings of three tiles each: V (fp16 in the fast kernel, bf16 otherwise) and K.  The
  // output staging reuses the first bytes.
  constexpr int NBUF = 3;
  constexpr int V_RING = 0, K_RING = V_RING + NBUF * C::TILE;
  constexpr int SC_RING = K_RING + NBUF * C::TILE;            // F8: per tile 64 K then 64 V scales
  constexpr int SC_TILE = F8 ? 2 * kBK * 4 : 0;
  constexpr int OUT_BYTES = ROWS * C::ROW;
  constexpr int SMEM = (SC_RING + NBUF * SC_TILE) > OUT_BYTES ? (SC_RING + NBUF * SC_TILE) : OUT_BYTES;
  __shared__ __align__(1024) unsigned char smem[SMEM];

  // workgroup -> (item, KV head): consecutive items of one head on one XCD (workgroups are
  // dealt round-robin over the 8 XCDs), so tiles sweeping the same K/V share its L2
  const int32_t total = n_items * a.Hkv;
  const int32_t per_xcd = (total + 7) / 8;
  const int32_t lin = (int32_t)(blockIdx.x % 8) * per_xcd + (int32_t)(blockIdx.x / 8);
  if (lin >= total) return;
  if constexpr (!F16) {
    if (__builtin_amdgcn_readfirstlane(wide[lin]) == 0) return;   // the fast kernel's output stands
  }
  const int hkv = lin / n_items;
  if (lin - hkv * n_items >= __builtin_amdgcn_readfirstlane(a.totals[2])) return;
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
  // With a sliding window the tile's first row sees keys from c + tok0 - window + 1 on: the
  // K/V tiles before the one holding that key are skipped.  Tile i of the loop below is
  // key tile t0 + i.
  const int32_t t0 = a.window > 0 ? max(0, c + tok0 - a.window + 1) / kBK : 0;
  const int32_t ntiles = (kend + kBK - 1) / kBK - t0;
  const int rowoff = (4 * w + (lane >> 4)) & 15;
  const int chunk_sw = (lane & 15) ^ swz(rowoff);
  const uint32_t lane_off_b = (uint32_t)(((int64_t)rowoff * row_elems + 8 * chunk_sw) * 2);   // bytes
  const int64_t blk_stride = (int64_t)kBlk * row_elems;
  // Block ids of a full tile (4 consecutive table entries, wave-uniform) are fetched one
  // iteration before they are needed, so no load waits on a table lookup; only the last,
  // partial tile computes clamped per-lane keys.
  // Staged copies (the fp16 V copy; on fp8 pools also the bf16 codes and the scales): the
  // staged blocks of this request are consecutive, block k/16 of the request at staged block
  // stage0 + k/16 (stage0 = its first staged block minus the first block it holds), and every
  // tile's four blocks are staged (zeros past seq_len), so whole tiles are read.
  const int32_t stage0 = (F16 || F8) ? __builtin_amdgcn_readfirstlane(a.req[r_id].stage) -
                                           v16_first_block(a.window, t, L)
                                     : 0;
  // block holding key 16e of the request: a table entry, or (fp8 pools) a staged block
  auto entry_blk = [&](int32_t e) -> int32_t { return F8 ? stage0 + e : table_row[e]; };
  struct Blocks { int32_t b0, b1, b2, b3; };
  auto fetch_blocks = [&](int32_t j) -> Blocks {
    j += t0;
    if (j * kBK + kBK > kend) return Blocks{0, 0, 0, 0};     // partial tile: not used
    if constexpr (F8) {
      const int32_t e0 = stage0 + 4 * j;
      if constexpr (F16) return Blocks{e0 + (w >> 2), e0 + (w >> 2) + 2, 0, 0};
      return Blocks{e0, e0 + 1, e0 + 2, e0 + 3};
    }
    // through the constant address space, so the compiler reads the (wave-uniform) entries
    // with a scalar load, which does not wait behind the tile loads in flight
    const __attribute__((address_space(4))) int32_t* e =
        (const __attribute__((address_space(4))) int32_t*)(table_row + 4 * j);
    if constexpr (F16) return Blocks{e[w >> 2], e[(w >> 2) + 2], 0, 0};   // this wave's two blocks
    return Blocks{e[0], e[1], e[2], e[3]};
  };
  // block of instruction u within the tile: wave-uniform ((w + WAVES*u) / 4)
  auto pick = [&](const Blocks& bl, int u) -> int32_t {
    if constexpr (F16) return u == 0 ? bl.b0 : bl.b1;
    const int bi = WAVES == 4 ? u : ((w >> 2) + (WAVES / 4) * u);
    return bi == 0 ? bl.b0 : bi == 1 ? bl.b1 : bi == 2 ? bl.b2 : bl.b3;
  };
  const uint32_t blk_bytes = (uint32_t)(blk_stride * 2);
  const uint64_t kc_b = (uint64_t)(uintptr_t)kc;
  const uint32_t kc_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)kc_b);
  const uint32_t kc_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(kc_b >> 32));
  auto issue = [&](const __bf16* base, int32_t j, const Blocks& bl, unsigned char* dst) {
    j += t0;
    if (F16 && j * kBK + kBK <= kend) {
#pragma unroll
      for (int u = 0; u < UK; ++u)
        load_lds16_at(kc_lo, kc_hi, (uint32_t)pick(bl, u), blk_bytes, lane_off_b, dst + (w + WAVES * u) * 1024);
    } else if (j * kBK + kBK <= kend) {
#pragma unroll
      for (int u = 0; u < UK; ++u)
        load_lds16(base + (int64_t)pick(bl, u) * blk_stride, lane_off_b, dst + (w + WAVES * u) * 1024);
    } else {
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        const int32_t kg = min(j * kBK + 4 * (w + WAVES * u) + (lane >> 4), kend - 1);
        const int64_t off = ((int64_t)entry_blk(kg >> 4) * kBlk + (kg & 15)) * row_elems + 8 * chunk_sw;
        load_lds16(base + off, dst + (w + WAVES * u) * 1024);
      }
    }
  };
  auto issue_k = [&](int32_t j, const Blocks& bl, unsigned char* dst) { issue(kc, j, bl, dst); };
  // F16: V from the transposed fp16 copy ([staged block][Hkv][D][16 keys in kperm order]).
  // In LDS a V tile is four 4 KB blocks of 128 dim rows x 32 bytes; the two 16-byte halves
  // of row d are swapped when bit 3 of d is set, which spreads a wave's operand reads (16
  // consecutive dims, one half) over all banks.  Load instruction u of wave w fills the 1 KB
  // piece I = w + WAVES*u: block I/4, dims 32(I%4) .. +31; lane l takes dim 32(I%4) + l/2,
  // half (l%2) ^ (bit 3 of the dim).
  static_assert(WAVES % 4 == 0, "a wave's V pieces share one dim range");
  const uint16_t* v16 = F16 ? (const uint16_t*)a.v_staged + (int64_t)stage0 * blk_stride + (int64_t)hkv * D * kBlk : nullptr;
  const uint64_t v16_b = (uint64_t)(uintptr_t)v16;
  const uint32_t v16_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v16_b);
  const uint32_t v16_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v16_b >> 32));
  const int vdim = 32 * (w & 3) + (lane >> 1);
  const uint32_t v16_lane_off_b = (uint32_t)(vdim * 32 + 16 * ((lane & 1) ^ ((vdim >> 3) & 1)));
  auto issue_v = [&](int32_t j, const Blocks& bl, unsigned char* dst) {
    if constexpr (F16) {
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        const int bi = (w + WAVES * u) >> 2;
        load_lds16_at(v16_lo, v16_hi, (uint32_t)(4 * (j + t0) + bi), blk_bytes, v16_lane_off_b,
                      dst + (w + WAVES * u) * 1024);
      }
    } else {
      issue(vc, j, bl, dst);
    }
  };
  // F8: the 64 K scales (wave 0) and, for the bf16 kernel, V scales (wave 1) of tile j, one
  // per lane, into the ring slot at dst (K scales at +0, V scales at +256); staged layout
  // [staged block][2][Hkv][16]
  auto issue_sc = [&](int32_t j, const Blocks&, unsigned char* dst) {
    if constexpr (F8) {
      if (w >= (F16 ? 1 : 2)) return;
      j += t0;
      const int32_t kg = min(j * kBK + lane, kend - 1);        // (the last tile: clamped keys)
      const int32_t blk = stage0 + (kg >> 4);
      load_lds4(a.k_scale + (((int64_t)blk * 2 + w) * a.Hkv + hkv) * 16 + (kg & 15), dst + 256 * w);
    }
  };

  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x16{};
  float m = kNegInf, lsum = 0.f;
  float lsum2 = 0.f;                                          // a second row-sum accumulator
  const int G = lane >> 4, i16 = lane & 15;

  // Per-lane LDS read addresses at ring slot 0, passed through an empty asm so the compiler
  // keeps them as they are and adds the slot and chunk offsets as read-instruction immediates
  // (no extra address registers per ring slot).
  //   K (A operand of QK^T): key row 32*sh + n, chunk (2kk + h) ^ swz(n)   (swz(32+n) == swz(n))
  //   V (transpose reads):   key rows 16qc + 4h + i16/4 (+8), whose swizzle does not depend on qc
  //   V^T, F16 (transposed copy): dim 32dt + n, half h ^ (bit 3 of n), one 16-byte read
  uint32_t koff[C::KC], voff[C::DT][2], voff16[C::DT];
  {
    const uint32_t kring = lds_addr(smem + K_RING), vring = lds_addr(smem + V_RING);
#pragma unroll
    for (int kk = 0; kk < C::KC; ++kk) {
      koff[kk] = kring + n * C::ROW + 16 * ((2 * kk + h) ^ swz(n));
      asm volatile("" : "+v"(koff[kk]));
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int r = 4 * h + (i16 >> 2) + 8 * hf;
        const int chunk = 4 * dt + 2 * (G & 1) + ((i16 & 3) >> 1);
        voff[dt][hf] = vring + r * C::ROW + 16 * (chunk ^ swz(r)) + 8 * (i16 & 1);
        asm volatile("" : "+v"(voff[dt][hf]));
      }
      voff16[dt] = vring + (32 * dt + n) * 32 + 16 * (h ^ ((n >> 3) & 1));
      if constexpr (F16) asm volatile("" : "+v"(voff16[dt]));
    }
  }
  // F8: per-lane base of the scale reads (this lane's keys start at 4h in each 8-key run);
  // the ring slot, the K/V half and the key run are immediates
  uint32_t scoff = lds_addr(smem + SC_RING) + 16 * h;
  asm volatile("" : "+v"(scoff));



  // Two wave groups in ping-pong.  Each wave alternates a matrix phase M(i) (O += V(i-1)
  // P(i-1), then S(i) = QK^T of K tile i) and a vector phase X(i) (mask, running max and the
  // probabilities P(i) of S(i)).  Waves 0-3 (group A) and 4-7 (group B) hold one wave of each
  // group per SIMD, and B runs one phase behind A, with a workgroup barrier between phases:
  // while one wave of a SIMD keeps the matrix core busy, the other does its exponentials.
  //
  // Slots (barrier-separated): A runs M(i) in slot 2i and X(i) in slot 2i+1; B runs M(i) in
  // slot 2i+1 and X(i) in slot 2i+2.  Tile i lives in ring slot i % 3.  K tile i is read in
  // slots 2i and 2i+1, V tile i in slots 2i+2 and 2i+3.  At the start of slot 2i every wave
  // issues its share of V(i+1), then of K(i+2) (their ring slots were last read in slot
  // 2i-1).  The end of slot 2i+1 waits until only the K(i+2) loads may still be in flight
  // (vmcnt counts in issue order): V(i+1) has two slots to spare before slot 2i+4 reads it,
  // K(i+2) gets four slots before slot 2i+4 reads it.
  auto vbuf = [&](int b) { return smem + V_RING + b * C::TILE; };
  auto kbuf = [&](int b) { return smem + K_RING + b * C::TILE; };
  auto scbuf = [&](int b) { return smem + SC_RING + b * SC_TILE; };
  const bool grp_a = w < WAVES / 2;                          // uniform
  auto bar = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  static_assert(UK == 2, "the wait counts below assume two load instructions per tile and wave");
  auto bar_loads = [&](int32_t i) {
    if (i + 2 < ntiles)
      asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  {
    const Blocks bl0 = fetch_blocks(0), bl1 = fetch_blocks(1);
    issue_k(0, bl0, kbuf(0));
    issue_v(0, bl0, vbuf(0));
    issue_sc(0, bl0, scbuf(0));
    if (ntiles > 1) issue_k(1, bl1, kbuf(1));
  }
  Blocks blV = fetch_blocks(1);                              // blocks of V(i+1)
  Blocks blK = fetch_blocks(2);                              // blocks of K(i+2)
  // the V slot that the first matrix phase multiplies by P = 0 holds zeros (finite)
  for (int c = tid; c < C::TILE / 16; c += NT) *(u32x4*)(vbuf(NBUF - 1) + 16 * c) = u32x4{0u, 0u, 0u, 0u};
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // P = i % 3 is a compile-time constant in every call below (the slot loop is unrolled by
  // three), so all LDS addresses are per-lane offsets plus immediates
  auto issue_slot = [&](int32_t i, auto par) {
    constexpr int P = decltype(par)::value;
    if (i + 1 < ntiles) {
      issue_v(i + 1, blV, vbuf((P + 1) % NBUF));
      issue_sc(i + 1, blV, scbuf((P + 1) % NBUF));         // before K(i+2): the waits count K last
    }
    if (i + 2 < ntiles) issue_k(i + 2, blK, kbuf((P + 2) % NBUF));
    blV = blK;
    blK = fetch_blocks(i + 3);
  };

  f32x16 s[2];
  // P of the last vector phase: fp16 pairs (fast kernel), or the bf16 high parts with pl
  // holding the bf16 roundings of the remainders
  u32x4 pb[4], pl[F16 ? 1 : 4];
#pragma unroll
  for (int c = 0; c < 4; ++c) pb[c] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < (F16 ? 1 : 4); ++c) pl[c] = u32x4{0u, 0u, 0u, 0u};
  // bf16 pools' fast kernel: the first two V^T chunks of the next matrix phase, read by the
  // vector phase before it (the fp8 kernel, at 252 registers with it, measured 0.3-1% slower
  // with it).  A matrix phase reads its operands from LDS with the other wave of its SIMD idle on
  // LDS (it does vector work), and at one reading wave per SIMD LDS serves about 90 B/clk per
  // CU, less than the products consume; the vector phase's reads run beside the other
  // wave's, so the matrix phase starts with two of its eight operand groups in registers.
  constexpr bool VPRE = F16 && !F8;
  u32x4 vpre[2][C::DT];
  // V^T operand of one 16-key chunk for the four d tiles (eight transpose reads)
  auto read_v = [&](int b, int qc, u32x4* va) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      if constexpr (F16) {
        // block qc of the tile (4 KB each): this lane's 8 keys of dim 32dt + n, one read
        va[dt] = __builtin_bit_cast(u32x4, lds_read16(voff16[dt] + b * C::TILE + 4096 * qc));
      } else {
        const bf16x4 v0 = tr_read(voff[dt][0] + b * C::TILE + 16 * qc * C::ROW);
        const bf16x4 v1 = tr_read(voff[dt][1] + b * C::TILE + 16 * qc * C::ROW);
        va[dt] = __builtin_bit_cast(u32x4, bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
      }
    }
  };
  if constexpr (VPRE) {                                     // M(0) multiplies the zeroed slot by P = 0
    read_v(NBUF - 1, 0, vpre[0]);
    read_v(NBUF - 1, 1, vpre[1]);
  }
  // The matrix phase as one stream of eight operand groups: the four V^T chunks of
  // O += V(i-1) P(i-1), then the four K groups of S(i) = QK^T (two k-chunks of both 32-key
  // halves, so consecutive products accumulate into different tiles).  Each group's LDS
  // reads are issued one group before its products, across the PV/QK boundary too, and
  // scheduling fences keep that order: the matrix core does not wait on LDS.  (VPRE: the
  // first two groups come read ahead in vpre.)
  // One code path for every tile: at i = 0 the PV products run on a zeroed V slot with
  // P = 0, and at i = ntiles the scores of a stale K slot are never used.
  auto phase_m = [&](int32_t i, auto par) {
    constexpr int P = decltype(par)::value;
    constexpr int Vb = (P + NBUF - 1) % NBUF;
    u32x4 buf[2][4];
    auto rd = [&](int q, u32x4* bb) {
      if (q < 4) {
        read_v(Vb, q, bb);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = 2 * (q - 4) + (e >> 1), sh = e & 1;
          bb[e] = __builtin_bit_cast(u32x4, lds_read16(koff[kk] + P * C::TILE + 32 * sh * C::ROW));
        }
      }
    };
    if constexpr (VPRE) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) buf[0][dt] = vpre[0][dt];
    } else {
      rd(0, buf[0]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (VPRE && q == 0) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) buf[1][dt] = vpre[1][dt];
      } else if (q + 1 < 8) {
        rd(q + 1, buf[(q + 1) & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      u32x4* bb = buf[q & 1];
      if (q < 4) {
        // O^T += V^T P^T for 16-key chunk q, one product per d tile (two in the bf16 kernel:
        // high parts, then low parts)
        if constexpr (F16) {
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, bb[dt]),
                                                           __builtin_bit_cast(f16x8, pb[q]), o[dt], 0, 0, 0);
        } else {
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bb[dt]),
                                                            __builtin_bit_cast(bf16x8, pb[q]), o[dt], 0, 0, 0);
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bb[dt]),
                                                            __builtin_bit_cast(bf16x8, pl[q]), o[dt], 0, 0, 0);
        }
      } else {
        // S^T of K tile i, k-chunks 2g and 2g+1 of both 32-key halves
        const int g = q - 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = 2 * g + (e >> 1), sh = e & 1;
          s[sh] = kk == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bb[e]), qf[kk],
                                                                    f32x16{}, 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bb[e]), qf[kk],
                                                                    s[sh], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto phase_x = [&](int32_t i, auto par) {
    constexpr int P = decltype(par)::value;
    if (i >= ntiles) return;
    // F8: the base-2 exponents against the reference the row has now, s k - m0, one FMA per
    // score with its key's K scale (score r of this lane is key 32sh + 8(r/4) + 4h + r%4 of
    // the tile), before the mask so that a masked score is -inf whatever the scale.  The max
    // below is then taken over these exponents, and the rare move of the reference shifts them.
    const float m0 = m == kNegInf ? 0.f : m;
    if constexpr (F8) {
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 k4 = *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)(
              scoff + P * SC_TILE + 4 * (32 * sh + 8 * q));
#pragma unroll
          for (int e = 0; e < 4; ++e) s[sh][4 * q + e] = __builtin_fmaf(s[sh][4 * q + e], k4[e], -m0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);                   // keep the scale reads' registers short-lived
    }
    // causal mask on the diagonal tiles, window mask on the tiles holding some row's window
    // start; masked scores are -inf before the max.  This lane's score r is key kt + off + 4h.
    const int32_t kt = (i + t0) * kBK;
    const bool diag = kt + kBK - 1 > c + tok0 || Tn < BQ;
    const bool edge = a.window > 0 && kt <= c + tok0 + Tn - 1 - a.window;
    if (diag || edge) {
      const int32_t lim = row_ok ? pos - kt - 4 * h : -1000000;      // off > lim: after the row
      // off <= lo: before the row's window (clamped to -1 .. 64 so it cannot overflow)
      const int64_t lo64 = (a.window > 0 && row_ok) ? (int64_t)pos - a.window - kt - 4 * h : -1;
      const int32_t lo = (int32_t)(lo64 < -1 ? -1 : (lo64 > 64 ? 64 : lo64));
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * sh + 8 * (r >> 2) + (r & 3);
          s[sh][r] = (off > lim || off <= lo) ? kNegInf : s[sh][r];
        }
      }
    }
    // two chains of three-operand maxima (one v_max3 per two scores)
    float mxa = fmaxf(s[0][0], s[0][1]), mxb = fmaxf(s[1][0], s[1][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      mxa = fmaxf(fmaxf(mxa, s[0][r]), s[0][r + 1]);
      mxb = fmaxf(fmaxf(mxb, s[1][r]), s[1][r + 1]);
    }
    float mx = max_xor32(fmaxf(mxa, mxb));
    // the row's max in base-2 exponent units (F8: the exponents were taken against m0)
    const float mxs = F8 ? mx + m0 : mx * sl;               // mx is finite or -inf, sl > 0
    // move the reference only when the row max grew by more than kLazy (or it is unset)
    if (__builtin_amdgcn_ballot_w64(mxs > m + kLazy) != 0) {
      const float m_new = mxs > m + kLazy ? mxs : m;
      const float alpha = m_new > m ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;   // m may be -inf
      m = m_new;
      lsum *= alpha;
      lsum2 *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
      if constexpr (F8) {
        // the exponents against the new reference (-inf stays -inf; the shift is finite)
        const float shift = m0 - (m == kNegInf ? 0.f : m);
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[sh][r] += shift;
        }
      }
    }
    const float m_use = m == kNegInf ? 0.f : m;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        // F8, bf16 kernel: the V scales of this group's eight keys (two 4-key runs)
        f32x4 vsc[2];
        if constexpr (F8 && !F16) {
#pragma unroll
          for (int hq = 0; hq < 2; ++hq)
            vsc[hq] = *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)(
                scoff + P * SC_TILE + 256 + 4 * (32 * sh + 8 * (2 * kh + hq)));
        }
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) {
          // (F8: s already holds the exponents)
          const float p0 = __builtin_amdgcn_exp2f(F8 ? s[sh][8 * kh + jj] : __builtin_fmaf(s[sh][8 * kh + jj], sl, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(F8 ? s[sh][8 * kh + jj + 1]
                                                     : __builtin_fmaf(s[sh][8 * kh + jj + 1], sl, -m_use));
          if constexpr (F16) {
            // rounded to nearest fp16 (p <= 2^kLazy, inside its range); l adds up the same
            // rounded values, so the output is an exact convex combination of V rows whose
            // weights are off by at most 2^-12 (relative)
            const f16x2 pr = {(_Float16)p0, (_Float16)p1};
            // one dot product with (1, 1) adds both rounded values into a float32 sum (the
            // products are exact); two accumulators halve the dependency chain
            const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
            if (jj & 2) lsum2 = __builtin_amdgcn_fdot2(pr, ones, lsum2, false);
            else lsum = __builtin_amdgcn_fdot2(pr, ones, lsum, false);
            pb[2 * sh + kh][jj >> 1] = __builtin_bit_cast(uint32_t, pr);
          } else {
            lsum += p0 + p1;
            float q0 = p0, q1 = p1;
            if constexpr (F8) {
              // times the keys' V scales for the PV product (score 8kh + jj is key 32sh +
              // 8(2kh + jj/4) + 4h + jj%4)
              q0 *= vsc[jj >> 2][jj & 3];
              q1 *= vsc[jj >> 2][(jj & 3) + 1];
            }
            const uint32_t h0 = __float_as_uint(q0) & 0xffff0000u, h1 = __float_as_uint(q1) & 0xffff0000u;
            const float r0 = q0 - __uint_as_float(h0), r1 = q1 - __uint_as_float(h1);
            pb[2 * sh + kh][jj >> 1] = __builtin_amdgcn_perm(h1, h0, 0x07060302u);   // {h0.hi16, h1.hi16}
            const bf16x2 lo = {(__bf16)r0, (__bf16)r1};
            pl[2 * sh + kh][jj >> 1] = __builtin_bit_cast(uint32_t, lo);
          }
        }
        if constexpr (F8) __builtin_amdgcn_sched_barrier(0);
      }
    }
    // for M(i + 1): V tile i, chunks 0 and 1.  V tile i was published by the barrier at the
    // end of slot 2i - 1 and is next overwritten by the V(i + 3) loads issued from slot 2i + 4
    // on; this phase runs in slot 2i + 1 (A) or 2i + 2 (B), and its reads complete before the
    // barrier that ends it (lgkmcnt(0)).
    if constexpr (VPRE) {
      read_v(P, 0, vpre[0]);
      read_v(P, 1, vpre[1]);
    }
  };

  // every wave passes 2 * ntiles + 3 barriers in the loop below
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  auto step = [&](int32_t i, auto par) {
    constexpr int P = decltype(par)::value;
    using Pn = std::integral_constant<int, (P + 1) % NBUF>;
    if (grp_a) issue_slot(i, par);
    phase_m(i, par);
    if (grp_a) bar(); else bar_loads(i);
    if (!grp_a) issue_slot(i + 1, Pn{});
    phase_x(i, par);
    if (grp_a) bar_loads(i); else bar();
  };
  if (!grp_a) {
    issue_slot(0, P0{});
    bar();
  }
  for (int32_t i = 0; i <= ntiles; i += 3) {
    step(i, P0{});
    if (i + 1 <= ntiles) step(i + 1, P1{});
    if (i + 2 <= ntiles) step(i + 2, P2{});
  }
  if (grp_a) bar();

  // normalise and stage the tile's output rows in LDS, then write them out coalesced
  lsum += lsum2;
  lsum += __shfl_xor(lsum, 32);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  __syncthreads();                                          // all waves done with the K/V tiles (the
                                                            // last barrier passed with every load landed)
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
  if (p.D != 128) return hipErrorInvalidValue;
  const PfItem* items = (const PfItem*)((char*)ws + p.off_pf);
  int32_t* wide = (int32_t*)((char*)ws + p.off_pf_wide);     // zeroed by the plan kernel
  const int64_t total = p.n_pf * p.Hkv;
  const dim3 grid((unsigned)((total + 7) / 8 * 8));
  if (p.f8) {   // the staged copies of fp8 pools (launched by launch_stage_fp8)
    hipLaunchKernelGGL((prefill_tile_mfma<128, kWaves, true, true>), grid, dim3(64 * kWaves), 0, s, a, items,
                       (int32_t)p.n_pf, wide);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // items whose dequantized V left fp16's range (normally none: these workgroups exit at once)
    hipLaunchKernelGGL((prefill_tile_mfma<128, kWaves, false, true>), grid, dim3(64 * kWaves), 0, s, a, items,
                       (int32_t)p.n_pf, wide);
    return hipGetLastError();
  }
  // bf16 pools: V to fp16 once (flagging out-of-range items), then the fast kernel on it
  if (!p.v16) return hipErrorInvalidValue;
  hipError_t e = launch_stage_v16(p, a, ws, s);
  if (e != hipSuccess) return e;
  AttnArgs av = a;
  av.v_staged = (char*)ws + p.off_v16;
  av.req = (const ReqOffsets*)((char*)ws + p.off_req);
  hipLaunchKernelGGL((prefill_tile_mfma<128, kWaves, true, false>), grid, dim3(64 * kWaves), 0, s, av, items,
                     (int32_t)p.n_pf, wide);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // items whose V left fp16's range (normally none: these workgroups exit at once)
  hipLaunchKernelGGL((prefill_tile_mfma<128, kWaves, false, false>), grid, dim3(64 * kWaves), 0, s, a, items,
                     (int32_t)p.n_pf, wide);
  return hipGetLastError();
}

}  // namespace pa
