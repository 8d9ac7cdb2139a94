// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace pa {

constexpr int kWave = 64;
constexpr int kCols = 16;          // query columns (token, head) of one small tile

// ---------------------------------------------------------------- element conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16 bits, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float x) { *p = f32_to_bf16_bits(x); }
};

// four fp8 E4M3 codes (one dword) to four bf16 values, exactly (4 significant bits fit in 8,
// and every E4M3 exponent is inside bf16's range)
typedef uint32_t pa_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ pa_u32x2 fp8x4_to_bf16x4(uint32_t w) {
  typedef float f32x2_ __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x4_ __attribute__((ext_vector_type(4)));
  const f32x2_ lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  const bf16x4_ r = {(__bf16)lo[0], (__bf16)lo[1], (__bf16)hi[0], (__bf16)hi[1]};
  return __builtin_bit_cast(pa_u32x2, r);
}

// ---------------------------------------------------------------- work decomposition
// A "small tile" is up to 16 query columns of one request and one KV head: `tile_tokens`
// consecutive query rows times `tile_heads` of the KV head's query heads, over one key
// split.  A "prefill tile" is `pf_tokens` consecutive rows times all query heads of one KV
// head (a bf16 matrix-core tile); it covers all keys in one pass.
struct Plan {
  int32_t R, H, Hkv, g, D, bs;
  int32_t tile_tokens, tile_heads, hsubs;
  int32_t split_keys;              // keys per split of a small tile
  int32_t pf_tokens;               // 0: prefill path off
  int32_t decode_kind;             // 0: vector kernel, 1: bf16 matrix-core kernel
  int32_t window;                  // sliding window in tokens (0: none)
  int32_t f8;                      // 1: fp8 pools (prefill requests read staged bf16 K codes)
  int32_t v16;                     // 1: prefill requests read V from a staged fp16 copy (bf16
                                   //    pools: V converted; fp8 pools: the codes times their scales)
  int32_t graph_max;               // > 0: the call is sized for every seq_len = graph_max (the
                                   //      planner counts device lengths clamped to it)
  int32_t inline_items;            // 1: no planner launch; the matrix-core small kernels and the
                                   //    merge derive their own items (at most 64 requests, no
                                   //    prefill-path request)
  int64_t n_small, n_merge, n_pf;  // item counts (host-computed); n_small counts tile-splits
  int64_t n_g1, n_g3;              // matrix-core small kernels: single-tile and grouped items
  int64_t n_stage;                 // staged blocks of the prefill requests
  // workspace layout (byte offsets)
  size_t off_req, off_small, off_merge, off_pf, off_pf_wide, off_pm, off_pl, off_pacc, off_g1, off_g3;
  size_t off_f8_k, off_f8_v, off_f8_s, off_v16, total_bytes;
};

struct alignas(16) SmallItem {
  int32_t r, tok0, hsub, split;
  int32_t nsplit, first;   // first: tile-split index of the (first) tile's split 0 (partials base)
  int32_t tile0, ntile;    // the item's first tile of its request and its tile count
};
struct alignas(16) MergeItem {
  int32_t r, tok0, hsub, first;
  int32_t nsplit;
  int32_t row0, ntok;      // the tile's first output row (query_start_loc[r] + tok0) and row count
  int32_t pad0;
};
struct alignas(8) PfItem {
  int32_t r, tok0;
};
// per-request offsets written by the planner (exclusive scans)
struct alignas(16) ReqOffsets {
  int32_t small, merge, pf, nsplit;
  int32_t stage;                       // first staged block of the request
  int32_t g1, g3;                      // offsets in the matrix-core small kernels' two item lists
  int32_t pad0;
};
// indices into the request offsets seen as int32 (the totals row req[R])
constexpr int kTotalSmall = 0, kTotalMerge = 1, kTotalPf = 2, kTotalG1 = 5, kTotalG3 = 6;

// Small-tile shape for a group of g query heads per KV head: 16 columns are 16/g tokens
// times the g heads, or (g >= 16) one token times 16 of its heads, the group then being cut
// into g/16 head subsets.
__host__ __device__ __forceinline__ void set_tile_shape(Plan& p) {
  if (p.g >= kCols) {
    p.tile_heads = kCols;
    p.tile_tokens = 1;
  } else {
    p.tile_heads = p.g;
    p.tile_tokens = kCols / p.g;
  }
  p.hsubs = (p.g + p.tile_heads - 1) / p.tile_heads;
}

// Classification of request r, identical on host and device.  Up to four small tiles (64
// query columns: decodes, speculative-verification rows, short chunks) stay on the small
// tiles, whose key splits spread a long context over many workgroups; longer chunks fill
// the prefill kernel's 256-row tiles.
constexpr int kPrefillMinCols = 4 * kCols;
__host__ __device__ __forceinline__ bool use_prefill_path(const Plan& p, int32_t t, int32_t L) {
  return p.pf_tokens > 0 && L > 0 && (int64_t)t * p.g > kPrefillMinCols;
}
// First block of a prefill-path request that the fp16 V copy holds: under a sliding window
// of w tokens its first row (at position L - t) sees keys from L - t - w + 1 on, and the
// prefill tiles start at a multiple of 64 keys (four 16-key blocks) below that.
__host__ __device__ __forceinline__ int32_t v16_first_block(int32_t window, int32_t t, int32_t L) {
  if (window <= 0) return 0;
  const int64_t k0 = (int64_t)L - t - window + 1;
  return k0 <= 0 ? 0 : (int32_t)(4 * (k0 / 64));
}
// Order of the keys of a 16-key block in a row of the transposed fp16 V copy: position q
// holds key kperm(q), bits 2 and 3 swapped (an involution).  It is the order in which the
// prefill kernel's P^T fragments hold their keys, so that a lane's 8 keys of one dim are
// one 16-byte read.
__host__ __device__ __forceinline__ int kperm(int q) { return (q & 3) | ((q & 4) << 1) | ((q & 8) >> 1); }
// Staged blocks of a prefill-path request: the blocks of every 64-key tile from
// v16_first_block on (the last tile's blocks past the request's end are staged as zeros), for
// the fp16 V copy and, on fp8 pools, the bf16 copies of the codes and the scales.  Block j of
// the request is staged block req.stage + j - v16_first_block.
__host__ __device__ __forceinline__ int32_t staged_blocks(const Plan& p, int32_t t, int32_t L) {
  if (!use_prefill_path(p, t, L) || !p.v16) return 0;
  return 4 * ((L + 63) / 64) - v16_first_block(p.window, t, L);
}
// Keys one small tile of a request with context L can see: all L, or with a sliding window
// of w tokens at most w + tile_tokens - 1 (the tile's rows are consecutive), plus up to 63
// because a tile's key range starts at a multiple of 64.
__host__ __device__ __forceinline__ int32_t small_key_span(const Plan& p, int32_t L) {
  if (p.window <= 0) return L;
  const int64_t span = (int64_t)p.window + p.tile_tokens + 62;
  return span < L ? (int32_t)span : L;
}
// First key of a small tile whose first row is at position pos0: 0, or the window start
// rounded down to a multiple of 64 (the key splits of the tile start there).
__host__ __device__ __forceinline__ int32_t small_key_base(int32_t window, int32_t pos0) {
  if (window <= 0 || pos0 - window + 1 <= 0) return 0;
  return ((pos0 - window + 1) / 64) * 64;
}
__host__ __device__ __forceinline__ int32_t small_nsplit(const Plan& p, int32_t L) {
  const int32_t span = small_key_span(p, L);
  return span <= 0 ? 1 : (span + p.split_keys - 1) / p.split_keys;
}
__host__ __device__ __forceinline__ void request_counts(const Plan& p, int32_t t, int32_t L,
                                                        int32_t* n_small, int32_t* n_merge,
                                                        int32_t* n_pf, int32_t* nsplit) {
  *n_small = *n_merge = *n_pf = 0;
  *nsplit = 1;
  if (t <= 0) return;
  if (use_prefill_path(p, t, L)) {
    *n_pf = (t + p.pf_tokens - 1) / p.pf_tokens;
    return;
  }
  const int32_t tiles = ((t + p.tile_tokens - 1) / p.tile_tokens) * p.hsubs;
  const int32_t ns = small_nsplit(p, L);
  *nsplit = ns;
  *n_small = tiles * ns;
  *n_merge = ns > 1 ? tiles : 0;
}

// The matrix-core small kernel's items: a request with one 16-column tile (a decode), or any
// request under a sliding window, gets one item per tile and key split; a wider request
// (speculative-verification rows, short chunks) gets one item per group of up to
// kGroupTiles consecutive tiles and key split, which reads each K/V block once for the group.
// (kGroupTiles tiles with bf16 pools; none with fp8 pools, whose kernel measured slower with
// the registers of a second tile than re-reading the codes)
//
// The list a request goes to depends only on t, the plan and the window, never on L: a call
// sized for a capacity (graph_max_seq_len) counts every request at L = capacity on the host,
// and the planner kernel recounts it at its device length, which may be anything from 0 (a
// padding row) up to the capacity.  Only the split count follows L, and it never decreases
// as L grows, so the device's counts never exceed the host's.  Both kernels zero the rows of
// a request with L = 0.
constexpr int kGroupTiles = 3;
__host__ __device__ __forceinline__ int32_t group_tiles(const Plan& p) { return p.f8 ? 1 : kGroupTiles; }
__host__ __device__ __forceinline__ void small_groups(const Plan& p, int32_t t, int32_t L, int32_t* n1, int32_t* n3) {
  *n1 = *n3 = 0;
  if (t <= 0 || use_prefill_path(p, t, L)) return;
  const int32_t tiles = ((t + p.tile_tokens - 1) / p.tile_tokens) * p.hsubs;
  const int32_t ns = small_nsplit(p, L);
  const int32_t gt = group_tiles(p);
  if (tiles == 1 || gt == 1 || p.window > 0) *n1 = tiles * ns;
  else *n3 = ((tiles + gt - 1) / gt) * ns;
}

// The items of the small tiles' lists, from the owning request's exclusive offsets (the
// planner's scans) and the item's index li within the request.  o_small: the request's first
// tile-split index (its partials); ns: its key splits; t, q0: its query rows and first row.
// single tile (a decode, or any request under a window or on fp8 pools): one item per
// (tile, split); also the vector kernel's per-tile list
__host__ __device__ __forceinline__ SmallItem single_item(const Plan& p, int32_t r, int32_t li, int32_t ns,
                                                          int32_t o_small) {
  const int32_t tile = li / ns;
  SmallItem it;
  it.r = r;
  it.tok0 = (tile / p.hsubs) * p.tile_tokens;
  it.hsub = tile % p.hsubs;
  it.split = li - tile * ns;
  it.nsplit = ns;
  it.first = o_small + tile * ns;
  it.tile0 = tile;
  it.ntile = 1;
  return it;
}
// group of up to group_tiles(p) consecutive tiles: one item per (group, split)
__host__ __device__ __forceinline__ SmallItem group_item(const Plan& p, int32_t r, int32_t li, int32_t ns,
                                                         int32_t o_small, int32_t t) {
  const int32_t tiles = ((t + p.tile_tokens - 1) / p.tile_tokens) * p.hsubs;
  const int32_t grp = li / ns;
  const int32_t tile0 = grp * group_tiles(p);
  SmallItem it;
  it.r = r;
  it.tok0 = (tile0 / p.hsubs) * p.tile_tokens;
  it.hsub = tile0 % p.hsubs;
  it.split = li - grp * ns;
  it.nsplit = ns;
  it.first = o_small + tile0 * ns;
  it.tile0 = tile0;
  it.ntile = min(group_tiles(p), tiles - tile0);
  return it;
}
// the merge of tile `tile` of a request with more than one split
__host__ __device__ __forceinline__ MergeItem merge_item(const Plan& p, int32_t r, int32_t tile, int32_t ns,
                                                         int32_t o_small, int32_t t, int32_t q0) {
  MergeItem it;
  it.r = r;
  it.tok0 = (tile / p.hsubs) * p.tile_tokens;
  it.hsub = tile % p.hsubs;
  it.first = o_small + tile * ns;
  it.nsplit = ns;
  it.row0 = q0 + it.tok0;
  it.ntok = min(p.tile_tokens, t - it.tok0);
  it.pad0 = 0;
  return it;
}

// Without a planner launch (Plan::inline_items: at most 64 requests, all on the small tiles)
// every workgroup of the small kernels and of the merge finds its own item: lane r of each
// wave counts request r with the planner's formulas, a wave prefix sum gives the offsets the
// planner's scan would, and the lane whose range holds the item's index owns it.
constexpr int kInlineMaxReqs = 64;
enum InlineList { kListSingle = 0, kListGroup = 1, kListMerge = 2 };
struct InlineOwner {
  int32_t r;                 // -1: the index is past the list's end (the workgroup exits)
  int32_t li;                // the item's index within its request's items
  int32_t o_small, ns, t, q0;
  int32_t L;                 // the request's seq_len as given (not clamped)
};
// Inclusive prefix sum over the 64 lanes with DPP moves: shifts by 1, 2, 4, 8 within each row
// of 16 lanes (a lane with no source lane adds 0), then the last lane of row 0 added to row 1
// and of row 2 to row 3 (row_bcast:15), then the last lane of row 1 to rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
  return v;
}
__device__ __forceinline__ InlineOwner inline_owner(const Plan& p, const int32_t* qsl, const int32_t* seq_lens,
                                                    int list, int32_t idx) {
  const int lane = threadIdx.x & 63;
  int32_t t = 0, q0 = 0, n_small = 0, n_list = 0, ns = 1, Lr = 0;
  if (lane < p.R) {
    q0 = qsl[lane];
    t = qsl[lane + 1] - q0;
    Lr = seq_lens[lane];
    // (as the planner: a call sized for a capacity counts lengths clamped to it)
    const int32_t L = p.graph_max > 0 ? min(Lr, p.graph_max) : Lr;
    int32_t nm, np, n1, n3;
    request_counts(p, t, L, &n_small, &nm, &np, &ns);
    small_groups(p, t, L, &n1, &n3);
    n_list = list == kListSingle ? n1 : list == kListGroup ? n3 : nm;
  }
  const int32_t end_list = wave_inclusive_sum(n_list), end_small = wave_inclusive_sum(n_small);
  const unsigned long long own = __ballot(idx >= end_list - n_list && idx < end_list);
  InlineOwner o;
  if (own == 0) {
    o.r = -1;
    return o;
  }
  const int w = __builtin_ctzll(own);                           // uniform: read the owner lane
  o.r = w;
  o.li = idx - __builtin_amdgcn_readlane(end_list - n_list, w);
  o.o_small = __builtin_amdgcn_readlane(end_small - n_small, w);
  o.ns = __builtin_amdgcn_readlane(ns, w);
  o.t = __builtin_amdgcn_readlane(t, w);
  o.q0 = __builtin_amdgcn_readlane(q0, w);
  o.L = __builtin_amdgcn_readlane(Lr, w);
  return o;
}

// Arguments common to the attention kernels.
struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* block_table;
  void* out;
  int32_t bs, stride, H, Hkv, g, D;
  int32_t tile_tokens, tile_heads, split_keys;
  int32_t window;                    // sliding window in tokens: a row at position p sees keys
                                     // p - window + 1 .. p; 0: keys 0 .. p
  float scale_log2e;                 // scale * log2(e): scores are kept in base 2
  // {small, merge, prefill} item counts the planner kernel wrote for this call (workspace).
  // Grids are sized on the host; a workgroup past the device count exits (the counts agree
  // except when a captured graph replays with shorter contexts than it was sized for).
  const int32_t* totals;
  // fp8 pools: float32 scales [num_slots, Hkv] of K and V (null: the pools hold q's dtype)
  const float* k_scale;
  const float* v_scale;
  // prefill requests: the transposed fp16 copy [staged block][Hkv][D][16] of their V blocks
  // (request r's block j at staged block req[r].stage + j - first, first = v16_first_block;
  // within a row, position q holds key kperm(q)).  On fp8 pools k_cache / v_cache / k_scale
  // of the prefill kernels point at the staged bf16 codes [staged block][16][Hkv][D] and
  // the staged scales, at the same staged block numbers.
  const void* v_staged;
  const ReqOffsets* req;
};

struct Partials {
  float* m;      // [n_small * Hkv * 16]
  float* l;      // [n_small * Hkv * 16]
  float* acc;    // [n_small * Hkv * 16 * D]
};

// ---------------------------------------------------------------- launchers (host)
hipError_t launch_kv_write(const void* k, const void* v, const int64_t* slots, void* kc, void* vc,
                           int64_t n, int32_t row_elems, int64_t num_slots, int32_t in_dtype,
                           int32_t cache_dtype, hipStream_t s);
hipError_t launch_plan(const Plan& p, const int32_t* qsl, const int32_t* seq_lens, void* ws, hipStream_t s);
hipError_t launch_kv_write_fp8(const void* k, const void* v, const int64_t* slots, void* kc, void* vc, float* ks,
                               float* vs, int64_t n, int32_t hkv, int32_t d, int64_t num_slots, int32_t in_dtype,
                               hipStream_t s);
hipError_t launch_copy_blocks(const void* src, void* dst, const int64_t* src_block, const int64_t* dst_block,
                              int64_t num_pairs, int64_t block_bytes, hipStream_t s);
hipError_t launch_small_valu(const Plan& p, const AttnArgs& a, void* ws, int32_t dtype, hipStream_t s);
hipError_t launch_small_mfma(const Plan& p, const AttnArgs& a, void* ws, hipStream_t s);
hipError_t launch_merge(const Plan& p, const AttnArgs& a, void* ws, int32_t dtype, hipStream_t s);
hipError_t launch_prefill_mfma(const Plan& p, const AttnArgs& a, void* ws, hipStream_t s);
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, hipStream_t s);
hipError_t launch_mfma_probe(int32_t iters, int32_t data, uint32_t* sink, int32_t grid, hipStream_t s);
int64_t mfma_probe_flops(int32_t iters, int32_t grid);
// fp8 pools: stage the prefill requests' blocks (bf16 codes, scales, the fp16 V copy), then
// run the prefill kernels on them
hipError_t launch_stage_fp8(const Plan& p, const AttnArgs& a, float scale_abs_log2e, void* ws, hipStream_t s);
// bf16 pools: copy the prefill requests' V blocks to fp16 (flagging, for the bf16 prefill
// kernel, the items whose V leaves fp16's range)
hipError_t launch_stage_v16(const Plan& p, const AttnArgs& a, void* ws, hipStream_t s);
bool small_mfma_supported(int32_t D, int32_t bs, bool fp8);
bool prefill_mfma_supported(int32_t D, int32_t bs, int32_t g);
int32_t prefill_tile_tokens(int32_t g);

}  // namespace pa
