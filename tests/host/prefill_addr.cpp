// Host replica of the prefill path's address arithmetic, checked against the allocations.
//
// The prefill kernels (attn_prefill_mfma.hip: the fp16 kernel and the bf16 redo kernel, for
// bf16 and for fp8 pools) and their staging kernels (v16_stage.hip, fp8_stage.hip) compute every global
// address from the planner's items and the batch layout.  This program redoes that
// arithmetic on the host, lane by lane, for every workgroup of every launch a batch makes,
// and checks each access against its buffer:
//   - the workgroup -> (item, KV head) map covers every pair exactly once;
//   - block-table entries read are inside the request's row and below ceil(L / bs): entries
//     past a request's last block are never read ("Attention over the pool" of "Engine v2:
//     one core for every request"), whether full tiles (entries 4j .. 4j+3, one tile ahead)
//     or the last, partial tile (keys clamped to kend - 1);
//   - K/V pool rows, the staged fp16 V rows (stage0 + 4(j + t0) + block), the staged bf16
//     codes and scales of fp8 pools (staged blocks of the request itself), q and out rows
//     are inside their buffers;
//   - ring slot i % 3 and the LDS destinations stay inside the kernel's shared memory.
// The pool block ids themselves come from the batch (every parity batch's tables hold valid
// ids); they are checked too.
//
// It also checks the composition of a 64-bit scalar base from two readfirstlane halves, the
// form the direct-to-LDS loads use (readfirstlane returns int): the low half has to go
// through uint32_t, or a base whose bit 31 is set gets its high word filled with ones.
//
// Input (stdin), one batch per record:
//   batch <name> R H Hkv D bs window f8 num_blocks stride num_tokens
//   <R + 1 query_start_loc> <R seq_lens> <R * stride block table>
// Prints failures (at most 20) and "checked N batches, M accesses"; exits non-zero on failure.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace {

int64_t failures = 0, accesses = 0;
std::string cur;

void expect(bool ok, const char* what, int64_t a = 0, int64_t b = 0, int64_t c = 0) {
  ++accesses;
  if (ok) return;
  if (++failures <= 20)
    std::printf("FAIL %s: %s (%lld, %lld, %lld)\n", cur.c_str(), what, (long long)a, (long long)b, (long long)c);
}
void in_range(int64_t first, int64_t count, int64_t size, const char* what) {
  expect(first >= 0 && first + count <= size, what, first, count, size);
}

// ---- the scalar-base composition of the direct loads
int32_t readfirstlane(uint32_t x) { return (int32_t)x; }   // the builtin's type: int
uint64_t compose_base(uint64_t b64) {                       // the kernel's form
  return ((uint64_t)(uint32_t)readfirstlane((uint32_t)(b64 >> 32)) << 32) |
         (uint64_t)(uint32_t)readfirstlane((uint32_t)b64);
}
uint64_t compose_base_sign_extended(uint64_t b64) {         // without the uint32_t casts
  return ((uint64_t)readfirstlane((uint32_t)(b64 >> 32)) << 32) | (uint64_t)(int64_t)readfirstlane((uint32_t)b64);
}

struct BatchIn {
  std::string name;
  int32_t R, H, Hkv, D, bs, window, f8, num_blocks, stride;
  int64_t N;
  std::vector<int32_t> qsl, lens, table;
};

constexpr int kWaves = 8, kRows = 32 * kWaves, kBK = 64, kBlk = 16, kNBuf = 3;

void check_batch(const BatchIn& B) {
  cur = B.name;
  const int32_t g = B.H / B.Hkv;
  // the prefill path's conditions (api.cpp: bf16 or fp8 pools at head_dim 128, block_size 16,
  // a group size that divides the 256-row tile)
  const bool pf_ok = B.bs == kBlk && B.D == 128 && kRows % g == 0;
  if (!pf_ok) return;
  pa::Plan p{};
  p.R = B.R; p.H = B.H; p.Hkv = B.Hkv; p.g = g; p.D = B.D; p.bs = B.bs;
  pa::set_tile_shape(p);
  p.pf_tokens = kRows / g;
  p.decode_kind = 1;
  p.window = B.window;
  p.f8 = B.f8;
  p.v16 = 1;

  // ---- the planner: per-request offsets (exclusive scans) and the prefill items
  struct Req { int32_t pf, stage; };
  std::vector<Req> req(B.R + 1);
  std::vector<std::pair<int32_t, int32_t>> items;           // (r, tok0)
  int64_t n_stage = 0;
  for (int32_t r = 0; r < B.R; ++r) {
    const int32_t t = B.qsl[r + 1] - B.qsl[r], L = B.lens[r];
    int32_t a, b, npf, d;
    pa::request_counts(p, t, L, &a, &b, &npf, &d);
    const int32_t st = pa::staged_blocks(p, t, L);
    req[r] = Req{(int32_t)items.size(), (int32_t)n_stage};
    const int32_t tiles = npf > 0 ? (t + p.pf_tokens - 1) / p.pf_tokens : 0;
    for (int32_t li = 0; li < npf; ++li) items.push_back({r, (tiles - 1 - li) * p.pf_tokens});
    n_stage += st;
  }
  req[B.R] = Req{(int32_t)items.size(), (int32_t)n_stage};
  const int64_t n_items = (int64_t)items.size();
  if (n_items == 0) return;

  const int64_t row_elems = (int64_t)B.Hkv * B.D;
  const int64_t blk_stride = kBlk * row_elems;
  const int64_t pool_elems = (int64_t)(B.num_blocks + 1) * blk_stride;   // + the scratch block
  const int64_t qo_elems = B.N * B.H * B.D;
  auto nblocks_of = [&](int32_t r) { return (B.lens[r] + kBlk - 1) / kBlk; };

  // ---- staging kernels (stage_v16, or stage_fp8 on fp8 pools): one workgroup per staged
  // block, request r's block j at staged block req[r].stage + j - first
  const int64_t row_elems_s = (int64_t)B.Hkv * B.D;
  for (int64_t sb = 0; sb < n_stage; ++sb) {
    int lo = 0, hi = B.R - 1;                                // owner: largest r with stage <= sb
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (req[mid].stage <= sb) lo = mid;
      else hi = mid - 1;
    }
    const int32_t r = lo, t = B.qsl[r + 1] - B.qsl[r], L = B.lens[r];
    expect(sb - req[r].stage < req[r + 1].stage - req[r].stage, "staged block owner", sb, r);
    const int32_t j = (int32_t)(sb - req[r].stage) + pa::v16_first_block(B.window, t, L);
    const int32_t nkeys = std::min(16, L - 16 * j);
    if (nkeys > 0) {
      expect(j < nblocks_of(r) && j < B.stride && j >= 0, "staging: table entry", r, j);
      const int32_t src = B.table[(size_t)r * B.stride + j];
      for (int lk = 0; lk < nkeys; ++lk)
        in_range(((int64_t)src * 16 + lk) * row_elems_s, row_elems_s, pool_elems, "staging: pool row");
      if (B.f8)
        for (int lk = 0; lk < nkeys; ++lk)
          in_range(((int64_t)src * 16 + lk) * B.Hkv, B.Hkv, (int64_t)(B.num_blocks + 1) * 16 * B.Hkv,
                   "fp8 staging: scale of a pool slot");
    }
    for (int head = 0; head < B.Hkv; ++head) {
      for (int tid = 0; tid < 256; ++tid) {
        const int od = tid >> 1, oh = tid & 1, lk = tid >> 4, lc = tid & 15;
        in_range((((int64_t)sb * B.Hkv + head) * B.D + od) * 16 + 8 * oh, 8, n_stage * blk_stride,
                 "staging: transposed fp16 V row");
        if (B.f8)
          in_range(((int64_t)sb * 16 + lk) * row_elems_s + (int64_t)head * B.D + 8 * lc, 8, n_stage * blk_stride,
                   "fp8 staging: bf16 code row");
      }
      if (B.f8)
        for (int x = 0; x < 32; ++x)
          in_range((((int64_t)sb * 2 + (x >> 4)) * B.Hkv + head) * 16 + (x & 15), 1, n_stage * 2 * B.Hkv * 16,
                   "fp8 staging: staged scale");
    }
    for (int32_t it = req[r].pf; it < req[r + 1].pf; ++it)
      in_range((int64_t)(B.Hkv - 1) * n_items + it, 1, n_items * B.Hkv, "staging: range flag");
  }

  // ---- the prefill kernels: the fp16 kernel and the bf16 redo kernel of the pool kind
  const int TILE = kBK * 2 * B.D, V_RING = 0, K_RING = V_RING + kNBuf * TILE;
  const int SC_RING = K_RING + kNBuf * TILE, SC_TILE = B.f8 ? 2 * kBK * 4 : 0;
  const int SMEM = std::max(SC_RING + kNBuf * SC_TILE, kRows * 2 * B.D);
  const int64_t total = n_items * B.Hkv;
  const int64_t grid = (total + 7) / 8 * 8, per_xcd = (total + 7) / 8;
  std::vector<int> seen(total, 0);
  for (int64_t bid = 0; bid < grid; ++bid) {
    const int64_t lin = (bid % 8) * per_xcd + bid / 8;
    if (lin >= total) continue;
    ++seen[lin];
    const int32_t hkv = (int32_t)(lin / n_items);
    const int64_t idx = lin - hkv * n_items;
    const int32_t r = items[idx].first, tok0 = items[idx].second;
    const int32_t b = B.qsl[r], t = B.qsl[r + 1] - b, L = B.lens[r], c = L - t;
    const int32_t BQ = kRows / g;
    const int32_t Tn = std::min(BQ, t - tok0);
    const int32_t kend = c + tok0 + Tn;
    expect(Tn >= 1 && kend >= 1 && kend <= L, "item rows and key range", r, tok0, kend);
    const int32_t t0 = B.window > 0 ? std::max(0, c + tok0 - B.window + 1) / kBK : 0;
    const int32_t ntiles = (kend + kBK - 1) / kBK - t0;
    expect(ntiles >= 1, "item has a tile", r, tok0, ntiles);
    const int32_t* trow = &B.table[(size_t)r * B.stride];
    const int32_t tvalid = nblocks_of(r);                    // entries of the request
    // K (and the redo kernel's V): pool rows through the table, or (fp8 pools) the staged
    // bf16 code rows at staged block numbers
    const int64_t kv_elems = B.f8 ? n_stage * blk_stride : pool_elems;
    const int32_t stage0 = req[r].stage - pa::v16_first_block(B.window, t, L);
    auto entry = [&](int32_t e, const char* what) -> int32_t {
      expect(e >= 0 && e < tvalid, what, r, e, tvalid);
      if (B.f8) {
        const int32_t sb = stage0 + e;                       // one of the request's staged blocks
        expect(sb >= req[r].stage && sb < req[r + 1].stage, "staged block of the request", r, sb);
        return sb;
      }
      expect(e < B.stride, what, r, e, B.stride);
      if (e < 0 || e >= B.stride) return 0;
      const int32_t blk = trow[e];
      expect(blk >= 0 && blk <= B.num_blocks, "block id", r, e, blk);
      return blk;
    };
    // the block ids fetched one tile ahead: fetch_blocks(j) for j up to ntiles + 4
    for (int32_t j = 0; j <= ntiles + 4; ++j) {
      const int32_t jj = j + t0;
      if (jj * kBK + kBK > kend) continue;                   // partial or past the end: no read
      for (int e = 0; e < 4; ++e) entry(4 * jj + e, "full-tile table entry");
    }
    for (int w = 0; w < kWaves; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        const int n = lane & 31, h = lane >> 5;
        const int m_row = 32 * w + n, head_l = m_row / BQ, token = m_row - head_l * BQ;
        if (token < Tn)
          for (int kk = 0; kk < B.D / 16; ++kk)
            in_range(((int64_t)(b + tok0 + token) * B.H + hkv * g + head_l) * B.D + 8 * h + 16 * kk, 8, qo_elems,
                     "q row");
        const int rowoff = (4 * w + (lane >> 4)) & 15;
        const int chunk_sw = (lane & 15) ^ (((rowoff & 3) << 2) | ((rowoff >> 2) & 3));
        const int64_t lane_off = (int64_t)rowoff * row_elems + 8 * chunk_sw;
        expect(2 * lane_off < (int64_t)1 << 32, "32-bit lane offset", lane_off);
        const int vdim = 32 * (w & 3) + (lane >> 1);
        const int64_t v16_lane = (vdim * 32 + 16 * ((lane & 1) ^ ((vdim >> 3) & 1))) / 2;
        for (int32_t i = 0; i < ntiles; ++i) {
          const int32_t j = i + t0, slot = i % kNBuf;
          const bool full = j * kBK + kBK <= kend;
          for (int u = 0; u < 2; ++u) {
            const int piece = w + kWaves * u;                // 1 KB piece of the tile
            in_range(K_RING + slot * TILE + piece * 1024 + 16 * lane, 16, SMEM, "K ring slot");
            in_range(V_RING + slot * TILE + piece * 1024 + 16 * lane, 16, SMEM, "V ring slot");
            int64_t koff;
            if (full) {
              const int bi = (w >> 2) + (kWaves / 4) * u;
              koff = (int64_t)entry(4 * j + bi, "full-tile table entry") * blk_stride + lane_off;
            } else {
              const int32_t kg = std::min(j * kBK + 4 * piece + (lane >> 4), kend - 1);
              expect(kg >= 0 && kg < L, "partial-tile key", r, kg, L);
              koff = ((int64_t)entry(kg >> 4, "partial-tile table entry") * kBlk + (kg & 15)) * row_elems +
                     8 * chunk_sw;
            }
            in_range((int64_t)hkv * B.D + koff, 8, kv_elems, "K row (and V row of the bf16 redo kernel)");
            {
              // the fp16 kernel's V: staged block stage0 + 4j + piece / 4
              const int64_t sb = (int64_t)stage0 + 4 * j + (piece >> 2);
              expect(sb >= req[r].stage && sb < req[r + 1].stage, "staged V block of the request", r, sb);
              in_range(sb * blk_stride + (int64_t)hkv * B.D * kBlk + v16_lane, 8, n_stage * blk_stride,
                       "staged V row");
            }
          }
          if (B.f8 && w < 2) {                               // scales: wave 0 K, wave 1 V (redo)
            const int32_t kg = std::min(j * kBK + lane, kend - 1);
            const int32_t blk = entry(kg >> 4, "scale block");
            in_range((((int64_t)blk * 2 + w) * B.Hkv + hkv) * 16 + (kg & 15), 1, n_stage * 2 * B.Hkv * 16,
                     "staged scale");
            in_range(SC_RING + slot * SC_TILE + 256 * w + 4 * lane, 4, SMEM, "scale ring slot");
          }
        }
      }
    // output rows of the tile (staged through LDS, written 16 bytes per thread)
    for (int ci = 0; ci < kRows * (B.D / 8); ++ci) {
      const int mr = ci / (B.D / 8), chunk = ci % (B.D / 8);
      const int hl = mr / BQ, tk = mr - hl * BQ;
      if (tk >= Tn) continue;
      in_range(((int64_t)(b + tok0 + tk) * B.H + hkv * g + hl) * B.D + 8 * chunk, 8, qo_elems, "out row");
    }
  }
  for (int64_t i = 0; i < total; ++i) expect(seen[i] == 1, "workgroup map covers each (item, KV head) once", i, seen[i]);
}

}  // namespace

int main() {
  // the scalar base: addresses with bit 31 of the low word clear and set
  int sign_cases = 0;
  for (uint64_t hi : {0x7f00ull, 0x7fffull, 0x1ull, 0x0ull})
    for (uint64_t lo : {0x0ull, 0x1000ull, 0x7fffff00ull, 0x80000000ull, 0x80001000ull, 0xfffff000ull}) {
      const uint64_t a = (hi << 32) | lo;
      cur = "scalar base";
      expect(compose_base(a) == a, "scalar base composition", (int64_t)a);
      // the form without the casts: wrong exactly when bit 31 is set (high word all ones)
      const bool bad = compose_base_sign_extended(a) != a;
      expect(bad == ((lo >> 31) & 1) && (!bad || (compose_base_sign_extended(a) >> 32) == 0xffffffffull),
             "sign-extended composition differs exactly for bit 31", (int64_t)a);
      ++sign_cases;
    }

  char tag[16], name[256];
  int batches = 0;
  while (std::scanf("%15s", tag) == 1) {
    if (std::strcmp(tag, "batch") != 0) { std::printf("bad input\n"); return 2; }
    BatchIn B;
    long long N;
    if (std::scanf("%255s %d %d %d %d %d %d %d %d %d %lld", name, &B.R, &B.H, &B.Hkv, &B.D, &B.bs, &B.window, &B.f8,
                   &B.num_blocks, &B.stride, &N) != 11) { std::printf("bad header\n"); return 2; }
    B.name = name;
    B.N = N;
    B.qsl.resize(B.R + 1);
    B.lens.resize(B.R);
    B.table.resize((size_t)B.R * B.stride);
    for (auto& x : B.qsl) if (std::scanf("%d", &x) != 1) return 2;
    for (auto& x : B.lens) if (std::scanf("%d", &x) != 1) return 2;
    for (auto& x : B.table) if (std::scanf("%d", &x) != 1) return 2;
    check_batch(B);
    ++batches;
  }
  std::printf("checked %d batches, %lld accesses, %d scalar bases\n", batches, (long long)accesses, sign_cases);
  if (failures) std::printf("%lld failures\n", (long long)failures);
  return failures ? 1 : 0;
}
