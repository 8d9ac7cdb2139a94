// C ABI of libpagedattn.so: argument validation (host copies only), the work plan, and the
// launches.  The operations and their arguments are those of write_kv / ReferenceBackend in
// "Engine v2: one core for every request" (sections "Flattened ragged batches" and
// "Attention over the pool"); see include/paged_attn.h for the contract.
#include "paged_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

namespace pa {
bool valu_head_dim_supported(int32_t D);
}

namespace {

thread_local std::string g_last_error;
thread_local int g_debug_checks = 0;
thread_local int g_path = 0;
thread_local int g_timing = 0;

// Kernel timing: event pairs recorded around each launch while timing is on.
struct TimedLaunch {
  hipEvent_t start, stop;
  int kind;
};
thread_local std::vector<TimedLaunch> g_events;   // created once, reused
thread_local size_t g_events_used = 0;
constexpr int kKinds = 5;

template <typename F>
hipError_t timed(int kind, hipStream_t s, F&& launch) {
  if (!g_timing) return launch();
  if (g_events_used == g_events.size()) {
    TimedLaunch t{};
    if (hipEventCreate(&t.start) != hipSuccess || hipEventCreate(&t.stop) != hipSuccess)
      return hipErrorOutOfMemory;
    g_events.push_back(t);
  }
  TimedLaunch& t = g_events[g_events_used++];
  t.kind = kind;
  hipError_t e = hipEventRecord(t.start, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  return hipEventRecord(t.stop, s);
}

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Options of the _ex entry points (NULL: defaults).  Reserved fields must be zero.
struct Options {
  int32_t window = 0, graph_max = 0;
  bool fp8 = false;
  const float* k_scale = nullptr;
  const float* v_scale = nullptr;
};
int read_options(const pa_attention_options* o, Options* out, bool need_scales) {
  *out = Options{};
  if (!o) return PA_OK;
  for (int64_t x : o->reserved)
    if (x != 0) return fail(PA_ERR_SHAPE, "pa_attention_options.reserved must be zero");
  if (o->reserved0 != 0) return fail(PA_ERR_SHAPE, "pa_attention_options.reserved0 must be zero");
  if (o->kv_cache_dtype != 0 && o->kv_cache_dtype != PA_DTYPE_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "kv_cache_dtype must be 0 or PA_DTYPE_FP8_E4M3");
  out->fp8 = o->kv_cache_dtype == PA_DTYPE_FP8_E4M3;
  out->k_scale = o->k_scale;
  out->v_scale = o->v_scale;
  if (need_scales && out->fp8 && (!o->k_scale || !o->v_scale))
    return fail(PA_ERR_NULL, "fp8 pools need k_scale and v_scale");
  if (o->sliding_window < 0) return fail(PA_ERR_SHAPE, "sliding_window must be >= 0");
  if (o->graph_max_seq_len < 0) return fail(PA_ERR_SHAPE, "graph_max_seq_len must be >= 0");
  out->window = o->sliding_window;
  out->graph_max = o->graph_max_seq_len;
  return PA_OK;
}

// Validates the host metadata and builds the plan.  Returns PA_OK or an error code.
int make_plan(int32_t R, int64_t N, int32_t H, int32_t Hkv, int32_t D, int32_t bs, int32_t stride,
              const int32_t* qsl, const int32_t* lens_host, int32_t dtype, int32_t window, int32_t graph_max,
              bool fp8, pa::Plan* out) {
  // with graph_max the launches are sized as if every seq_len were graph_max
  const bool sized_for_capacity = graph_max > 0;
  auto len_of = [&](int32_t r) { return sized_for_capacity ? graph_max : lens_host[r]; };
  if (R < 0 || N < 0) return fail(PA_ERR_METADATA, "num_reqs and num_tokens must be >= 0");
  if (N > INT32_MAX) return fail(PA_ERR_SHAPE, "num_tokens must fit in int32");
  if (H <= 0 || Hkv <= 0 || H % Hkv != 0)
    return fail(PA_ERR_SHAPE, "num_heads must be a positive multiple of num_kv_heads");
  if (!pa::valu_head_dim_supported(D))
    return fail(PA_ERR_SHAPE, "head_dim must be one of 8, 16, 32, 48, 64, 96, 128, 256");
  if (bs <= 0) return fail(PA_ERR_SHAPE, "block_size must be >= 1");
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return fail(PA_ERR_DTYPE, "unknown dtype code");
  if (R > 0 && (!qsl || (!lens_host && !sized_for_capacity)))
    return fail(PA_ERR_NULL, "host copies of query_start_loc / seq_lens are required");
  if (R == 0) {
    if (N != 0) return fail(PA_ERR_METADATA, "num_tokens > 0 with no requests");
  } else {
    if (qsl[0] != 0) return fail(PA_ERR_METADATA, "query_start_loc[0] must be 0");
    if ((int64_t)qsl[R] != N) return fail(PA_ERR_METADATA, "query_start_loc[num_reqs] must equal num_tokens");
  }
  if (window < 0) return fail(PA_ERR_SHAPE, "sliding_window must be >= 0");
  pa::Plan p{};
  p.R = R; p.H = H; p.Hkv = Hkv; p.g = H / Hkv; p.D = D; p.bs = bs;
  p.window = window;
  p.graph_max = graph_max;
  if (graph_max > 0)
    for (int32_t r = 0; r < R; ++r)
      if ((int64_t)(qsl[r + 1] - qsl[r]) * p.g > pa::kPrefillMinCols)
        return fail(PA_ERR_SHAPE, "graph_max_seq_len: request " + std::to_string(r) +
                                      " has more than 64 query columns (rows x group heads)");
  pa::set_tile_shape(p);
  const bool auto_path = g_path == 0 || g_path == 2;
  p.pf_tokens = (dtype == PA_DTYPE_BF16 && auto_path && pa::prefill_mfma_supported(D, bs, p.g))
                    ? pa::prefill_tile_tokens(p.g) : 0;
  p.f8 = fp8 ? 1 : 0;
  p.v16 = p.pf_tokens > 0 ? 1 : 0;
  p.decode_kind = (dtype == PA_DTYPE_BF16 && auto_path && pa::small_mfma_supported(D, bs, fp8)) ? 1 : 0;
  if (fp8 && p.decode_kind != 1)
    return fail(PA_ERR_DTYPE, "fp8 pools need dtype bf16, block_size 16, head_dim 64 or 128 and the automatic path");

  // pass 1: validate and measure the small-tile work to size the key splits
  double small_keys = 0;
  int32_t span_max = 0;
  for (int32_t r = 0; r < R; ++r) {
    const int32_t t = qsl[r + 1] - qsl[r];
    const int32_t L = len_of(r);
    if (t < 0) return fail(PA_ERR_METADATA, "query_start_loc must be non-decreasing (request " + std::to_string(r) + ")");
    if (L < 0) return fail(PA_ERR_METADATA, "seq_lens must be >= 0 (request " + std::to_string(r) + ")");
    if (L > 0 && t > L)
      return fail(PA_ERR_METADATA, "request " + std::to_string(r) + " has more query rows than its seq_len");
    if ((int64_t)(L + bs - 1) / bs > stride)
      return fail(PA_ERR_METADATA, "block_table_stride too small for seq_len of request " + std::to_string(r));
    if (t > 0 && L > 0 && !pa::use_prefill_path(p, t, L)) {
      small_keys += (double)pa::small_key_span(p, L) * ((t + p.tile_tokens - 1) / p.tile_tokens) * p.hsubs;
      span_max = std::max(span_max, pa::small_key_span(p, L));
    }
  }
  // Key splits: enough workgroups to fill 256 compute units several times over, but at
  // most 2048 keys per split so long contexts are cut into balanced pieces (1024 measured
  // slower: more partials to write and merge for the same reads).
  // A small batch would get many short splits that way, and merging their partials then
  // costs more than the attention (16 decodes of <= 2048 keys: 64-key splits, a 21 us merge):
  // splits also grow until no tile has more than 8.
  const double target = small_keys * Hkv / 2048.0;
  int32_t split = 64;
  while (split < 2048 && (double)split * 2 <= target) split *= 2;
  while (split < 2048 && (int64_t)split * 8 < span_max) split *= 2;
  // Whole waves of workgroups: when the small tiles' workgroups would not fill the GPU once
  // (about four run per CU at a time), a shorter split (any multiple of 64 keys, down to a
  // quarter, at most 16 per tile) can make them fill it: the split with the fewest
  // (waves of workgroups) x (keys per split) wins.
  {
    auto small_wgs = [&](int32_t s) {
      pa::Plan q = p;
      q.split_keys = s;
      int64_t n = 0;
      for (int32_t r = 0; r < R; ++r) {
        int32_t a, b, c, d;
        const int32_t t = qsl[r + 1] - qsl[r];
        if (q.decode_kind == 1) {
          pa::small_groups(q, t, len_of(r), &a, &b);
          n += a + b;
        } else {
          pa::request_counts(q, t, len_of(r), &a, &b, &c, &d);
          n += a;
        }
      }
      return n * Hkv;
    };
    constexpr int64_t kConcurrentWGs = 4 * 256;
    const int64_t n0 = small_wgs(split);
    if (n0 > 0 && n0 < kConcurrentWGs) {
      int64_t best_cost = ((n0 + kConcurrentWGs - 1) / kConcurrentWGs) * (int64_t)split;
      int32_t best = split;
      for (int32_t s = split - 64; s >= std::max(64, split / 4); s -= 64) {
        if ((span_max + s - 1) / s > 16) break;
        const int64_t n = small_wgs(s);
        const int64_t cost = ((n + kConcurrentWGs - 1) / kConcurrentWGs) * (int64_t)s;
        if (cost < best_cost) {
          best_cost = cost;
          best = s;
        }
      }
      split = best;
    }
  }
  p.split_keys = split;

  int64_t ns = 0, nm = 0, np = 0, ng = 0, n1 = 0, n3 = 0;
  for (int32_t r = 0; r < R; ++r) {
    int32_t a, b, c, d;
    pa::request_counts(p, qsl[r + 1] - qsl[r], len_of(r), &a, &b, &c, &d);
    ns += a; nm += b; np += c;
    pa::small_groups(p, qsl[r + 1] - qsl[r], len_of(r), &a, &b);
    n1 += a; n3 += b;
    ng += pa::staged_blocks(p, qsl[r + 1] - qsl[r], len_of(r));
  }
  if (ns > INT32_MAX / 2 || nm > INT32_MAX / 2 || np > INT32_MAX / 2 || ng > INT32_MAX / 2)
    return fail(PA_ERR_SHAPE, "batch too large for the work lists");
  // the prefill kernel addresses staged scales with 32-bit offsets per workgroup
  if (p.f8 && ng * 2 * Hkv * 16 * 4 > (int64_t)INT32_MAX) return fail(PA_ERR_SHAPE, "fp8 prefill: too many staged blocks");
  p.n_small = ns; p.n_merge = nm; p.n_pf = np; p.n_stage = ng;
  p.n_g1 = n1; p.n_g3 = n3;
  // a small batch of decode-like requests needs no planner launch: the small kernels and the
  // merge find their own items (one request per lane of a wave)
  p.inline_items = (p.decode_kind == 1 && R <= pa::kInlineMaxReqs && np == 0 && g_path != 2) ? 1 : 0;

  size_t off = 0;
  p.off_req = off;   off = align_up(off + sizeof(pa::ReqOffsets) * (size_t)(R + 1), 256);
  p.off_small = off; off = align_up(off + sizeof(pa::SmallItem) * (size_t)(p.decode_kind == 1 ? 0 : ns), 256);
  p.off_merge = off; off = align_up(off + sizeof(pa::MergeItem) * (size_t)nm, 256);
  p.off_pf = off;    off = align_up(off + sizeof(pa::PfItem) * (size_t)np, 256);
  p.off_pf_wide = off; off = align_up(off + sizeof(int32_t) * (size_t)np * Hkv, 256);
  const size_t nparts = nm > 0 ? (size_t)ns * Hkv * pa::kCols : 0;
  p.off_pm = off;    off = align_up(off + 4 * nparts, 256);
  p.off_pl = off;    off = align_up(off + 4 * nparts, 256);
  p.off_pacc = off;  off = align_up(off + 4 * nparts * (size_t)D, 256);
  const bool mfma_lists = p.decode_kind == 1;
  p.off_g1 = off;    off = align_up(off + sizeof(pa::SmallItem) * (size_t)(mfma_lists ? n1 : 0), 256);
  p.off_g3 = off;    off = align_up(off + sizeof(pa::SmallItem) * (size_t)(mfma_lists ? n3 : 0), 256);
  // fp8 pools: staged bf16 codes (K, and V for the bf16 redo kernel) and scales of the
  // prefill requests
  const size_t ng8 = p.f8 ? (size_t)ng : 0;
  p.off_f8_k = off;   off = align_up(off + 2 * ng8 * bs * Hkv * D, 256);
  p.off_f8_v = off;   off = align_up(off + 2 * ng8 * bs * Hkv * D, 256);
  p.off_f8_s = off;   off = align_up(off + 4 * ng8 * 2 * Hkv * bs, 256);
  // the fp16 copy of the prefill requests' V blocks (fp8 pools: codes times scales)
  p.off_v16 = off;    off = align_up(off + 2 * (p.v16 ? (size_t)ng : 0) * bs * Hkv * D, 256);
  p.total_bytes = off;
  *out = p;
  return PA_OK;
}

}  // namespace

// Scratch of paged_attention_varlen_noalloc: its workspace, for callers that cannot
// allocate.  Every GPU the library runs on holds its own copy for the life of the process.
// Host code never passes this name to a kernel (on the host it is only a stand-in for the
// device symbol): the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on its first use there.
int scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_LAUNCH, "device index out of range for the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PA_ERR_LAUNCH, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

// The attention call behind both entry points: validation, the plan, the launches.
// scratch_call: the workspace is the library's own scratch array on the current device, of
// workspace_bytes; its address is fetched once the batch is known to fit.
int attention_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* query_start_loc,
                   const int32_t* seq_lens, const int32_t* block_table, int32_t block_size, float scale, void* out,
                   int32_t num_reqs, int64_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_table_stride, int64_t num_slots, const int32_t* query_start_loc_host,
                   const int32_t* seq_lens_host, void* workspace, size_t workspace_bytes, int32_t dtype,
                   hipStream_t stream, const pa_attention_options* options, bool scratch_call) {
  if (block_table_stride < 0) return fail(PA_ERR_METADATA, "block_table_stride must be >= 0");
  Options opt;
  int rc = read_options(options, &opt, true);
  if (rc != PA_OK) return rc;
  const int32_t graph_max = opt.graph_max;
  pa::Plan p;
  rc = make_plan(num_reqs, num_tokens, num_heads, num_kv_heads, head_dim, block_size, block_table_stride,
                 query_start_loc_host, seq_lens_host, dtype, opt.window, opt.graph_max, opt.fp8, &p);
  if (rc != PA_OK) return rc;
  if (num_reqs == 0) return PA_OK;
  if (!query_start_loc || !seq_lens || !block_table || (!workspace && !scratch_call))
    return fail(PA_ERR_NULL, "null pointer argument");
  if (num_tokens > 0 && (!q || !out || !k_cache || !v_cache)) return fail(PA_ERR_NULL, "null pointer argument");
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace))
    return fail(PA_ERR_SHAPE, "q, out, caches and workspace must be 16-byte aligned");
  if (num_slots < block_size || num_slots % block_size != 0)
    return fail(PA_ERR_SHAPE, "num_slots must be a positive multiple of block_size");
  if (workspace_bytes < p.total_bytes)
    return fail(PA_ERR_WORKSPACE, scratch_call ? "batch needs " + std::to_string(p.total_bytes) +
                                                     " bytes of scratch, more than the no-alloc maximum of " +
                                                     std::to_string(workspace_bytes) + " bytes"
                                               : "workspace too small: need " + std::to_string(p.total_bytes) + " bytes");
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale must be finite");
  if (scratch_call) {
    rc = scratch_of_current_device(&workspace);
    if (rc != PA_OK) return rc;
  }
  if (g_debug_checks && graph_max == 0) {   // (sized-for-capacity calls may be captured: no sync)
    std::vector<int32_t> tb((size_t)num_reqs * block_table_stride);
    if (!tb.empty() && hipMemcpy(tb.data(), block_table, sizeof(int32_t) * tb.size(), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_LAUNCH, "debug check: copy of block_table failed");
    const int64_t nb = num_slots / block_size;
    for (int32_t r = 0; r < num_reqs; ++r) {
      const int32_t used = (seq_lens_host[r] + block_size - 1) / block_size;
      for (int32_t j = 0; j < used; ++j) {
        const int32_t blk = tb[(size_t)r * block_table_stride + j];
        if (blk < 0 || blk >= nb)
          return fail(PA_ERR_RANGE, "block_table[" + std::to_string(r) + "][" + std::to_string(j) + "] out of range");
      }
    }
  }
  pa::AttnArgs a{};
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.qsl = query_start_loc; a.seq_lens = seq_lens; a.block_table = block_table; a.out = out;
  a.bs = block_size; a.stride = block_table_stride; a.H = num_heads; a.Hkv = num_kv_heads;
  a.g = p.g; a.D = head_dim; a.tile_tokens = p.tile_tokens; a.tile_heads = p.tile_heads;
  a.split_keys = p.split_keys;
  a.window = p.window;
  a.totals = (const int32_t*)((const char*)workspace + p.off_req + sizeof(pa::ReqOffsets) * (size_t)num_reqs);
  a.k_scale = opt.fp8 ? opt.k_scale : nullptr;
  a.v_scale = opt.fp8 ? opt.v_scale : nullptr;
  a.scale_log2e = scale * 1.4426950408889634f;

  hipError_t e = hipSuccess;
  if (!p.inline_items)
    e = timed(PA_KIND_PLAN, stream, [&] { return pa::launch_plan(p, query_start_loc, seq_lens, workspace, stream); });
  if (e == hipSuccess && p.n_pf > 0)
    e = timed(PA_KIND_PREFILL, stream, [&] {
      return p.f8 ? pa::launch_stage_fp8(p, a, std::max(std::fabs(a.scale_log2e), 1e-30f), workspace, stream)
                  : pa::launch_prefill_mfma(p, a, workspace, stream);
    });
  if (e == hipSuccess && p.n_small > 0)
    e = timed(PA_KIND_SMALL, stream, [&] {
      return p.decode_kind == 1 ? pa::launch_small_mfma(p, a, workspace, stream)
                                : pa::launch_small_valu(p, a, workspace, dtype, stream);
    });
  if (e == hipSuccess && p.n_merge > 0)
    e = timed(PA_KIND_MERGE, stream, [&] { return pa::launch_merge(p, a, workspace, dtype, stream); });
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, std::string("attention launch: ") + hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" {

const char* paged_attn_last_error(void) { return g_last_error.c_str(); }

void paged_attn_set_debug_checks(int32_t enable) { g_debug_checks = enable != 0; }

void paged_attn_set_path(int32_t path) { g_path = path; }

void paged_attn_set_timing(int32_t enable) {
  g_timing = enable != 0;
  g_events_used = 0;
}

int paged_attn_timing_report(double* total_ms, int32_t* count, int32_t n_kinds) {
  g_last_error.clear();
  if (!total_ms || !count) return fail(PA_ERR_NULL, "null pointer argument");
  const int k = std::min<int>(std::max<int>(n_kinds, 0), kKinds);
  for (int i = 0; i < k; ++i) { total_ms[i] = 0.0; count[i] = 0; }
  for (size_t i = 0; i < g_events_used; ++i) {
    TimedLaunch& t = g_events[i];
    if (hipEventSynchronize(t.stop) != hipSuccess) return fail(PA_ERR_LAUNCH, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) return fail(PA_ERR_LAUNCH, "event timing failed");
    if (t.kind < k) {
      total_ms[t.kind] += ms;
      count[t.kind] += 1;
    }
  }
  g_events_used = 0;
  return k;
}

int paged_kv_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                   void* v_cache, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int64_t num_slots, int32_t in_dtype, int32_t cache_dtype, hipStream_t stream) {
  g_last_error.clear();
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens must be >= 0");
  if (num_kv_heads <= 0 || head_dim <= 0) return fail(PA_ERR_SHAPE, "num_kv_heads and head_dim must be > 0");
  if (num_slots < 1) return fail(PA_ERR_SHAPE, "num_slots must be >= 1 (the scratch slot)");
  if ((in_dtype != PA_DTYPE_F32 && in_dtype != PA_DTYPE_BF16) ||
      (cache_dtype != PA_DTYPE_F32 && cache_dtype != PA_DTYPE_BF16))
    return fail(PA_ERR_DTYPE, "unknown dtype code");
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(PA_ERR_NULL, "null pointer argument");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (row > INT32_MAX) return fail(PA_ERR_SHAPE, "num_kv_heads * head_dim too large");
  if (g_debug_checks) {
    std::vector<int64_t> s((size_t)num_tokens);
    if (hipMemcpy(s.data(), slot_mapping, sizeof(int64_t) * s.size(), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_LAUNCH, "debug check: copy of slot_mapping failed");
    std::unordered_set<int64_t> seen;
    for (size_t i = 0; i < s.size(); ++i) {
      if (s[i] >= num_slots) return fail(PA_ERR_RANGE, "slot_mapping[" + std::to_string(i) + "] out of range");
      if (s[i] >= 0 && !seen.insert(s[i]).second)
        return fail(PA_ERR_RANGE, "slot_mapping[" + std::to_string(i) + "] repeats a slot");
    }
  }
  const hipError_t e = timed(PA_KIND_KV_WRITE, stream, [&] {
    return pa::launch_kv_write(k, v, slot_mapping, k_cache, v_cache, num_tokens, (int32_t)row, num_slots,
                               in_dtype, cache_dtype, stream);
  });
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, std::string("kv write launch: ") + hipGetErrorString(e));
  return PA_OK;
}

int paged_kv_write_fp8(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache, void* v_cache,
                       float* k_scale, float* v_scale, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                       int64_t num_slots, int32_t in_dtype, hipStream_t stream) {
  g_last_error.clear();
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens must be >= 0");
  if (num_kv_heads <= 0 || head_dim <= 0 || head_dim > 256)
    return fail(PA_ERR_SHAPE, "num_kv_heads must be > 0 and head_dim in 1 .. 256");
  if (num_slots < 1) return fail(PA_ERR_SHAPE, "num_slots must be >= 1 (the scratch slot)");
  if (in_dtype != PA_DTYPE_F32 && in_dtype != PA_DTYPE_BF16) return fail(PA_ERR_DTYPE, "in_dtype must be f32 or bf16");
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
    return fail(PA_ERR_NULL, "null pointer argument");
  if (g_debug_checks) {
    std::vector<int64_t> s((size_t)num_tokens);
    if (hipMemcpy(s.data(), slot_mapping, sizeof(int64_t) * s.size(), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_LAUNCH, "debug check: copy of slot_mapping failed");
    std::unordered_set<int64_t> seen;
    for (size_t i = 0; i < s.size(); ++i) {
      if (s[i] >= num_slots) return fail(PA_ERR_RANGE, "slot_mapping[" + std::to_string(i) + "] out of range");
      if (s[i] >= 0 && !seen.insert(s[i]).second)
        return fail(PA_ERR_RANGE, "slot_mapping[" + std::to_string(i) + "] repeats a slot");
    }
  }
  const hipError_t e = timed(PA_KIND_KV_WRITE, stream, [&] {
    return pa::launch_kv_write_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, num_tokens, num_kv_heads,
                                   head_dim, num_slots, in_dtype, stream);
  });
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, std::string("kv write launch: ") + hipGetErrorString(e));
  return PA_OK;
}

int paged_copy_blocks(const void* src, void* dst, const int64_t* src_block, const int64_t* dst_block,
                      int64_t num_pairs, int64_t block_bytes, int64_t num_src_blocks, int64_t num_dst_blocks,
                      hipStream_t stream) {
  g_last_error.clear();
  if (num_pairs < 0) return fail(PA_ERR_SHAPE, "num_pairs must be >= 0");
  if (block_bytes <= 0 || block_bytes % 16 != 0) return fail(PA_ERR_SHAPE, "block_bytes must be a positive multiple of 16");
  if (num_pairs == 0) return PA_OK;
  if (!src || !dst || !src_block || !dst_block) return fail(PA_ERR_NULL, "null pointer argument");
  if (!aligned16(src) || !aligned16(dst)) return fail(PA_ERR_SHAPE, "src and dst must be 16-byte aligned");
  if (g_debug_checks) {
    std::vector<int64_t> sb((size_t)num_pairs), db((size_t)num_pairs);
    if (hipMemcpy(sb.data(), src_block, 8 * sb.size(), hipMemcpyDefault) != hipSuccess ||
        hipMemcpy(db.data(), dst_block, 8 * db.size(), hipMemcpyDefault) != hipSuccess)
      return fail(PA_ERR_LAUNCH, "debug check: copy of the block ids failed");
    std::unordered_set<int64_t> dsts;
    for (size_t i = 0; i < sb.size(); ++i) {
      if (sb[i] < 0 || sb[i] >= num_src_blocks) return fail(PA_ERR_RANGE, "src_block[" + std::to_string(i) + "] out of range");
      if (db[i] < 0 || db[i] >= num_dst_blocks) return fail(PA_ERR_RANGE, "dst_block[" + std::to_string(i) + "] out of range");
      if (!dsts.insert(db[i]).second) return fail(PA_ERR_RANGE, "dst_block[" + std::to_string(i) + "] repeats a block");
    }
    if (src == dst)
      for (size_t i = 0; i < sb.size(); ++i)
        if (dsts.count(sb[i]) && db[i] != sb[i])
          return fail(PA_ERR_RANGE, "src_block[" + std::to_string(i) + "] is also a destination");
  }
  const hipError_t e = timed(PA_KIND_KV_WRITE, stream, [&] {
    return pa::launch_copy_blocks(src, dst, src_block, dst_block, num_pairs, block_bytes, stream);
  });
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, std::string("block copy launch: ") + hipGetErrorString(e));
  return PA_OK;
}

size_t paged_attention_workspace_bytes(int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                       int32_t dtype) {
  return paged_attention_workspace_bytes_ex(num_reqs, num_tokens, num_heads, num_kv_heads, head_dim, block_size,
                                            query_start_loc_host, seq_lens_host, dtype, nullptr);
}

size_t paged_attention_workspace_bytes_ex(int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                          int32_t dtype, const pa_attention_options* options) {
  pa::Plan p;
  const std::string keep = g_last_error;
  Options opt;
  int rc = read_options(options, &opt, false);
  if (rc == PA_OK)
    rc = make_plan(num_reqs, num_tokens, num_heads, num_kv_heads, head_dim, block_size, INT32_MAX,
                   query_start_loc_host, seq_lens_host, dtype, opt.window, opt.graph_max, opt.fp8, &p);
  g_last_error = keep;
  return rc == PA_OK ? p.total_bytes : 0;
}

int paged_attention_varlen(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* query_start_loc, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t block_size, float scale, void* out,
                           int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_table_stride,
                           int64_t num_slots, const int32_t* query_start_loc_host,
                           const int32_t* seq_lens_host, int32_t max_query_len,
                           int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                           int32_t dtype, hipStream_t stream) {
  return paged_attention_varlen_ex(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, block_size, scale,
                                   out, num_reqs, num_tokens, num_heads, num_kv_heads, head_dim, block_table_stride,
                                   num_slots, query_start_loc_host, seq_lens_host, max_query_len, max_seq_len,
                                   workspace, workspace_bytes, dtype, stream, nullptr);
}

int paged_attention_varlen_ex(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* query_start_loc, const int32_t* seq_lens,
                              const int32_t* block_table, int32_t block_size, float scale, void* out,
                              int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_table_stride,
                              int64_t num_slots, const int32_t* query_start_loc_host,
                              const int32_t* seq_lens_host, int32_t max_query_len,
                              int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                              int32_t dtype, hipStream_t stream, const pa_attention_options* options) {
  g_last_error.clear();
  (void)max_query_len;
  (void)max_seq_len;
  return attention_impl(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, block_size, scale, out, num_reqs,
                        num_tokens, num_heads, num_kv_heads, head_dim, block_table_stride, num_slots,
                        query_start_loc_host, seq_lens_host, workspace, workspace_bytes, dtype, stream, options, false);
}

int paged_attention_varlen_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* query_start_loc, const int32_t* seq_lens,
                                   const int32_t* block_table, int32_t block_size, float scale, void* out,
                                   int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_table_stride,
                                   int64_t num_slots, const int32_t* query_start_loc_host,
                                   const int32_t* seq_lens_host, int32_t max_query_len,
                                   int32_t max_seq_len, int32_t dtype, hipStream_t stream,
                                   const pa_attention_options* options) {
  g_last_error.clear();
  (void)max_query_len;
  (void)max_seq_len;
  return attention_impl(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, block_size, scale, out, num_reqs,
                        num_tokens, num_heads, num_kv_heads, head_dim, block_table_stride, num_slots,
                        query_start_loc_host, seq_lens_host, nullptr, (size_t)PA_NOALLOC_SCRATCH_BYTES, dtype,
                        stream, options, true);
}

int paged_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, hipStream_t stream) {
  g_last_error.clear();
  if (!buf || !sink) return fail(PA_ERR_NULL, "null pointer argument");
  if (bytes <= 0 || bytes % 16 != 0 || !aligned16(buf)) return fail(PA_ERR_SHAPE, "bytes must be a positive multiple of 16, buf 16-byte aligned");
  if (grid < 1 || grid > 65536) return fail(PA_ERR_SHAPE, "grid must be in 1 .. 65536");
  const hipError_t e = pa::launch_read_probe(buf, bytes, sink, grid, stream);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, std::string("read probe launch: ") + hipGetErrorString(e));
  return PA_OK;
}

int paged_mfma_probe(int32_t iters, int32_t grid, int32_t data, uint32_t* sink, int64_t* flops, hipStream_t stream) {
  g_last_error.clear();
  if (!sink) return fail(PA_ERR_NULL, "null pointer argument");
  if (iters < 1 || iters > (1 << 20)) return fail(PA_ERR_SHAPE, "iters must be in 1 .. 2^20");
  if (grid < 1 || grid > 65536) return fail(PA_ERR_SHAPE, "grid must be in 1 .. 65536");
  if (data != 0 && data != 1) return fail(PA_ERR_SHAPE, "data must be 0 (small integers) or 1 (random values)");
  if (flops) *flops = pa::mfma_probe_flops(iters, grid);
  const hipError_t e = pa::launch_mfma_probe(iters, data, sink, grid, stream);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, std::string("matrix probe launch: ") + hipGetErrorString(e));
  return PA_OK;
}

}  // extern "C"
