/*
 * paged_attn.h: C ABI of the paged KV write and paged varlen attention library
 * (libpagedattn.so, HIP for gfx950).
 *
 * The operations are the attention backend of "Engine v2: one core for every request"
 * (inference.shantanugoel.com, chapter 31): write_kv and ReferenceBackend.forward in section
 * "Attention over the pool", with the batch described by BatchMeta in section "Flattened
 * ragged batches".
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, on the current HIP device; pointers are device
 *     pointers unless the name ends in _host.  The caller allocates and owns every buffer,
 *     including the workspace; the library never allocates device memory, never frees, and
 *     keeps no pointer after returning.  The one exception is the fixed scratch array of
 *     paged_attention_varlen_noalloc, a static device array each GPU holds from the
 *     library's load until the process ends.
 *   - dtype codes: PA_DTYPE_F32 (IEEE float32) and PA_DTYPE_BF16 (bfloat16).
 *   - Work is enqueued on `stream` and is asynchronous; nothing synchronises the device.
 *     The KV write of a step must be enqueued before the attention that reads it, on the
 *     same stream (a row's own key is in its visible range, and a block adopted from the
 *     prefix cache may be written in the same step).
 *   - Return value: PA_OK (0) on success, a negative PA_ERR_* code otherwise; then nothing
 *     was enqueued (except for PA_ERR_LAUNCH) and paged_attn_last_error() describes why.
 *     Validation reads only the host copies of the metadata.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_OK 0
#define PA_ERR_NULL (-1)        /* a required pointer is NULL */
#define PA_ERR_SHAPE (-2)       /* unsupported or inconsistent sizes (heads, head_dim, block_size) */
#define PA_ERR_DTYPE (-3)       /* unknown dtype code, or a combination not supported */
#define PA_ERR_METADATA (-4)    /* query_start_loc / seq_lens / table width inconsistent */
#define PA_ERR_WORKSPACE (-5)   /* workspace smaller than paged_attention_workspace_bytes() */
#define PA_ERR_LAUNCH (-6)      /* a kernel launch failed (hipGetLastError reported it) */
#define PA_ERR_RANGE (-7)       /* debug checks only: slot or block id out of range, duplicate slot */

#define PA_DTYPE_F32 0
#define PA_DTYPE_BF16 1
#define PA_DTYPE_FP8_E4M3 2     /* KV pools only: OCP E4M3 codes with a float32 scale per (slot, KV head) */

/*
 * paged_kv_write: write_kv of "Attention over the pool".
 *
 * For every new token i < num_tokens, its K row k[i] and V row v[i] (each num_kv_heads *
 * head_dim elements, layout [num_tokens, num_kv_heads, head_dim], dtype in_dtype) are
 * copied into row s of the pools k_cache / v_cache seen as [num_slots, num_kv_heads,
 * head_dim] (the pool [num_blocks + 1, block_size, num_kv_heads, head_dim], num_slots =
 * (num_blocks + 1) * block_size), where s = slot_mapping[i] (int64) if it is >= 0 and
 * s = num_slots - 1 (the scratch slot of the pool's extra last block) if it is negative:
 * padding rows carry slot -1.  Values are cast to cache_dtype with round-to-nearest-even
 * when the dtypes differ; otherwise the copy is bit-exact.  Every other pool element is
 * left unchanged.
 *
 * Preconditions (not checked unless debug checks are on): slot_mapping[i] < num_slots, and
 * non-negative slots are distinct (several padding rows may share the scratch slot, whose
 * content is then one of theirs).
 */
int paged_kv_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                   void* v_cache, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int64_t num_slots, int32_t in_dtype, int32_t cache_dtype, hipStream_t stream);

/*
 * paged_kv_write_fp8: write_kv into quantized pools.  ReferenceBackend.dequantize of
 * "Attention over the pool" reads a quantized pool as its codes' values times the scale kept
 * beside it for each (slot, KV head); this is the write that matches it.
 *
 * For every token i and KV head h, the row x = k[i, h, :] (and likewise v) becomes
 *     scale = max_d |x_d| / 448   (1 if the row is all zero; float32 division)
 *     code_d = the fp8 E4M3 value nearest to x_d / scale (float32 division, ties to even;
 *              E4M3 here is the OCP "FN" format: largest finite 448, no infinities)
 * stored at row s of k_cache / v_cache ([num_slots, num_kv_heads, head_dim] bytes) and at
 * k_scale / v_scale[s * num_kv_heads + h] ([num_slots, num_kv_heads] float32), with
 * s = slot_mapping[i], or num_slots - 1 if it is negative.  k, v: [num_tokens,
 * num_kv_heads, head_dim] in in_dtype (PA_DTYPE_F32 or PA_DTYPE_BF16); head_dim <= 256.
 * Preconditions and errors as for paged_kv_write; values must be finite.
 */
int paged_kv_write_fp8(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache, void* v_cache,
                       float* k_scale, float* v_scale, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                       int64_t num_slots, int32_t in_dtype, hipStream_t stream);

/*
 * paged_copy_blocks: the block copies of preemption and prefix sharing, swap_out /
 * swap_in of "Engine v2: one core for every request" (section "Preemption") and the
 * copy-on-write of a shared block (vllm-lite README, paged KV cache).
 *
 * For every pair i < num_pairs, block dst_block[i] of dst becomes a copy of block
 * src_block[i] of src, where a block is block_bytes contiguous bytes: for a pool tensor
 * [num_blocks + 1, block_size, num_kv_heads, head_dim] that is block_size * num_kv_heads *
 * head_dim * element size.  Call once per pool tensor (K, V).
 *   swap_out:      src = pool, dst = staging buffer, dst_block = 0 .. n-1
 *   swap_in:       src = staging buffer, src_block = 0 .. n-1, dst = pool
 *   copy-on-write: src = dst = pool
 *   src, dst          device memory, or host memory pinned with hipHostMalloc (reached over
 *                     PCIe); 16-byte aligned; src has num_src_blocks blocks, dst
 *                     num_dst_blocks.
 *   src_block, dst_block  [num_pairs] int64, device-accessible.
 *   block_bytes       a positive multiple of 16.
 * Pairs are copied in parallel.  Preconditions (checked only with debug checks on): ids in
 * range, dst_block entries distinct, and when src == dst no destination is another pair's
 * source.  Errors: PA_ERR_SHAPE (sizes, alignment), PA_ERR_NULL, PA_ERR_RANGE (debug),
 * PA_ERR_LAUNCH.  With timing on, the launch is counted as kind PA_KIND_KV_WRITE.
 */
int paged_copy_blocks(const void* src, void* dst, const int64_t* src_block, const int64_t* dst_block,
                      int64_t num_pairs, int64_t block_bytes, int64_t num_src_blocks, int64_t num_dst_blocks,
                      hipStream_t stream);

/*
 * paged_attention_workspace_bytes: device workspace paged_attention_varlen needs for this
 * batch (same arguments as there).  Depends only on the host metadata; returns 0 when the
 * arguments are invalid (the attention call would then report why).
 */
size_t paged_attention_workspace_bytes(int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       const int32_t* query_start_loc_host,
                                       const int32_t* seq_lens_host, int32_t dtype);

/*
 * paged_attention_varlen: ReferenceBackend.forward of "Attention over the pool", over one
 * flattened ragged batch (BatchMeta of "Flattened ragged batches").
 *
 *   q, out            [num_tokens, num_heads, head_dim], dtype.  out is fully written.
 *   k_cache, v_cache  [num_slots / block_size, block_size, num_kv_heads, head_dim], dtype;
 *                     read only.
 *   query_start_loc   [num_reqs + 1] int32: request r owns flattened rows
 *                     query_start_loc[r] .. query_start_loc[r+1]-1 (t_r rows).
 *   seq_lens          [num_reqs] int32: context length L_r including this step's tokens.
 *   block_table       [num_reqs, block_table_stride] int32: physical block ids of request r
 *                     in logical order; entries past ceil(L_r / block_size) are never read.
 *   *_host            host copies of query_start_loc and seq_lens (must equal the device
 *                     arrays); max_query_len / max_seq_len are their maxima (informational).
 *
 * Row i of request r is at position L_r - t_r + i and attends keys 0 .. that position:
 *     out[row, h, :] = sum_j softmax_j(scale * <q[row, h, :], K_j>) V_j,
 * where K_j / V_j is position j of the request read from slot
 * block_table[r][j / block_size] * block_size + j % block_size, head kv = h / (H / Hkv)
 * (query heads grouped contiguously onto KV heads).  Requests with seq_len 0 or no rows
 * (padding) produce zero rows.  Arithmetic is float32: bfloat16 inputs feed the matrix
 * cores with float32 accumulation.  In the PV product, probabilities carry at least 11
 * significant bits: fp16 probabilities against V converted to fp16 (prefill chunks, while
 * |v| <= 65504; the conversion is exact for |v| >= 2^-14 and moves smaller values by at most
 * 2^-25), else a bf16 pair (high part and the bf16 rounding of the remainder).
 * out is rounded to nearest-even.
 *
 * Supported: head_dim in {8, 16, 32, 48, 64, 96, 128, 256}; block_size >= 1 (the bf16
 * matrix-core paths need block_size 16, and head_dim 48, 64 or 128 for decode-like tiles
 * (64 or 128 on fp8 pools), 128 for prefill chunks; other shapes use the vector path, and a
 * prefill chunk at another head_dim runs as groups of decode-like tiles); num_heads %
 * num_kv_heads == 0; q,
 * out, caches and workspace 16-byte aligned.  workspace must hold
 * paged_attention_workspace_bytes().
 *
 * Preconditions not checked (unless debug checks are on): block ids in range; the K/V
 * of every visible position has been written.
 */
int paged_attention_varlen(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* query_start_loc, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t block_size, float scale, void* out,
                           int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_table_stride,
                           int64_t num_slots, const int32_t* query_start_loc_host,
                           const int32_t* seq_lens_host, int32_t max_query_len,
                           int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                           int32_t dtype, hipStream_t stream);

/*
 * Options of the _ex entry points; a NULL pointer means all defaults (the plain entry
 * points above).  reserved[] must be zero.
 *
 *   sliding_window     0: a row at position p attends keys 0 .. p.  w > 0: only the last w
 *                      of them, keys max(0, p - w + 1) .. p: the `window` argument of
 *                      ReferenceBackend.forward ("Attention over the pool": a key is
 *                      allowed iff k_pos > q_pos - window).  Blocks wholly before every
 *                      row's window are not read.  Negative values are rejected.
 *   graph_max_seq_len  0: the launches are sized from seq_lens_host.  M > 0: they are sized
 *                      for every seq_len = M instead, so one enqueued call (for instance
 *                      captured in a HIP graph for a batch padded to a fixed shape, pad_to
 *                      of "Flattened ragged batches") serves any device seq_lens <= M on
 *                      replay: the work lists are rebuilt on the device from the device
 *                      seq_lens, and workgroups beyond them exit.  seq_lens_host may then
 *                      be NULL; query_start_loc_host must still describe the (fixed) rows.
 *                      Every request must have rows x (num_heads / num_kv_heads) <= 64
 *                      (decode and verification batches); seq_lens above M are a
 *                      precondition violation (not checked).  No call made by the library
 *                      inside such a capture allocates or uses hipMemset.
 *   kv_cache_dtype     PA_DTYPE_FP8_E4M3: k_cache / v_cache hold fp8 codes (one byte per
 *                      element) written by paged_kv_write_fp8, and every key and value is
 *                      its code's value times its (slot, KV head) scale from k_scale /
 *                      v_scale (ReferenceBackend.dequantize).  Needs dtype PA_DTYPE_BF16,
 *                      block_size 16 and head_dim 64 or 128; every request then takes the
 *                      small-tile kernel (K codes and V codes convert exactly to bf16; each
 *                      score is multiplied by its key's K scale and each probability by its
 *                      key's V scale).  Else PA_ERR_DTYPE.
 */
typedef struct pa_attention_options {
  int32_t sliding_window;
  int32_t graph_max_seq_len;
  int32_t kv_cache_dtype;      /* 0: the pools hold `dtype`; PA_DTYPE_FP8_E4M3: fp8 codes, see below */
  int32_t reserved0;
  const float* k_scale;        /* fp8 pools: [num_slots, num_kv_heads] float32 scales of K and V */
  const float* v_scale;
  int64_t reserved[4];
} pa_attention_options;

/* paged_attention_workspace_bytes with options (the workspace depends on the window, the
 * sizing and the pool dtype; the scale pointers are not read here and may be NULL). */
size_t paged_attention_workspace_bytes_ex(int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          const int32_t* query_start_loc_host,
                                          const int32_t* seq_lens_host, int32_t dtype,
                                          const pa_attention_options* options);

/* paged_attention_varlen with options; the same contract otherwise.  The workspace must
 * hold paged_attention_workspace_bytes_ex() for the same options. */
int paged_attention_varlen_ex(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* query_start_loc, const int32_t* seq_lens,
                              const int32_t* block_table, int32_t block_size, float scale, void* out,
                              int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_table_stride,
                              int64_t num_slots, const int32_t* query_start_loc_host,
                              const int32_t* seq_lens_host, int32_t max_query_len,
                              int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                              int32_t dtype, hipStream_t stream, const pa_attention_options* options);

/*
 * paged_attention_varlen_noalloc: paged_attention_varlen_ex without a workspace argument, for
 * callers that cannot allocate device memory around the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments (minus workspace
 * and workspace_bytes), same contract, same kernels and the same results bit for bit.
 *
 * The workspace is a fixed scratch array of PA_NOALLOC_SCRATCH_BYTES bytes inside the
 * library, one per GPU, held from the library's load until the process ends; its device
 * address is looked up once per device on the first call there.  A batch whose workspace
 * (paged_attention_workspace_bytes_ex for the same options) exceeds that size is refused
 * with PA_ERR_WORKSPACE before anything is enqueued.  The call allocates no device memory
 * and calls no hipMalloc, hipFree or hipMemset.
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the last call's
 * contents: each call rewrites everything it reads (the planner writes the work lists and
 * clears the per-item flags before any kernel reads them), so nothing needs clearing
 * between calls.  Calls that may overlap on one GPU (different streams without ordering,
 * or different threads) race on the array: order them on one stream.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
int paged_attention_varlen_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* query_start_loc, const int32_t* seq_lens,
                                   const int32_t* block_table, int32_t block_size, float scale, void* out,
                                   int32_t num_reqs, int64_t num_tokens, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_table_stride,
                                   int64_t num_slots, const int32_t* query_start_loc_host,
                                   const int32_t* seq_lens_host, int32_t max_query_len,
                                   int32_t max_seq_len, int32_t dtype, hipStream_t stream,
                                   const pa_attention_options* options);

/*
 * paged_attn_set_debug_checks: when enable != 0, later calls on this thread also copy
 * slot_mapping / block_table to the host (synchronously) and check the preconditions
 * above, returning PA_ERR_RANGE on a violation.  Off by default.
 */
void paged_attn_set_debug_checks(int32_t enable);

/* Description of the last non-zero return on this thread ("" if none). */
const char* paged_attn_last_error(void);

/*
 * Selects the attention kernels (for tests and measurement): 0 = automatic (default),
 * 1 = vector-ALU tile kernel for every request, 2 = automatic, but with the work planner
 * launched for every batch (by default a batch of at most 64 requests that all run on the
 * matrix-core small tiles gets no planner launch: each workgroup of the small-tile kernel
 * and of the split merge derives its own work item from query_start_loc and seq_lens).
 * Applies to later calls on this thread.
 */
void paged_attn_set_path(int32_t path);

/*
 * Kernel timing (measurement only).  While enabled, every launch the library makes on this
 * thread is bracketed by a pair of HIP events recorded on the caller's stream.
 * paged_attn_timing_report waits for those events, writes per-kind sums of the elapsed
 * milliseconds (total_ms[kind]) and launch counts (count[kind]) for kinds
 * 0 = KV write, 1 = work planner, 2 = prefill tile kernel, 3 = small-tile kernel,
 * 4 = split merge, and forgets the recorded launches.  Returns the number of kinds written
 * (min(n_kinds, 5)), or a negative PA_ERR_* code.
 */
#define PA_KIND_KV_WRITE 0
#define PA_KIND_PLAN 1
#define PA_KIND_PREFILL 2
#define PA_KIND_SMALL 3
#define PA_KIND_MERGE 4
void paged_attn_set_timing(int32_t enable);
int paged_attn_timing_report(double* total_ms, int32_t* count, int32_t n_kinds);

/*
 * paged_hbm_read_probe (measurement only, not part of the attention path): reads `bytes`
 * bytes of device memory at `buf` once, with a grid of `grid` workgroups of 256 threads, so
 * that a caller can time the achievable HBM read rate that the decode kernels are measured
 * against beside the specification.
 *   buf    device memory, 16-byte aligned; bytes a positive multiple of 16.
 *   sink   one device uint32 the kernel may write (to keep its loads alive).
 *   grid   1 .. 65536.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_LAUNCH.
 */
int paged_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, hipStream_t stream);

/*
 * paged_mfma_probe (measurement only, not part of the attention path): `grid` workgroups of
 * 512 threads each run `iters` rounds of eight independent 32x32x16 bf16 matrix products with
 * no memory traffic, so that a caller can time the matrix-core rate the chip sustains under
 * its clock and power limits, beside the 2.5 PFLOP/s specification the prefill kernel is
 * measured against.
 *   iters  1 .. 2^20;  grid 1 .. 65536.
 *   data   0: operands are small integers (0 .. 7); 1: random bf16 values in [-2, 2), as
 *          attention's are (the sustained rate depends on the operands' bits).
 *   sink   one device uint32 the kernel may write (to keep its products alive).
 *   flops  optional host int64: receives the launch's floating-point operation count.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_LAUNCH.
 */
int paged_mfma_probe(int32_t iters, int32_t grid, int32_t data, uint32_t* sink, int64_t* flops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
