/*
 * CPU oracle for the paged KV write and for paged varlen attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file:
 * only the test suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Written from "Engine v2: one core for every request" (inference.shantanugoel.com,
 * chapter 31), sections "Flattened ragged batches" (BatchMeta, the slot formula) and
 * "Attention over the pool" (write_kv, ReferenceBackend.forward), with the gather step
 * described in the vllm-lite README (section on the paged KV cache: slots are
 * block_id * block_size + offset, read in logical order) and its grouped-query note
 * (query heads fold contiguously onto KV heads, kv = h / (H / Hkv)).
 *
 * Everything is plain loops (float64 arithmetic), in the order the pages describe:
 *   write:      for each new token i (increasing), slot = slot_mapping[i], a negative slot
 *               is redirected to the pool's last slot, then the token's Hkv*D row is copied
 *               (cast to the cache dtype) into that slot.
 *   attention:  for each request r, gather its first seq_len context rows through its block
 *               table (logical order), then for each of its t query rows i (position
 *               seq_len - t + i) and each query head h: scores over keys 0..position, max,
 *               exponentials, sum, weighted sum of V, divide.  Two passes, no tiling.
 *               With a sliding window of w > 0 tokens, only the last w of those keys take
 *               part (keys position-w+1 .. position), as ReferenceBackend.forward's
 *               `allowed = k_pos > q_pos - window` states in "Attention over the pool".
 *               Requests with seq_len == 0 or no query rows leave their rows at zero.
 *
 * dtype codes: 0 = float32, 1 = bfloat16 (stored as the upper 16 bits of a float32),
 * 2 = fp8 E4M3 pools with a float32 scale per (slot, KV head).  Rounding to an output dtype
 * is round-to-nearest-even, done once from float64.
 *
 * Quantized pools ("Attention over the pool": ReferenceBackend.dequantize multiplies each
 * gathered K or V row by its scale, which quantized pools keep beside K and V).  The pages
 * fix the read side only; the write side taken here is the plainest one that read supports:
 * per (token, KV head) row, scale = max|x| / 448 (the largest fp8 E4M3 value; 1 for an
 * all-zero row) and the stored codes are x / scale rounded to the nearest fp8 E4M3 value.
 * Those two divisions and the max are done in float32, the precision the kernel computes
 * them in, since they decide the stored codes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_FP8 2

/* Value of element idx of an array of the given dtype, exactly, as a double. */
static double load_elem(const void* base, int64_t idx, int dtype) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 (ties to even), returned as its 16-bit pattern.
 * Done directly from the double (no intermediate float rounding): the value is scaled so
 * that one unit is the bfloat16 spacing at its binade (8 significant bits; spacing never
 * below the subnormal step 2^-133), rounded with rint (ties-to-even in the default mode),
 * and scaled back. */
static uint16_t round_to_bf16(double x) {
    if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
    if (isinf(x)) return (uint16_t)(x > 0 ? 0x7F80u : 0xFF80u);
    if (x == 0.0) return (uint16_t)(signbit(x) ? 0x8000u : 0x0000u);
    int e;
    (void)frexp(x, &e);                 /* x = m * 2^e, 0.5 <= |m| < 1 */
    int q = e - 8;                      /* spacing of 8-significant-bit numbers in this binade */
    if (q < -133) q = -133;
    double r = ldexp(rint(ldexp(x, -q)), q);
    const double max_bf16 = 3.38953138925153547590470800371487866880e38; /* (2 - 2^-7) * 2^127 */
    float f;
    if (fabs(r) > max_bf16) f = (r > 0) ? INFINITY : -INFINITY;
    else f = (float)r;                  /* exact: r has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(bits >> 16);
}

static void store_elem(void* base, int64_t idx, int dtype, double x) {
    if (dtype == ORACLE_F32) ((float*)base)[idx] = (float)x; /* C cast: round to nearest even */
    else ((uint16_t*)base)[idx] = round_to_bf16(x);
}

/* bfloat16 pattern of a double, exposed so the rounding can be pinned on its own. */
uint16_t oracle_round_to_bf16(double x) { return round_to_bf16(x); }

/*
 * fp8 E4M3, the OCP "FN" variant: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * field 0 holds the subnormals m * 2^-9; there are no infinities and S.1111.111 is NaN, so
 * the largest finite magnitude is 1.75 * 2^8 = 448.
 */
double oracle_fp8_e4m3_decode(uint8_t b) {
    const int e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (b & 0x80) ? -v : v;
}

/* Nearest fp8 E4M3 value to y (ties to even); magnitudes beyond 448 saturate to 448 and NaN
 * becomes the NaN code.  The value is rounded on the spacing of its binade (2^(E-3) for
 * |y| in [2^E, 2^(E+1)), E >= -6; 2^-9 below 2^-6), then encoded. */
uint8_t oracle_fp8_e4m3_encode(float y) {
    if (isnan(y)) return 0x7F;
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    const double a = fabs((double)y);
    if (a == 0.0) return sign;
    int E;
    (void)frexp(a, &E);                 /* a = f * 2^E, 0.5 <= f < 1 */
    E -= 1;                             /* a in [2^E, 2^(E+1)) */
    const int q = (E < -6 ? -6 : E) - 3;
    const double r = ldexp(rint(ldexp(a, -q)), q);
    if (r >= 448.0) return sign | 0x7E;
    if (r == 0.0) return sign;
    int Er;
    (void)frexp(r, &Er);
    Er -= 1;
    if (Er < -6) return sign | (uint8_t)ldexp(r, 9);                     /* subnormal: r = m * 2^-9 */
    return sign | (uint8_t)((Er + 7) << 3) | (uint8_t)(ldexp(r, -Er) * 8.0 - 8.0);
}

/* One (token, KV head) row of D values to fp8 codes and its scale (see the header). */
static void quantize_row(const void* x, int64_t base, int32_t d, int32_t in_dtype, uint8_t* codes, float* scale) {
    float amax = 0.0f;
    for (int32_t i = 0; i < d; ++i) {
        const float f = fabsf((float)load_elem(x, base + i, in_dtype));
        if (f > amax) amax = f;
    }
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (int32_t i = 0; i < d; ++i) codes[i] = oracle_fp8_e4m3_encode((float)load_elem(x, base + i, in_dtype) / s);
    *scale = s;
}

/*
 * write_kv into quantized pools: token i's K and V rows ([N, Hkv, D], in_dtype) become fp8
 * codes in row s of k_cache / v_cache ([num_slots, Hkv, D] bytes) and their scales in
 * k_scale / v_scale ([num_slots, Hkv] float32), s = slot_mapping[i] or the last slot if it is
 * negative.
 */
int oracle_kv_write_fp8(const void* k, const void* v, const int64_t* slot_mapping, uint8_t* k_cache,
                        uint8_t* v_cache, float* k_scale, float* v_scale, int64_t num_tokens,
                        int32_t num_kv_heads, int32_t head_dim, int64_t num_slots, int32_t in_dtype) {
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    for (int64_t i = 0; i < num_tokens; ++i)
        if (slot_mapping[i] >= num_slots) return -1;
    /* Rows with a slot of their own are independent (distinct slots are a precondition of
     * write_kv) and are quantized in parallel; every padding row targets the last slot, where
     * the last padding row in order is the one that stays, so only that one is written. */
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < num_tokens; ++i) {
        if (slot_mapping[i] < 0) continue;
        const int64_t s = slot_mapping[i];
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            const int64_t src = i * row + (int64_t)h * head_dim, dst = s * row + (int64_t)h * head_dim;
            quantize_row(k, src, head_dim, in_dtype, k_cache + dst, k_scale + s * num_kv_heads + h);
            quantize_row(v, src, head_dim, in_dtype, v_cache + dst, v_scale + s * num_kv_heads + h);
        }
    }
    for (int64_t i = num_tokens - 1; i >= 0; --i) {
        if (slot_mapping[i] >= 0) continue;
        const int64_t s = num_slots - 1;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            const int64_t src = i * row + (int64_t)h * head_dim, dst = s * row + (int64_t)h * head_dim;
            quantize_row(k, src, head_dim, in_dtype, k_cache + dst, k_scale + s * num_kv_heads + h);
            quantize_row(v, src, head_dim, in_dtype, v_cache + dst, v_scale + s * num_kv_heads + h);
        }
        break;
    }
    return 0;
}

/*
 * Block copies of "Engine v2: one core for every request": swap_out gathers a preempted
 * request's blocks of each pool tensor into a host copy, swap_in writes a saved copy into
 * newly allocated blocks (index_copy_ over the pool's blocks), and copy-on-write copies a
 * shared block into a private one before the step (vllm-lite README, paged KV cache).  One
 * rule covers all three: for each pair i, in increasing i, the block_bytes bytes of block
 * src_block[i] of src become block dst_block[i] of dst.  Returns -1 on a negative id.
 */
int oracle_copy_blocks(const void* src, void* dst, const int64_t* src_block, const int64_t* dst_block,
                       int64_t num_pairs, int64_t block_bytes) {
    for (int64_t i = 0; i < num_pairs; ++i)
        if (src_block[i] < 0 || dst_block[i] < 0) return -1;
    for (int64_t i = 0; i < num_pairs; ++i) {
        const unsigned char* from = (const unsigned char*)src + src_block[i] * block_bytes;
        unsigned char* to = (unsigned char*)dst + dst_block[i] * block_bytes;
        for (int64_t b = 0; b < block_bytes; ++b) to[b] = from[b];
    }
    return 0;
}

/*
 * write_kv ("Attention over the pool"): k, v are [N, Hkv, D] in in_dtype; the caches are
 * [num_slots, Hkv, D] in cache_dtype (the pool [blocks, block_size, Hkv, D] seen as flat
 * slots).  Returns 0, or -1 if a slot is out of range (nothing is written in that case).
 */
int oracle_kv_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                    void* v_cache, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                    int64_t num_slots, int32_t in_dtype, int32_t cache_dtype) {
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    const int64_t scratch = num_slots - 1;
    for (int64_t i = 0; i < num_tokens; ++i)
        if (slot_mapping[i] >= num_slots) return -1;
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t s = slot_mapping[i] >= 0 ? slot_mapping[i] : scratch;
        for (int64_t e = 0; e < row; ++e) {
            store_elem(k_cache, s * row + e, cache_dtype, load_elem(k, i * row + e, in_dtype));
            store_elem(v_cache, s * row + e, cache_dtype, load_elem(v, i * row + e, in_dtype));
        }
    }
    return 0;
}

/* gather_context over a quantized pool: each element is its code's value times the scale of
 * its (slot, KV head) row (ReferenceBackend.dequantize). */
static void gather_fp8(const uint8_t* cache, const float* scale, const int32_t* table_row, int32_t length,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim, double* out) {
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    for (int32_t p = 0; p < length; ++p) {
        const int64_t slot = (int64_t)table_row[p / block_size] * block_size + p % block_size;
        for (int64_t e = 0; e < row; ++e)
            out[(int64_t)p * row + e] = oracle_fp8_e4m3_decode(cache[slot * row + e]) *
                                        (double)scale[slot * num_kv_heads + e / head_dim];
    }
}

/*
 * gather_context: the first `length` token rows of a request, in logical order.  Position p
 * lives at slot table[p / block_size] * block_size + p % block_size.  out is [length, Hkv, D].
 */
void oracle_gather_context(const void* cache, const int32_t* table_row, int32_t length,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           int32_t dtype, double* out) {
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    for (int32_t p = 0; p < length; ++p) {
        int64_t slot = (int64_t)table_row[p / block_size] * block_size + p % block_size;
        for (int64_t e = 0; e < row; ++e) out[(int64_t)p * row + e] = load_elem(cache, slot * row + e, dtype);
    }
}

/*
 * ReferenceBackend.forward ("Attention over the pool").
 *
 * q, out: [N, H, D] in dtype; caches: [num_slots, Hkv, D] in kv_dtype (dtype, or fp8 codes
 * with k_scale / v_scale [num_slots, Hkv]); query_start_loc [R+1]; seq_lens [R]; block_table
 * [R, stride].  scale multiplies every score.  window > 0: sliding window (see above).
 * out_f64, if not NULL, receives the unrounded float64 result ([N, H, D]).
 * row_mask, if not NULL, selects the flattened rows to compute ([N] bytes, nonzero = compute);
 * rows not selected are left untouched in both outputs.
 * Returns 0, or -1 on inconsistent metadata (then nothing is written).
 */
int oracle_paged_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* query_start_loc, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t block_size, double scale, void* out,
                           double* out_f64, int32_t num_reqs, int64_t num_tokens,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_table_stride, int64_t num_slots, int32_t dtype,
                           const uint8_t* row_mask, int32_t window, int32_t kv_dtype,
                           const float* k_scale, const float* v_scale) {
    if (kv_dtype != dtype && (kv_dtype != ORACLE_FP8 || !k_scale || !v_scale)) return -1;
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || block_size <= 0) return -1;
    if (query_start_loc[0] != 0 || query_start_loc[num_reqs] != num_tokens) return -1;
    for (int32_t r = 0; r < num_reqs; ++r) {
        int32_t t = query_start_loc[r + 1] - query_start_loc[r];
        int32_t len = seq_lens[r];
        if (t < 0 || len < 0) return -1;
        if (len > 0 && t > len) return -1;
        int32_t nblk = (len + block_size - 1) / block_size;
        if (nblk > block_table_stride) return -1;
        for (int32_t b = 0; b < nblk; ++b) {
            int64_t blk = block_table[(int64_t)r * block_table_stride + b];
            if (blk < 0 || (blk + 1) * block_size > num_slots) return -1;
        }
    }
    const int32_t group = num_heads / num_kv_heads;
    const int64_t qrow = (int64_t)num_heads * head_dim;
    const int64_t kvrow = (int64_t)num_kv_heads * head_dim;

    for (int32_t r = 0; r < num_reqs; ++r) {
        const int32_t begin = query_start_loc[r], end = query_start_loc[r + 1];
        const int32_t length = seq_lens[r];
        if (length == 0 || begin == end) {          /* padding row: output stays zero */
            for (int64_t i = begin; i < end; ++i) {
                if (row_mask && !row_mask[i]) continue;
                for (int64_t e = 0; e < qrow; ++e) {
                    store_elem(out, i * qrow + e, dtype, 0.0);
                    if (out_f64) out_f64[i * qrow + e] = 0.0;
                }
            }
            continue;
        }
        const int32_t t = end - begin;
        int any = 0;
        for (int32_t i = 0; i < t && !any; ++i) any = !row_mask || row_mask[begin + i];
        if (!any) continue;

        const int32_t* table_row = block_table + (int64_t)r * block_table_stride;
        double* ctx_k = (double*)malloc(sizeof(double) * (size_t)length * (size_t)kvrow);
        double* ctx_v = (double*)malloc(sizeof(double) * (size_t)length * (size_t)kvrow);
        if (!ctx_k || !ctx_v) { free(ctx_k); free(ctx_v); return -2; }
        if (kv_dtype == ORACLE_FP8) {
            gather_fp8((const uint8_t*)k_cache, k_scale, table_row, length, block_size, num_kv_heads, head_dim, ctx_k);
            gather_fp8((const uint8_t*)v_cache, v_scale, table_row, length, block_size, num_kv_heads, head_dim, ctx_v);
        } else {
            oracle_gather_context(k_cache, table_row, length, block_size, num_kv_heads, head_dim, dtype, ctx_k);
            oracle_gather_context(v_cache, table_row, length, block_size, num_kv_heads, head_dim, dtype, ctx_v);
        }

        int failed = 0;
        #pragma omp parallel for collapse(2) schedule(dynamic, 1)
        for (int32_t i = 0; i < t; ++i) {
            for (int32_t h = 0; h < num_heads; ++h) {
                const int64_t row = (int64_t)begin + i;
                if (row_mask && !row_mask[row]) continue;
                const int32_t kvh = h / group;
                const int32_t q_pos = length - t + i;       /* the last t positions of the context */
                /* first visible key: 0, or with a window of w tokens the first with k_pos > q_pos - w */
                const int32_t j0 = (window > 0 && q_pos - window + 1 > 0) ? q_pos - window + 1 : 0;
                double* s = (double*)malloc(sizeof(double) * (size_t)(q_pos + 1));
                double* acc = (double*)calloc((size_t)head_dim, sizeof(double));
                double* qv = (double*)malloc(sizeof(double) * (size_t)head_dim);
                if (!s || !acc || !qv) {
                    free(s); free(acc); free(qv);
                    #pragma omp atomic write
                    failed = 1;
                    continue;
                }
                for (int32_t d = 0; d < head_dim; ++d) qv[d] = load_elem(q, row * qrow + (int64_t)h * head_dim + d, dtype);
                /* pass 1: scores of keys j0 .. q_pos and their maximum */
                double m = -INFINITY;
                for (int32_t j = j0; j <= q_pos; ++j) {
                    const double* kj = ctx_k + (int64_t)j * kvrow + (int64_t)kvh * head_dim;
                    double dot = 0.0;
                    for (int32_t d = 0; d < head_dim; ++d) dot += qv[d] * kj[d];
                    s[j] = scale * dot;
                    if (s[j] > m) m = s[j];
                }
                /* pass 2: exponentials, their sum and the weighted sum of V */
                double l = 0.0;
                for (int32_t j = j0; j <= q_pos; ++j) {
                    const double w = exp(s[j] - m);
                    const double* vj = ctx_v + (int64_t)j * kvrow + (int64_t)kvh * head_dim;
                    l += w;
                    for (int32_t d = 0; d < head_dim; ++d) acc[d] += w * vj[d];
                }
                for (int32_t d = 0; d < head_dim; ++d) {
                    const double o = acc[d] / l;
                    const int64_t idx = row * qrow + (int64_t)h * head_dim + d;
                    store_elem(out, idx, dtype, o);
                    if (out_f64) out_f64[idx] = o;
                }
                free(s); free(acc); free(qv);
            }
        }
        free(ctx_k);
        free(ctx_v);
        if (failed) return -2;
    }
    return 0;
}
