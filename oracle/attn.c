/*
 * attn.c -- paged GQA decode attention of the oracle (test infrastructure
 * only).
 *
 * Semantics ([ATOM] description, K/V bullet; sglang-jax #1776,
 * "Modifications", qblock prefill bullet): the attend reads the FP8 tiles
 * back, the key scale multiplies the score of its key, the value scale
 * weights its value row, and nothing is ever rounded to the cache format on
 * the way -- here everything after decoding is double precision.
 *
 * For row (b, r, hq) with G = Hq / Hkv:
 *   h      = hq / G                     (consecutive query heads share a KV
 *                                        head -- a reading)
 *   n      = context_lens[b] - R + r + 1   visible keys 0 .. n-1 (the R
 *                                        verify rows are causal among
 *                                        themselves -- a reading)
 *   slot_j = block_tables[b][j / bs] * bs + j % bs
 *   k_j[d] = decode(k_code[slot_j, h, d]) * k_scale[slot_j, h]
 *   v_j[d] = decode(v_code[slot_j, h, d]) * v_scale[slot_j, h]
 *   out    = softmax_j(softmax_scale * q . k_j) weighted sum of v_j
 * with out = 0 when n <= 0 (a reading: an empty row yields zeros, not NaN).
 *
 * The optional split into partitions of partition_tokens keys, each reduced
 * to (max score, sum of exp, exp-weighted value sum) and merged by
 * log-sum-exp, exists to pin the merge algebra: it must equal the unsplit
 * result to rounding.
 *
 * Parity pins: torch float64 softmax(q K^T) V on the dequantized keys,
 * single-key and constant-score closed forms, MTP-row / prefix equivalence,
 * GQA == MHA with replicated KV, split == unsplit.
 *
 * fo_sparse_decode_attn is the same attention over selected blocks (see its
 * comment); pins: torch on the explicitly gathered keys, full selection ==
 * dense, single key, empty blocks and block order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

void fo_attend_dense(const double* q, const double* keys, const double* vals,
                     int64_t n, int64_t D, double scale, double* out) {
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    if (n <= 0) return;
    double* s = (double*)malloc((size_t)n * sizeof(double));
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += q[d] * keys[j * D + d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        const double p = exp(s[j] - m);
        l += p;
        for (int64_t d = 0; d < D; ++d) out[d] += p * vals[j * D + d];
    }
    for (int64_t d = 0; d < D; ++d) out[d] /= l;
    free(s);
}

/* fo_decode of every code, tabulated once when the library loads. */
static double g_value[2][256];

__attribute__((constructor)) static void build_value_tables(void) {
    for (int fmt = 0; fmt < 2; ++fmt)
        for (unsigned c = 0; c < 256; ++c) g_value[fmt][c] = fo_decode(fmt, c);
}

/* One key or value row of the cache, dequantized into dst[0..D). */
static void dequant_row(int fmt, const uint8_t* cache, const float* scales,
                        int64_t slot, int64_t h, int64_t cache_stride_slot,
                        int64_t cache_stride_head, int64_t scale_stride_slot,
                        int64_t scale_stride_head, int64_t D, double* dst) {
    const uint8_t* c = cache + slot * cache_stride_slot + h * cache_stride_head;
    const double s =
        (double)scales[slot * scale_stride_slot + h * scale_stride_head];
    for (int64_t d = 0; d < D; ++d) dst[d] = g_value[fmt][c[d]] * s;
}

/* Reduce keys [j0, j1) of a gathered row set to (max, sum, weighted sum). */
static void partial_reduce(const double* q, const double* keys,
                           const double* vals, int64_t j0, int64_t j1,
                           int64_t D, double scale, double* m_out,
                           double* l_out, double* acc) {
    double m = -INFINITY;
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += q[d] * keys[j * D + d];
        if (scale * dot > m) m = scale * dot;
    }
    double l = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += q[d] * keys[j * D + d];
        const double p = exp(scale * dot - m);
        l += p;
        for (int64_t d = 0; d < D; ++d) acc[d] += p * vals[j * D + d];
    }
    *m_out = m;
    *l_out = l;
}

static void attend_one_row(
    int fmt, const uint16_t* q_row, const uint8_t* k_cache,
    const uint8_t* v_cache, int64_t cache_stride_slot,
    int64_t cache_stride_head, const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    const int32_t* bt_row, const int32_t* valid_row, int64_t n, int64_t h,
    int64_t D, int64_t block_size, double softmax_scale,
    int64_t partition_tokens, double* out) {
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    if (n <= 0) return;
    double* q = (double*)malloc((size_t)D * sizeof(double));
    double* keys = (double*)malloc((size_t)(n * D) * sizeof(double));
    double* vals = (double*)malloc((size_t)(n * D) * sizeof(double));
    for (int64_t d = 0; d < D; ++d) q[d] = (double)fo_bf16_to_f32(q_row[d]);
    /* page-table walk: position j lives in block bt_row[j / bs] at offset
     * j % bs; with a valid row, only offsets below the block's valid count
     * are keys (the others are skipped, not zeroed) */
    int64_t kept = 0;
    for (int64_t j = 0; j < n; ++j) {
        const int64_t i = j / block_size, o = j % block_size;
        if (valid_row && o >= (int64_t)valid_row[i]) continue;
        const int64_t slot = (int64_t)bt_row[i] * block_size + o;
        dequant_row(fmt, k_cache, k_scale, slot, h, cache_stride_slot,
                    cache_stride_head, scale_stride_slot, scale_stride_head, D,
                    keys + kept * D);
        dequant_row(fmt, v_cache, v_scale, slot, h, cache_stride_slot,
                    cache_stride_head, scale_stride_slot, scale_stride_head, D,
                    vals + kept * D);
        ++kept;
    }
    n = kept;
    if (n == 0) {
        free(vals);
        free(keys);
        free(q);
        return;
    }
    if (partition_tokens <= 0) {
        fo_attend_dense(q, keys, vals, n, D, softmax_scale, out);
    } else {
        /* split at absolute multiples of partition_tokens, then merge by
         * log-sum-exp: out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p */
        const int64_t np = (n + partition_tokens - 1) / partition_tokens;
        double* pm = (double*)malloc((size_t)np * sizeof(double));
        double* pl = (double*)malloc((size_t)np * sizeof(double));
        double* pacc = (double*)malloc((size_t)(np * D) * sizeof(double));
        double M = -INFINITY;
        for (int64_t p = 0; p < np; ++p) {
            const int64_t j0 = p * partition_tokens;
            const int64_t j1 =
                j0 + partition_tokens < n ? j0 + partition_tokens : n;
            partial_reduce(q, keys, vals, j0, j1, D, softmax_scale, &pm[p],
                           &pl[p], pacc + p * D);
            if (pm[p] > M) M = pm[p];
        }
        double lsum = 0.0;
        for (int64_t p = 0; p < np; ++p) {
            const double w = exp(pm[p] - M);
            lsum += w * pl[p];
            for (int64_t d = 0; d < D; ++d) out[d] += w * pacc[p * D + d];
        }
        for (int64_t d = 0; d < D; ++d) out[d] /= lsum;
        free(pacc);
        free(pl);
        free(pm);
    }
    free(vals);
    free(keys);
    free(q);
}

void fo_paged_decode_attn(
    int fmt,
    const uint16_t* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head,
    const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens,
    int64_t B, int64_t R, int64_t Hq, int64_t Hkv, int64_t D,
    int64_t block_size, double softmax_scale, int64_t partition_tokens,
    const int64_t* rows_sel, int64_t n_rows_sel, double* out) {
    const int64_t G = Hq / Hkv;
    const int64_t total = rows_sel ? n_rows_sel : B * R * Hq;
    for (int64_t i = 0; i < total; ++i) {
        const int64_t flat = rows_sel ? rows_sel[i] : i;
        const int64_t hq = flat % Hq;
        const int64_t r = (flat / Hq) % R;
        const int64_t b = flat / (Hq * R);
        const int64_t n = (int64_t)context_lens[b] - R + r + 1;
        attend_one_row(fmt,
                       q + b * q_stride_b + r * q_stride_row + hq * q_stride_head,
                       k_cache, v_cache, cache_stride_slot, cache_stride_head,
                       k_scale, v_scale, scale_stride_slot, scale_stride_head,
                       block_tables + b * block_table_stride, NULL, n, hq / G,
                       D, block_size, softmax_scale, partition_tokens,
                       out + i * D);
    }
}

/*
 * Decode attention over selected blocks ([ATOM] description, K/V bullet:
 * the sparse GQA kernel reads E4M3 tiles with the same scale handling;
 * FreeToken #354, description: the selection keys are 16-bit and the
 * cache is fetched, as codes, for the chosen rows alone). The selected blocks of request b are its page table, in
 * position order; block_valid[b][i] (0 .. bs) counts the tokens of the i-th
 * selected block that are keys, from its start. Virtual position
 * j = i * bs + o is a key iff o < block_valid[b][i]; row r of R sees the
 * virtual positions 0 .. context_lens[b] - R + r (context_lens counts
 * virtual positions). Everything else is fo_paged_decode_attn.
 */
void fo_sparse_decode_attn(
    int fmt,
    const uint16_t* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head,
    const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* block_valid, int64_t block_valid_stride,
    const int32_t* context_lens,
    int64_t B, int64_t R, int64_t Hq, int64_t Hkv, int64_t D,
    int64_t block_size, double softmax_scale,
    const int64_t* rows_sel, int64_t n_rows_sel, double* out) {
    const int64_t G = Hq / Hkv;
    const int64_t total = rows_sel ? n_rows_sel : B * R * Hq;
    for (int64_t i = 0; i < total; ++i) {
        const int64_t flat = rows_sel ? rows_sel[i] : i;
        const int64_t hq = flat % Hq;
        const int64_t r = (flat / Hq) % R;
        const int64_t b = flat / (Hq * R);
        const int64_t n = (int64_t)context_lens[b] - R + r + 1;
        attend_one_row(fmt,
                       q + b * q_stride_b + r * q_stride_row + hq * q_stride_head,
                       k_cache, v_cache, cache_stride_slot, cache_stride_head,
                       k_scale, v_scale, scale_stride_slot, scale_stride_head,
                       block_tables + b * block_table_stride,
                       block_valid + b * block_valid_stride, n, hq / G, D,
                       block_size, softmax_scale, 0, out + i * D);
    }
}
