/*
 * oracle.h -- plain, slow CPU reference for the FP8 E4M3 paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library
 * and its Python binding) may include, link or call this code; only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no source with the GPU path: its own codec tables, its own
 * loops, double-precision accumulation.
 *
 * What it follows (page titles, with the part of the page):
 *   [ATOM]  "fix(qwen4-exp): register the QSA FP8 scale planes for KV
 *           offload" (ROCm/ATOM #2655), description, K/V bullet: one FP32
 *           scale per (token, KV head) = row amax / FP8 max; the attend
 *           applies each key's scale to that key's score and the value's
 *           scale to its probability weight.
 *   [FT]    "feat(kvcache): store the KV cache as fp8 e4m3 codes"
 *           (FreeToken #354), description: head_dim codes + ONE fp32
 *           symmetric scale per row, uint8 code buffer with the 16-bit
 *           geometry; and the fix commit "give the V tensor its own row
 *           pitch in the fp8 KV store": K and V each carry their own pitch,
 *           codes are checked against a round-to-nearest-even reference.
 *   [SGJ]   "feat(dsa): implement fp8 KV cache (e4m3) with a bf16 indexer
 *           cache" (sglang-jax #1776), description and "Three design
 *           points": e4m3 range 448, 0.0156 subnormal floor, ~6% vs ~12.5%
 *           worst-case relative error for e4m3 vs e5m2.
 *   [OCPMX] OCP Microscaling Formats (MX) Specification v1.0: E2M1 (FP4,
 *           bias 1, max 6, no inf/NaN) and the E8M0 shared scale 2^(c-127).
 *   [OFP8]  OCP 8-bit Floating Point Specification (OFP8) rev. 1.0: the bit
 *           layouts of E4M3 (bias 7, no infinities, S.1111.111 = NaN, max
 *           448) and E5M2 (bias 15, IEEE-style inf/NaN, max 57344).
 *
 * Parity status of every function is stated at its definition.
 */
#ifndef FP8KV_ORACLE_H
#define FP8KV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { FO_E4M3 = 0, FO_E5M2 = 1 };

/* ---- codec (e4m3.c) ---------------------------------------------------- */
double   fo_decode(int fmt, unsigned code);          /* NaN for NaN codes      */
unsigned fo_encode(int fmt, float f);                /* nearest, ties-to-even, */
                                                     /* saturating to +-max    */
double   fo_fmt_max(int fmt);                        /* 448 or 57344           */
void     fo_encode_array(int fmt, const float* in, int64_t n, uint8_t* out);
void     fo_decode_array(int fmt, const uint8_t* in, int64_t n, double* out);
float    fo_bf16_to_f32(uint16_t bits);

/* ---- per-row quantizer and paged scatter (quant.c) ---------------------- */
void fo_quantize_row(int fmt, const float* x, int64_t D, uint8_t* codes,
                     float* scale);
/* fo_quantize_row over n_rows bf16 rows of x (row pitch x_stride elements);
 * codes [n_rows, D] and scales [n_rows], both dense. */
void fo_quantize_rows_bf16(int fmt, const uint16_t* x, int64_t n_rows,
                           int64_t D, int64_t x_stride, uint8_t* codes,
                           float* scales);
void fo_kv_quant_scatter_bf16(
    const uint16_t* k, int64_t k_stride_tok, int64_t k_stride_head,
    const uint16_t* v, int64_t v_stride_tok, int64_t v_stride_head,
    int64_t num_tokens, int64_t num_kv_heads, int64_t head_dim,
    const int64_t* slot_ids, int64_t num_slots,
    uint8_t* k_cache, uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    float* k_scale, float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head);

/* The unscaled cache: every element encoded by itself in fmt (saturating),
 * placed like the scaled codes, no scale planes. Parity: pinned by the
 * codec pins, torch casts of in-range values and a sentinel pool. */
void fo_kv_scatter_unscaled_bf16(
    int fmt,
    const uint16_t* k, int64_t k_stride_tok, int64_t k_stride_head,
    const uint16_t* v, int64_t v_stride_tok, int64_t v_stride_head,
    int64_t num_tokens, int64_t num_kv_heads, int64_t head_dim,
    const int64_t* slot_ids, int64_t num_slots,
    uint8_t* k_cache, uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head);

/* ---- attention (attn.c) ------------------------------------------------- */
/* Dense softmax attention of one query row over n already-dequantized keys:
 * out[d] = sum_j softmax_j(scale * q.k_j) * v_j[d], all in double. n == 0
 * gives out = 0. */
void fo_attend_dense(const double* q, const double* keys, const double* vals,
                     int64_t n, int64_t D, double scale, double* out);

/* Paged GQA decode attention over a quantized cache (fmt codes + fp32 row
 * scales). Rows are (b, r, hq) with r in [0, R) the verify rows of request
 * b; row r sees cache tokens 0 .. context_lens[b] - R + r. When
 * partition_tokens > 0 the keys are split at multiples of partition_tokens,
 * each part is reduced to (max, sum, weighted sum) and the parts are merged
 * by log-sum-exp. rows_sel (n_rows_sel entries, flat index
 * (b*R + r)*Hq + hq) restricts the work to those rows and packs out as
 * [n_rows_sel, D]; rows_sel == NULL computes every row into [B, R, Hq, D]. */
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
    const int64_t* rows_sel, int64_t n_rows_sel, double* out);

/* The same attention over selected blocks: block_tables rows list each
 * request's selected blocks in position order; block_valid[b][i] counts the
 * keys of the i-th selected block from its start (0 .. block_size).
 * Virtual position j = i * block_size + o is a key iff o < block_valid[b][i];
 * row r sees virtual positions 0 .. context_lens[b] - R + r. */
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
    const int64_t* rows_sel, int64_t n_rows_sel, double* out);

/* ---- compressed index keys and the index scorer (index.c) --------------
 * [ATOM] description, compressed-index bullet and the stacked-scorer
 * paragraph. Parity: the codec is pinned by closed forms, the OCP tables
 * and brute force; the nibble order and the zero-group code are
 * conventions (parity unpinned beyond self-consistency); the scorer is
 * pinned by closed forms and an independent float64 evaluation. */
enum { FO_KEYS_MXFP4 = 0, FO_KEYS_E4M3 = 1 };
double fo_e2m1_value(unsigned code);                 /* 4-bit code -> value   */
double fo_e8m0_value(unsigned code);                 /* 2^(code - 127)        */
void   fo_mxfp4_encode_group(const float* x, uint8_t* packed, uint8_t* exp_code);
void   fo_index_keys_mxfp4(const uint16_t* keys, int64_t n, int64_t d, int64_t ks,
                           uint8_t* packed, int64_t ps, uint8_t* exps, int64_t es);
void   fo_index_keys_pool(const uint16_t* raw, int64_t rs, int64_t d, int64_t g0,
                          int64_t g1, double* out);
uint16_t fo_bf16_rne(double x);                      /* one rounding to bf16  */
void   fo_index_keys_build_bf16(const uint16_t* raw, int64_t rs, int64_t d, int64_t g0,
                                int64_t g1, uint16_t* out);
void   fo_index_score(int key_format, const uint16_t* q, int64_t qb, int64_t qr, int64_t qh,
                      const float* w, int64_t wb, int64_t wr, int64_t wh,
                      const void* codes, int64_t cb, int64_t cs,
                      const void* scales, int64_t sb, int64_t ss,
                      int64_t B, int64_t R, int64_t H, int64_t D, int64_t N, double* out);

#ifdef __cplusplus
}
#endif

#endif
