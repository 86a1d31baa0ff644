/*
 * quant.c -- per-row quantizer and paged scatter of the oracle (test
 * infrastructure only).
 *
 * Row format ([FT] description; [ATOM] description, K/V bullet): one
 * (token, KV head) row of K, and separately of V, becomes head_dim FP8
 * codes plus ONE fp32 symmetric scale equal to the row's absolute maximum
 * divided by the format's largest finite value (448 for e4m3).
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes):
 *   - the scale is the IEEE binary32 quotient amax / 448 (a division, not a
 *     multiplication by a rounded reciprocal);
 *   - each code is the nearest-even FP8 value of the binary32 quotient
 *     x / scale: the quotient is rounded to binary32 first, then to FP8,
 *     which is what a framework cast (x / scale).to(fp8) computes -- the
 *     FreeToken fix commit checks codes against such a reference;
 *   - an all-zero row has scale 0 and every code is the encoding of the
 *     (signed) zero input, with no division;
 *   - inputs are finite.
 *
 * Scatter: row (t, h) of K lands at k_cache[slot_ids[t] * cache_stride_slot
 * + h * cache_stride_head + d] and its scale at k_scale[slot_ids[t] *
 * scale_stride_slot + h * scale_stride_head]; V likewise. K and V are read
 * with their OWN token and head strides (the FreeToken V-pitch fix). A slot
 * id < 0 or >= num_slots writes nothing.
 *
 * Parity pins: codes equal torch's (x / scale).to(float8_e4m3fn) cast; the
 * row maximum always encodes to +-448 (dynamic row scales cannot overflow the format); reconstruction
 * within the format's relative half-ulp; zero rows; the strided-pitch
 * scenario of the FreeToken fix with distinct K and V pitches; sentinel
 * pools that show exactly the addressed rows change.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "oracle.h"

void fo_quantize_row(int fmt, const float* x, int64_t D, uint8_t* codes,
                     float* scale) {
    float amax = 0.0f;
    for (int64_t d = 0; d < D; ++d) {
        const float a = fabsf(x[d]);
        if (a > amax) amax = a;
    }
    const float fmax = (float)fo_fmt_max(fmt);     /* 448 or 57344, exact */
    const float s = amax / fmax;                    /* IEEE binary32 division */
    for (int64_t d = 0; d < D; ++d) {
        const float q = (s == 0.0f) ? x[d] : x[d] / s;  /* binary32 quotient */
        codes[d] = (uint8_t)fo_encode(fmt, q);
    }
    *scale = s;
}

void fo_quantize_rows_bf16(int fmt, const uint16_t* x, int64_t n_rows,
                           int64_t D, int64_t x_stride, uint8_t* codes,
                           float* scales) {
    float* row = (float*)malloc((size_t)D * sizeof(float));
    for (int64_t i = 0; i < n_rows; ++i) {
        for (int64_t d = 0; d < D; ++d)
            row[d] = fo_bf16_to_f32(x[i * x_stride + d]);
        fo_quantize_row(fmt, row, D, codes + i * D, scales + i);
    }
    free(row);
}

void fo_kv_quant_scatter_bf16(
    const uint16_t* k, int64_t k_stride_tok, int64_t k_stride_head,
    const uint16_t* v, int64_t v_stride_tok, int64_t v_stride_head,
    int64_t num_tokens, int64_t num_kv_heads, int64_t head_dim,
    const int64_t* slot_ids, int64_t num_slots,
    uint8_t* k_cache, uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    float* k_scale, float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head) {
    float* row = (float*)malloc((size_t)head_dim * sizeof(float));
    uint8_t* codes = (uint8_t*)malloc((size_t)head_dim);
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int64_t slot = slot_ids[t];
        if (slot < 0 || slot >= num_slots) continue;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            for (int kv = 0; kv < 2; ++kv) {
                const uint16_t* src = kv == 0
                    ? k + t * k_stride_tok + h * k_stride_head
                    : v + t * v_stride_tok + h * v_stride_head;
                uint8_t* dst = (kv == 0 ? k_cache : v_cache) +
                               slot * cache_stride_slot + h * cache_stride_head;
                float* sdst = (kv == 0 ? k_scale : v_scale) +
                              slot * scale_stride_slot + h * scale_stride_head;
                for (int64_t d = 0; d < head_dim; ++d)
                    row[d] = fo_bf16_to_f32(src[d]);
                float s;
                fo_quantize_row(FO_E4M3, row, head_dim, codes, &s);
                for (int64_t d = 0; d < head_dim; ++d) dst[d] = codes[d];
                *sdst = s;
            }
        }
    }
    free(codes);
    free(row);
}

/* The unscaled cache ("feat(dsa): implement fp8 KV cache (e4m3) with a bf16
 * indexer cache", sglang-jax #1776, description and "Three design points":
 * new K/V are cast to the cache dtype with no scale). Each element is
 * encoded by itself in fmt (nearest, ties to even, saturating to the
 * format's largest finite value) and placed like the scaled codes; there
 * are no scale planes. */
void fo_kv_scatter_unscaled_bf16(
    int fmt,
    const uint16_t* k, int64_t k_stride_tok, int64_t k_stride_head,
    const uint16_t* v, int64_t v_stride_tok, int64_t v_stride_head,
    int64_t num_tokens, int64_t num_kv_heads, int64_t head_dim,
    const int64_t* slot_ids, int64_t num_slots,
    uint8_t* k_cache, uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head) {
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int64_t slot = slot_ids[t];
        if (slot < 0 || slot >= num_slots) continue;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            for (int kv = 0; kv < 2; ++kv) {
                const uint16_t* src = kv == 0
                    ? k + t * k_stride_tok + h * k_stride_head
                    : v + t * v_stride_tok + h * v_stride_head;
                uint8_t* dst = (kv == 0 ? k_cache : v_cache) +
                               slot * cache_stride_slot + h * cache_stride_head;
                for (int64_t d = 0; d < head_dim; ++d)
                    dst[d] = (uint8_t)fo_encode(fmt, fo_bf16_to_f32(src[d]));
            }
        }
    }
}
