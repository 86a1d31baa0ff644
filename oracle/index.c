/* index.c -- CPU oracle for the compressed-index keys and the index scorer.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
 *
 * Source: "fix(qwen4-exp): register the QSA FP8 scale planes for KV
 * offload" (ROCm/ATOM #2655), description: the compressed index keys are
 * stored either as FP8 with one fp32 scale per row, or as MXFP4 -- packed
 * E2M1 pairs with one E8M0 exponent per 32 dims, the exponent chosen high
 * enough that no element of the group overflows; the decode-sized scorer stacks rows x index
 * heads into the MFMA M dimension and applies the per-head ReLU before the
 * heads are summed. The scored quantity, per (row r, key n):
 *     score[r, n] = sum_h w[r, h] * max(0, q[r, h, :] . k^[n, :])
 * with k^ the dequantized key.
 *
 * Readings (stated where the page is silent):
 *   - E2M1 is the OCP FP4 format: 1 sign, 2 exponent bits (bias 1), 1
 *     mantissa bit; no inf/NaN; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
 *   - E8M0 code c is the scale 2^(c - 127) (c = 255, NaN, is never written).
 *   - The upward-rounded group exponent: e is the smallest integer with
 *     amax <= 6 * 2^e, found by exact comparison; code = e + 127, clamped
 *     to [0, 254]. An all-zero group gets code 127.
 *   - Each element is x / 2^e (exact) rounded to the nearest E2M1 magnitude,
 *     ties to the even code, with the sign of x kept.
 *   - Packing: byte j of a group holds element 2j in its low nibble and
 *     element 2j+1 in its high nibble.
 * Everything is evaluated in double; nothing here is blocked or reordered.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "oracle.h"

/* OCP E2M1: value of a 4-bit code, built from its bit fields. */
double fo_e2m1_value(unsigned code) {
    const unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag;
    if (e == 0)
        mag = 0.5 * (double)m;                       /* subnormal: m * 2^(1-1) / 2 */
    else
        mag = ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E8M0: the power-of-two scale of an exponent code. */
double fo_e8m0_value(unsigned code) { return ldexp(1.0, (int)code - 127); }

/* Nearest E2M1 code to |v| (v already divided by the group scale), ties
 * to the even code, by exhaustive search over the 8 magnitudes. */
static unsigned e2m1_nearest(double av) {
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned c = 0; c < 8; ++c) {
        const double d = fabs(fo_e2m1_value(c) - av);
        if (d < best_d || (d == best_d && (c & 1u) == 0 && (best & 1u) != 0)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* One group of 32 values: the exponent code and 16 packed bytes. */
void fo_mxfp4_encode_group(const float* x, uint8_t* packed, uint8_t* exp_code) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i)
        if (fabs((double)x[i]) > amax) amax = fabs((double)x[i]);
    int e = 0;
    if (amax > 0.0) {
        /* smallest e with amax <= 6 * 2^e, by exact comparison */
        e = -127;
        while (e < 127 && !(amax <= 6.0 * ldexp(1.0, e))) ++e;
    }
    *exp_code = (uint8_t)(e + 127);
    const double scale = ldexp(1.0, e);
    for (int j = 0; j < 16; ++j) {
        unsigned nib[2];
        for (int t = 0; t < 2; ++t) {
            const double v = (double)x[2 * j + t] / scale;     /* exact */
            unsigned c = e2m1_nearest(fabs(v));
            if (signbit(v)) c |= 8u;
            nib[t] = c;
        }
        packed[j] = (uint8_t)(nib[0] | (nib[1] << 4));
    }
}

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* MXFP4 index keys: n keys of d bf16 values (row stride ks elements) ->
 * packed [n, d/2] bytes (row stride ps) + exponent codes [n, d/32] (row
 * stride es). */
void fo_index_keys_mxfp4(const uint16_t* keys, int64_t n, int64_t d, int64_t ks,
                         uint8_t* packed, int64_t ps, uint8_t* exps, int64_t es) {
    float g[32];
    for (int64_t i = 0; i < n; ++i)
        for (int64_t grp = 0; grp < d / 32; ++grp) {
            for (int t = 0; t < 32; ++t) g[t] = (float)bf16_value(keys[i * ks + grp * 32 + t]);
            fo_mxfp4_encode_group(g, packed + i * ps + grp * 16, exps + i * es + grp);
        }
}

/* Dequantized key element d of key i. */
static double key_value(int key_format, const void* codes, int64_t cs, const void* scales,
                        int64_t ss, int64_t i, int64_t d) {
    if (key_format == FO_KEYS_MXFP4) {
        const uint8_t byte = ((const uint8_t*)codes)[i * cs + d / 2];
        const unsigned c = (d & 1) ? (byte >> 4) : (byte & 15u);
        const unsigned ec = ((const uint8_t*)scales)[i * ss + d / 32];
        return fo_e2m1_value(c) * fo_e8m0_value(ec);
    }
    const uint8_t c = ((const uint8_t*)codes)[i * cs + d];
    return fo_decode(FO_E4M3, c) * (double)((const float*)scales)[i * ss];
}

/* score[b, r, n] = sum_h w[b, r, h] * max(0, q[b, r, h, :] . k^[b, n, :]),
 * in double. q bf16 bits with element strides (qb, qr, qh); w fp32 with
 * strides (wb, wr, wh); keys of request b at codes + b*cb, row stride cs
 * (bytes), scales at + b*sb, row stride ss (elements of fp32 for E4M3,
 * bytes for MXFP4). out [B, R, N] contiguous. */
void fo_index_score(int key_format, const uint16_t* q, int64_t qb, int64_t qr, int64_t qh,
                    const float* w, int64_t wb, int64_t wr, int64_t wh,
                    const void* codes, int64_t cb, int64_t cs,
                    const void* scales, int64_t sb, int64_t ss,
                    int64_t B, int64_t R, int64_t H, int64_t D, int64_t N, double* out) {
    for (int64_t b = 0; b < B; ++b) {
        const uint8_t* cbase = (const uint8_t*)codes + b * cb;
        const void* sbase = key_format == FO_KEYS_MXFP4
                                ? (const void*)((const uint8_t*)scales + b * sb)
                                : (const void*)((const float*)scales + b * sb);
        for (int64_t r = 0; r < R; ++r)
            for (int64_t n = 0; n < N; ++n) {
                double score = 0.0;
                for (int64_t h = 0; h < H; ++h) {
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        dot += bf16_value(q[b * qb + r * qr + h * qh + d]) *
                               key_value(key_format, cbase, cs, sbase, ss, n, d);
                    score += (double)w[b * wb + r * wr + h * wh] * (dot > 0.0 ? dot : 0.0);
                }
                out[(b * R + r) * N + n] = score;
            }
    }
}

/* Index-key builder ([ATOM] description, compressed-index bullet: the raw
 * index keys are kept in BF16, averaged in groups first and normalized
 * after; a group may span two prefill chunks). Compressed key g of a request is
 *     m[d] = (r[4g][d] + r[4g+1][d] + r[4g+2][d] + r[4g+3][d]) / 4
 *     k[d] = m[d] / ||m||_2            (k = 0 when m = 0)
 * evaluated in double for groups g0 .. g1-1 of raw keys r (bf16 bits, row
 * stride rs elements); out[(g - g0) * d + i] = k[i]. Which group a key
 * belongs to depends only on its position, never on the chunk it arrived
 * in. */
void fo_index_keys_pool(const uint16_t* raw, int64_t rs, int64_t d, int64_t g0,
                        int64_t g1, double* out) {
    for (int64_t g = g0; g < g1; ++g) {
        double* k = out + (g - g0) * d;
        double ss = 0.0;
        for (int64_t i = 0; i < d; ++i) {
            double s = 0.0;
            for (int t = 0; t < 4; ++t) s += bf16_value(raw[(4 * g + t) * rs + i]);
            k[i] = s / 4.0;
            ss += k[i] * k[i];
        }
        const double n = sqrt(ss);
        for (int64_t i = 0; i < d; ++i) k[i] = n > 0.0 ? k[i] / n : 0.0;
    }
}

/* bf16 bits of the bf16 value nearest to x (finite, |x| < 2^128), ties to
 * the value with an even last mantissa bit: one rounding straight from
 * double. bf16 keeps 8 significant bits for exponents >= -126 and a fixed
 * quantum of 2^-133 below (subnormals). The rounded value is exactly a
 * float, whose upper 16 bits are the bf16 encoding. */
uint16_t fo_bf16_rne(double x) {
    const double a = fabs(x);
    double r = 0.0;
    if (a > 0.0) {
        int e2;
        frexp(a, &e2);                       /* a = f * 2^e2, f in [0.5, 1)  */
        const int e = e2 - 1;                /* a in [2^e, 2^(e+1))          */
        const double quantum = ldexp(1.0, (e < -126 ? -126 : e) - 7);
        const double n = a / quantum;        /* exact: a power-of-two scale  */
        double k = floor(n);
        const double frac = n - k;           /* exact                        */
        if (frac > 0.5 || (frac == 0.5 && fmod(k, 2.0) != 0.0)) k += 1.0;
        r = k * quantum;                     /* exact, representable as float */
    }
    float f = (float)r;
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    if (signbit(x)) bits |= 0x80000000u;
    return (uint16_t)(bits >> 16);
}

/* Compressed keys g0 .. g1-1 of one request as bf16 bits: the pooled and
 * normalized key of fo_index_keys_pool (double), rounded once to bf16 --
 * the "compressed keys are bf16 before they are quantized" reading;
 * out[(g - g0) * d + i]. */
void fo_index_keys_build_bf16(const uint16_t* raw, int64_t rs, int64_t d, int64_t g0,
                              int64_t g1, uint16_t* out) {
    double k[512];
    for (int64_t g = g0; g < g1; ++g) {
        fo_index_keys_pool(raw, rs, d, g, g + 1, k);
        for (int64_t i = 0; i < d; ++i) out[(g - g0) * d + i] = fo_bf16_rne(k[i]);
    }
}
