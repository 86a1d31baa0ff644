/*
 * e4m3.c -- FP8 codec of the oracle (test infrastructure only).
 *
 * The value of every code is built from its bit fields as the OCP OFP8
 * specification defines them; encoding picks, by exhaustive comparison, the
 * representable magnitude nearest to |f| and breaks exact ties toward the
 * code whose mantissa LSB is 0 (round-to-nearest-even, the rounding the
 * FreeToken fix commit names for its reference quantizer). Out-of-range
 * magnitudes saturate to the largest finite value: a row scale of
 * amax / FP8 max never needs it ([ATOM] description, K/V bullet: with a
 * scale taken from each row, no value leaves the format's range), so saturation only decides what a caller that
 * passes larger values gets.
 *
 * Parity pins: decode table against torch's float8_e4m3fn / float8_e5m2
 * views of all 256 codes; encode against torch's RNE casts inside the
 * finite range, and against the closed forms max 448, min normal 2^-6,
 * worst-case relative error 1/17 (e4m3) and 1/9 (e5m2).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "oracle.h"

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs float arithmetic evaluated in float (FLT_EVAL_METHOD 0)"
#endif

/* Field widths of the two formats [OFP8]. */
static int exp_bits(int fmt) { return fmt == FO_E4M3 ? 4 : 5; }
static int man_bits(int fmt) { return fmt == FO_E4M3 ? 3 : 2; }
static int bias(int fmt) { return fmt == FO_E4M3 ? 7 : 15; }

/* Value of one code, read field by field [OFP8]. */
double fo_decode(int fmt, unsigned code) {
    const int eb = exp_bits(fmt), mb = man_bits(fmt);
    const unsigned sign = (code >> 7) & 1u;
    const unsigned e = (code >> mb) & ((1u << eb) - 1u);
    const unsigned m = code & ((1u << mb) - 1u);
    const unsigned emax_field = (1u << eb) - 1u;
    double mag;
    if (fmt == FO_E4M3) {
        /* E4M3: no infinities; only S.1111.111 is NaN. */
        if (e == emax_field && m == ((1u << mb) - 1u)) return NAN;
    } else {
        /* E5M2: all-ones exponent is inf (m == 0) or NaN (m != 0). */
        if (e == emax_field) {
            if (m != 0) return NAN;
            return sign ? -INFINITY : INFINITY;
        }
    }
    if (e == 0) {
        /* subnormal: 2^(1 - bias) * m / 2^mb */
        mag = ldexp((double)m / (double)(1u << mb), 1 - bias(fmt));
    } else {
        mag = ldexp(1.0 + (double)m / (double)(1u << mb), (int)e - bias(fmt));
    }
    return sign ? -mag : mag;
}

/* The non-negative half of each format's table (codes 0..127), filled once
 * from fo_decode when the library is loaded. */
static double g_table[2][128];

__attribute__((constructor)) static void build_tables(void) {
    for (int fmt = 0; fmt < 2; ++fmt)
        for (unsigned c = 0; c < 128; ++c) g_table[fmt][c] = fo_decode(fmt, c);
}

/* Largest finite magnitude: found by scanning the table, not assumed. */
double fo_fmt_max(int fmt) {
    double best = 0.0;
    for (unsigned c = 0; c < 128; ++c) {
        const double v = g_table[fmt][c];
        if (isfinite(v) && v > best) best = v;
    }
    return best;
}

/* Nearest finite non-negative code to magnitude a (a >= 0, finite), ties to
 * the even code. Every finite code is compared; nothing assumes order. */
static unsigned nearest_magnitude_code(int fmt, double a) {
    unsigned best = 0;
    double best_err = INFINITY;
    for (unsigned c = 0; c < 128; ++c) {
        const double v = g_table[fmt][c];
        if (!isfinite(v)) continue;
        const double err = fabs(v - a);      /* exact: both are short binaries */
        if (err < best_err || (err == best_err && (c & 1u) == 0u)) {
            best = c;
            best_err = err;
        }
    }
    return best;
}

unsigned fo_encode(int fmt, float f) {
    if (isnan(f)) return 0x7Fu;          /* a NaN code in both formats */
    const unsigned sign = signbit(f) ? 0x80u : 0x00u;
    double a = fabs((double)f);
    const double mx = fo_fmt_max(fmt);
    if (a > mx) a = mx;                                      /* saturate */
    return sign | nearest_magnitude_code(fmt, a);
}

void fo_encode_array(int fmt, const float* in, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)fo_encode(fmt, in[i]);
}

void fo_decode_array(int fmt, const uint8_t* in, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = fo_decode(fmt, in[i]);
}

/* bfloat16 is the upper half of an IEEE binary32: widening is exact. */
float fo_bf16_to_f32(uint16_t bits) {
    const uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return f;
}
