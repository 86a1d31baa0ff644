/*
 * Exhaustive check of the quantizer's quotient on the CPU.
 *
 * The kernel forms x / s (s = fp32(amax / 448)) from one IEEE reciprocal r
 * of s and one FMA correction:  q0 = x*r,  e = fma(-q0, s, x),
 * q = copysign(fma(e, r, q0), x)  -- with x and s first scaled by 2^64 when
 * s < 2^-100 so r stays finite. This program runs that exact sequence of
 * IEEE binary32 operations for EVERY positive bf16 row maximum a and EVERY
 * bf16 x with |x| <= a, both signs (so -0 too: without the copysign the
 * correction turns -0 into +0), and counts the pairs whose E4M3
 * round-to-nearest-even code differs from the code of the correctly rounded
 * quotient x / s. The E4M3 encoder here is a plain nearest-value search over
 * the code table, independent of the kernel's bit-level encoder.
 *
 * Prints "pairs=<n> code_diffs=<n>"; exit status 0 iff code_diffs == 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bf16(uint32_t b) { uint32_t w = b << 16; float f; memcpy(&f, &w, 4); return f; }

static double table[127];           /* non-negative finite E4M3 values */

static unsigned nearest_code(float q) {
    double a = fabs((double)q);
    if (a > 448.0) a = 448.0;
    unsigned best = 0;
    double be = INFINITY;
    for (unsigned c = 0; c < 127; ++c) {
        double e = fabs(table[c] - a);
        if (e < be || (e == be && (c & 1u) == 0)) { be = e; best = c; }
    }
    return (signbit(q) ? 0x80u : 0u) | best;
}

int main(void) {
    for (unsigned c = 0; c < 127; ++c) {
        unsigned e = c >> 3, m = c & 7;
        table[c] = e ? ldexp(1.0 + m / 8.0, (int)e - 7) : ldexp(m / 8.0, -6);
    }
    long long pairs = 0, diffs = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, diffs)
    for (int ab = 1; ab < 0x7F80; ++ab) {
        const float a = from_bf16((uint32_t)ab);
        const float s = a / 448.0f;
        const float f = s < 0x1p-100f ? 0x1p64f : 1.0f;
        const float ss = s * f;
        const float r = 1.0f / ss;
        float last_q, last_q1;
        for (int sign = 0; sign < 2; ++sign) {
            last_q = last_q1 = -1.0f;
            for (int xb = 0; xb <= ab; ++xb) {
                const float x = from_bf16((uint32_t)xb | (sign ? 0x8000u : 0u));
                const float xs = x * f;
                const float q0 = xs * r;
                const float e = fmaf(-q0, ss, xs);
                const float q1 = copysignf(fmaf(e, r, q0), x);
                const float q = x / s;
                ++pairs;
                /* same bits as the previous pair: same codes */
                if (memcmp(&q, &last_q, 4) == 0 && memcmp(&q1, &last_q1, 4) == 0) continue;
                last_q = q;
                last_q1 = q1;
                if (memcmp(&q, &q1, 4) != 0 && nearest_code(q) != nearest_code(q1)) ++diffs;
            }
        }
    }
    printf("pairs=%lld code_diffs=%lld\n", pairs, diffs);
    return diffs == 0 ? 0 : 1;
}
