// fp8kv_device.h -- device helpers of the gfx950 FP8 KV kernels.
//
// Wave64 lane tricks (DPP row reductions), the E4M3 encoder used by the
// quantizer, the exact E4M3 -> bf16 / fp16 widening used by the decode
// kernel (hardware v_cvt_scalef32_pk_{bf16,f16}_fp8 with unit scale: every
// E4M3 value is exactly representable in both), and an 8 x 4 byte
// transpose built from v_perm_b32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8kv {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;
constexpr int kBufferWord3 = 0x00020000;   // gfx9 raw buffer descriptor flags (32-bit data format)

// Raw buffer descriptor over [base, base + bytes): loads past the end read
// 0, stores past the end are dropped (the range check covers the VGPR
// offset; keep the SGPR offset 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferWord3);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) {
    return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
    return __uint_as_float(w & 0xFFFF0000u);
}

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15). Inputs are
// non-negative floats, so their bit patterns order like unsigned integers.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false)); // row_ror:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false)); // row_ror:8
    return v;
}

// Four fp32 values -> four E4M3 codes (bytes 0..3), round to nearest even,
// magnitudes above 448 saturating to +-448: the gfx950 OCP converter after
// a clamp (the quantizer's quotients never exceed 448 * (1 + 2^-23)).
__device__ __forceinline__ uint32_t e4m3x4_encode(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
    b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
    c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
    d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Four fp32 values -> four E5M2 codes, round to nearest even, magnitudes
// above 57344 saturating to +-57344 (the gfx950 OCP converter after a clamp).
constexpr float kE5M2Max = 57344.0f;
__device__ __forceinline__ uint32_t e5m2x4_encode(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -kE5M2Max, kE5M2Max);
    b = __builtin_amdgcn_fmed3f(b, -kE5M2Max, kE5M2Max);
    c = __builtin_amdgcn_fmed3f(c, -kE5M2Max, kE5M2Max);
    d = __builtin_amdgcn_fmed3f(d, -kE5M2Max, kE5M2Max);
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    return (uint32_t)w;
}

// q[i] = x[i] / scale for every element of a row, each the correctly rounded
// quotient: one IEEE reciprocal of the scale and one FMA correction per
// element (Markstein): q0 = x*r, e = x - q0*s (exact), q = q0 + e*r, with
// the sign of x restored (the correction turns -0 into +0). A zero scale
// divides by 1 (the row's codes are then the signed zeros of x). Scales
// below 2^-100 are first multiplied by 2^64, as are their elements (exact),
// so the reciprocal stays finite; that path is taken by the whole wave.
// Checked exhaustively: for every bf16 row maximum and every bf16 element of
// either sign up to it in magnitude, the E4M3 code of q equals that of the
// IEEE quotient.
template <int N>
__device__ __forceinline__ void row_quotients(const float (&x)[N], float scale, float (&q)[N]) {
#pragma clang fp contract(off)
    if (__builtin_expect(__any(scale < 0x1p-100f && scale != 0.0f), 0)) {
        const float f = scale < 0x1p-100f ? 0x1p64f : 1.0f;
        const float ss = scale == 0.0f ? 1.0f : scale * f;
        const float rcp = 1.0f / ss;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float xs = scale == 0.0f ? x[i] : x[i] * f;
            const float q0 = xs * rcp;
            const float e = __builtin_fmaf(-q0, ss, xs);
            q[i] = __builtin_copysignf(__builtin_fmaf(e, rcp, q0), x[i]);
        }
    } else {
        const float ss = scale == 0.0f ? 1.0f : scale;
        const float rcp = 1.0f / ss;                 // IEEE binary32 division
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float q0 = x[i] * rcp;
            const float e = __builtin_fmaf(-q0, ss, x[i]);
            q[i] = __builtin_copysignf(__builtin_fmaf(e, rcp, q0), x[i]);
        }
    }
}

// The E4M3 row quantizer of one (token, KV head) row held by a 16-lane DPP
// row (EPL elements per lane, each exactly a bf16 value): amax over the
// row, scale = fp32(amax / 448) by IEEE division, each code the E4M3 RNE of
// the correctly rounded quotient x / scale (x itself when the scale is 0),
// 4 codes per packed word. Every kernel that writes cache rows uses this.
template <int EPL>
__device__ __forceinline__ void quantize_row_e4m3(const float (&x)[EPL], float& scale,
                                                  uint32_t (&packed)[EPL / 4]) {
#pragma clang fp contract(off)
    uint32_t amax_bits = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) amax_bits = max(amax_bits, __float_as_uint(x[i]) & 0x7FFFFFFFu);
    amax_bits = row16_max_u32(amax_bits);
    const float amax = __uint_as_float(amax_bits);
    scale = amax / kE4M3Max;                  // IEEE binary32 division
    float qv[EPL];
    row_quotients(x, scale, qv);
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i)
        packed[i] = e4m3x4_encode(qv[4 * i], qv[4 * i + 1], qv[4 * i + 2], qv[4 * i + 3]);
}

// Two E4M3 codes (16-bit half HI of w) -> two bf16, exact.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}
// Two E4M3 codes (16-bit half HI of w) -> two fp16, exact.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    f16x2 r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// 8 codes (two dwords) -> 8 bf16 in order.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    uint32_t r[4] = {e4m3x2_to_bf16x2<false>(lo), e4m3x2_to_bf16x2<true>(lo),
                     e4m3x2_to_bf16x2<false>(hi), e4m3x2_to_bf16x2<true>(hi)};
    return __builtin_bit_cast(bf16x8, r);
}
// 8 codes (two dwords) -> 8 fp16 in order.
__device__ __forceinline__ f16x8 e4m3x8_to_f16x8(uint32_t lo, uint32_t hi) {
    uint32_t r[4] = {e4m3x2_to_f16x2<false>(lo), e4m3x2_to_f16x2<true>(lo),
                     e4m3x2_to_f16x2<false>(hi), e4m3x2_to_f16x2<true>(hi)};
    return __builtin_bit_cast(f16x8, r);
}

// The same for E5M2 codes (OCP E5M2: every finite value is exact in bf16
// and in fp16, of which it is the top byte).
template <bool HI>
__device__ __forceinline__ uint32_t e5m2x2_to_bf16x2(uint32_t w) {
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}
template <bool HI>
__device__ __forceinline__ uint32_t e5m2x2_to_f16x2(uint32_t w) {
    f16x2 r = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ bf16x8 e5m2x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    uint32_t r[4] = {e5m2x2_to_bf16x2<false>(lo), e5m2x2_to_bf16x2<true>(lo),
                     e5m2x2_to_bf16x2<false>(hi), e5m2x2_to_bf16x2<true>(hi)};
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    f16x2 r = {(_Float16)a, (_Float16)b};   // round to nearest even
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

}  // namespace fp8kv
