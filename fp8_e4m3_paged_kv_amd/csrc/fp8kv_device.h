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

// E4M3 (OCP E4M3FN) code of a finite fp32 value: round to nearest, ties to
// the even code, magnitudes above 448 saturate to 448. Both rounding ranges
// are computed and selected, so the wave never diverges.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
    const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
    const float a = fminf(fabsf(q), kE4M3Max);
    // normal range (a >= 2^-6): round the fp32 mantissa to 3 bits
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    const uint32_t normal = (b >> 20) - (120u << 3);   // rebias 127 -> 7
    // subnormal range (a < 2^-6): integer multiple of 2^-9, nearest even
    const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
    return sign | (a >= 0x1p-6f ? normal : sub);
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

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    f16x2 r = {(_Float16)a, (_Float16)b};   // round to nearest even
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Transpose a 4 x 4 byte block: rows a..d (one dword each) -> columns.
// c[i] holds byte i of a, b, c, d in bytes 0..3.
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c,
                                             uint32_t d, uint32_t out[4]) {
    const uint32_t ab_lo = perm(b, a, 0x05010400u);   // a0 b0 a1 b1
    const uint32_t ab_hi = perm(b, a, 0x07030602u);   // a2 b2 a3 b3
    const uint32_t cd_lo = perm(d, c, 0x05010400u);   // c0 d0 c1 d1
    const uint32_t cd_hi = perm(d, c, 0x07030602u);   // c2 d2 c3 d3
    out[0] = perm(cd_lo, ab_lo, 0x05040100u);         // a0 b0 c0 d0
    out[1] = perm(cd_lo, ab_lo, 0x07060302u);         // a1 b1 c1 d1
    out[2] = perm(cd_hi, ab_hi, 0x05040100u);         // a2 b2 c2 d2
    out[3] = perm(cd_hi, ab_hi, 0x07060302u);         // a3 b3 c3 d3
}

}  // namespace fp8kv
