// index_score.hip -- compressed-index keys and the decode-sized index scorer
// ("fix(qwen4-exp): register the QSA FP8 scale planes for KV offload",
// ROCm/ATOM #2655, description: the compressed-index bullet and the stacked
// decode scorer paragraph).
//
// Keys. A compressed index key (head_dim 128) is stored either as E4M3
// codes with one fp32 scale (the KV cache's row quantizer), or as MXFP4:
// 64 bytes of E2M1 pairs (element 2j in the low nibble of byte j) and one
// E8M0 exponent per 32 dims, the exponent the smallest e with
// amax <= 6 * 2^e so that no group clips; each element is x / 2^e rounded
// to the nearest E2M1 value, ties to the even code, sign kept.
//
// Scorer. For request b, query row r and key n:
//     score[b, r, n] = sum_h w[b, r, h] * max(0, q[b, r, h, :] . k^[b, n, :])
// One v_mfma_f32_16x16x32_bf16 chain (4 k-steps over 128 dims) multiplies
// the 16 index heads of one query row (M) by 16 keys (N, widened exactly to
// bf16 once per tile and shared by every row of the wave): the heads fill
// the MFMA rows, as rows x heads do in the page's stacked scorer. Lane
// (g, i) then holds the dots of heads 4g .. 4g+3 with key i; the ReLU and
// the head weights are applied in the lane, and four rows at a time are
// summed over the four lane groups by two cross-lane swaps
// (v_permlane32_swap, v_permlane16_swap), which leave row 4c + g of the
// quad in lane group g. E4M3 key scales are >= 0, so they multiply the
// summed score; MXFP4 exponents vary along the dims and are folded into the
// widened keys (E2M1 * 2^e is exact in bf16). The ReLU and head weights cost
// two VALU ops per (row, head, key), which bounds the kernel together with
// the MFMAs: on gfx950 a wave's own vector instructions beside its MFMAs
// overlap them only in part.
#include <hip/hip_runtime.h>

#include "fp8kv_device.h"
#include "fp8kv_internal.h"

namespace fp8kv {
namespace {

constexpr int kScoreWaves = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStoreNT = 2;         // cache policy of the score stores: non-temporal

// ---------------------------------------------------------------- keys
// Encode one key held by a 16-lane DPP row: lane li holds dims 8li .. 8li+7
// as floats (each exactly a bf16 value). E4M3: the KV row quantizer (row
// amax, IEEE amax/448, correctly rounded quotients, RNE + saturating
// encode), codes at code_row + 8li, the scale by lane 0. MXFP4: a group of
// 32 dims is one quad of lanes; 4 code bytes per lane at code_row + 4li,
// the group's E8M0 code by the quad's first lane. BF16: the values
// themselves, 16 bytes per lane. Nothing is stored when `store` is false.
template <int FMT>
__device__ __forceinline__ void encode_key(const float (&x)[8], int li, bool store,
                                           uint8_t* code_row, void* scale_row) {
#pragma clang fp contract(off)
    if (FMT == kKeysBF16) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (__float_as_uint(x[2 * i]) >> 16) | (__float_as_uint(x[2 * i + 1]) & 0xFFFF0000u);
        if (store) *reinterpret_cast<uint4*>(code_row + li * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        return;
    }
    if (FMT == kKeysE4M3) {
        float scale;
        uint32_t packed[2];
        quantize_row_e4m3<8>(x, scale, packed);      // the KV row quantizer
        if (store) {
            *reinterpret_cast<uint2*>(code_row + li * 8) = make_uint2(packed[0], packed[1]);
            if (li == 0) *static_cast<float*>(scale_row) = scale;
        }
    } else {
        uint32_t amax_bits = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax_bits = max(amax_bits, __float_as_uint(x[i]) & 0x7FFFFFFFu);
        amax_bits = max(amax_bits, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax_bits, 0xB1, 0xF, 0xF, false));
        amax_bits = max(amax_bits, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax_bits, 0x4E, 0xF, 0xF, false));
        const float amax = __uint_as_float(amax_bits);
        int e = 0;
        if (amax > 0.0f) {
            int ex;
            const float mant = frexpf(amax, &ex);       // amax = mant * 2^ex, mant in [.5, 1)
            e = mant <= 0.75f ? ex - 3 : ex - 2;         // smallest e with amax <= 6 * 2^e
            e = max(e, -127);
        }
        // v = x / 2^e (exact wherever a code boundary lies), then the
        // hardware E2M1 converter with unit scale: round to nearest even,
        // sign kept; element 2j in the low nibble of byte j
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = ldexpf(x[i], -e);
        uint32_t packed = 0;
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[0], v[1], 1.0f, 0);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[2], v[3], 1.0f, 1);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[4], v[5], 1.0f, 2);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[6], v[7], 1.0f, 3);
        if (store) {
            *reinterpret_cast<uint32_t*>(code_row + li * 4) = packed;
            if ((li & 3) == 0) static_cast<uint8_t*>(scale_row)[li >> 2] = (uint8_t)(e + 127);
        }
    }
}

// One 16-lane DPP row per key (8 bf16 per lane), 4 keys per wave step, two
// steps, four waves: 32 keys per workgroup.
template <int FMT>
__global__ __launch_bounds__(256) void index_keys_kernel(IndexKeysParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane >> 4;
    const int li = lane & 15;
    const int64_t key0 = (int64_t)blockIdx.x * 32 + wave * 8;
    uint4 raw[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int64_t key = min(key0 + 4 * s + sub, p.num_keys - 1);
        raw[s] = *reinterpret_cast<const uint4*>(p.keys + key * p.key_stride + li * 8);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int64_t key = key0 + 4 * s + sub;
        const uint32_t wds[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(wds[i]);
            x[2 * i + 1] = bf16_hi(wds[i]);
        }
        const int64_t k = min(key, p.num_keys - 1);
        encode_key<FMT>(x, li, key < p.num_keys, p.codes + k * p.code_stride,
                        FMT == kKeysE4M3
                            ? (void*)(static_cast<float*>(p.scales) + k * p.scale_stride)
                            : (void*)(static_cast<uint8_t*>(p.scales) + k * p.scale_stride));
    }
}

// Sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    return v;
}

// Index-key builder: compressed key g of request b is the mean of raw keys
// 4g .. 4g+3, L2-normalized and rounded to bf16, then encoded as above.
// One 16-lane row per compressed key (its lanes read 8 dims of each of the
// 4 raw keys), 32 keys per workgroup; grid y = request.
template <int FMT>
__global__ __launch_bounds__(256) void index_keys_build_kernel(IndexBuildParams p) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane >> 4;
    const int li = lane & 15;
    const int b = blockIdx.y;
    const int64_t gi0 = (int64_t)blockIdx.x * 32 + wave * 8;
    const int64_t ng = p.g1 - p.g0;
    const uint16_t* raw_b = p.raw + (int64_t)b * p.raw_stride_b;
    uint4 raw[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int64_t g = p.g0 + min(gi0 + 4 * s + sub, ng - 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                raw_b + (4 * g + t) * p.raw_stride_tok + li * 8));
            raw[s][t] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int64_t gi = gi0 + 4 * s + sub;
        float m[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w0 = (&raw[s][0].x)[i], w1 = (&raw[s][1].x)[i];
            const uint32_t w2 = (&raw[s][2].x)[i], w3 = (&raw[s][3].x)[i];
            m[2 * i] = ((bf16_lo(w0) + bf16_lo(w1)) + (bf16_lo(w2) + bf16_lo(w3))) * 0.25f;
            m[2 * i + 1] = ((bf16_hi(w0) + bf16_hi(w1)) + (bf16_hi(w2) + bf16_hi(w3))) * 0.25f;
        }
        // scale the mean by a power of two that brings its largest element
        // to [0.5, 1) (exact), so the sum of squares neither underflows nor
        // overflows; the normalized key does not depend on the scale
        uint32_t amax_bits = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax_bits = max(amax_bits, __float_as_uint(m[i]) & 0x7FFFFFFFu);
        int ex = 0;
        frexpf(__uint_as_float(row16_max_u32(amax_bits)), &ex);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            m[i] = ldexpf(m[i], -ex);
            ss = __builtin_fmaf(m[i], m[i], ss);
        }
        const float n = __builtin_sqrtf(row16_sum(ss));
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float c = n > 0.f ? m[i] / n : 0.f;
            x[i] = (float)(__bf16)c;                      // round to nearest even
        }
        const int64_t g = p.g0 + min(gi, ng - 1);
        uint8_t* code_row = p.codes + (int64_t)b * p.code_stride_b + g * p.code_stride_key;
        void* scale_row = FMT == kKeysE4M3
                              ? (void*)(static_cast<float*>(p.scales) + (int64_t)b * p.scale_stride_b +
                                        g * p.scale_stride_key)
                              : (void*)(static_cast<uint8_t*>(p.scales) + (int64_t)b * p.scale_stride_b +
                                        g * p.scale_stride_key);
        encode_key<FMT>(x, li, gi < ng, code_row, scale_row);
    }
}

// ---------------------------------------------------------------- scorer
// A 16-key tile, widened to the bf16 B operand of four k-steps. Lane
// (g, i): key i of the tile, dims [32g, 32g + 32); k-step k takes dims
// 32g + 8k .. +7, and q is read with the same permutation of the dims.
// Loads go through buffer descriptors bounded by the request's keys: keys
// past the end read as 0 and are never stored.
template <int FMT>
struct KeyTile {
    uint4 raw[2];        // E4M3: the lane's 32 code bytes; MXFP4: 16 packed bytes in raw[0]
    uint32_t exp;        // MXFP4: E8M0 code of group g of key i
    float kscale;        // E4M3: scale of key i

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t srs,
                                         uint32_t koff, uint32_t soff) {
        typedef int intx4 __attribute__((ext_vector_type(4)));
        const intx4 a = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)koff, 0, 0);
        raw[0] = make_uint4(a[0], a[1], a[2], a[3]);
        if (FMT == kKeysE4M3) {
            const intx4 c = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)koff + 16, 0, 0);
            raw[1] = make_uint4(c[0], c[1], c[2], c[3]);
            kscale = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, (int)soff, 0, 0));
        } else {
            exp = __builtin_amdgcn_raw_buffer_load_b8(srs, (int)soff, 0, 0);
        }
    }

    __device__ __forceinline__ void widen(bf16x8 (&kb)[4]) const {
        if (FMT == kKeysE4M3) {
            kb[0] = e4m3x8_to_bf16x8(raw[0].x, raw[0].y);
            kb[1] = e4m3x8_to_bf16x8(raw[0].z, raw[0].w);
            kb[2] = e4m3x8_to_bf16x8(raw[1].x, raw[1].y);
            kb[3] = e4m3x8_to_bf16x8(raw[1].z, raw[1].w);
        } else {
            // 2^(exp - 127) as an fp32 scale (code 0 is the subnormal 2^-127)
            const float s = exp == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(exp << 23);
            const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // one dword = 8 E2M1 codes = dims 32g + 8k .. +7, element 2j in the low nibble
                uint32_t h[4];
                h[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[k], s, 0));
                h[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[k], s, 1));
                h[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[k], s, 2));
                h[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[k], s, 3));
                kb[k] = __builtin_bit_cast(bf16x8, h);
            }
        }
    }
};

// a and b exchanged between the lower and upper 32 lanes, then summed: the
// lower half holds a(l) + a(l + 32), the upper half b(l - 32) + b(l).
__device__ __forceinline__ float swap32_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same between 16-lane rows 2c and 2c + 1: row 2c holds a(l) + a(l + 16),
// row 2c + 1 holds b(l - 16) + b(l).
__device__ __forceinline__ float swap16_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(x, 0) on the bit pattern: negative floats are negative integers. One
// integer max, where a float max needs its operand canonicalized first.
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// A tile's parity within its key chunk as a type: the loops are unrolled so
// that every step's parity, and so its store count, is known at compile time.
template <bool B>
struct Parity {
    static constexpr bool value = B;
};

// Byte offset that every store range check rejects (request spans are
// below 2^30 bytes, so the sum of two such offsets is rejected too).
constexpr uint32_t kDropped = 0x40000000u;

// Rows x heads stacking. With HP index heads per row (H padded up to a
// power of two, HP <= 16), one 16-row MFMA tile stacks RPT = 16 / HP query
// rows x HP heads: M-row m is row m / HP, head m % HP ("4 rows x 4 index
// heads into one M = 16 operand" for HP = 4). A wave carries NT such tiles
// (NT * RPT rows: 8 rows at HP = 16, 16 at HP = 8, 32 below), in two halves
// of NT / 2 tiles whose MFMAs and epilogues alternate. Lane (g, i) of a
// tile's result holds M-rows 4g .. 4g+3 for key i, so the ReLU and the
// weights of those 4 (row, head) pairs are applied in the lane; then
//   HP = 16: the 4 lane groups hold quarters of one row: 4 tiles are summed
//            by two swaps (v_permlane32_swap, v_permlane16_swap), leaving
//            tile 4c + g's row in lane group g;
//   HP = 8:  pairs of lane groups hold halves of a row: tiles 2v, 2v+1 are
//            summed by one v_permlane16_swap;
//   HP = 4:  lane group g holds row g of the tile whole;
//   HP = 2, 1: lane group g holds 2 or 4 rows whole.
// Every half thus ends with OS = NT * RPT / 8 "slots": one value per lane,
// lane group g holding the scores of one row for the tile's 16 keys, which
// one 4-byte store per lane writes (64 bytes per lane group).
template <int HP>
struct Stack {
    static constexpr int RPT = 16 / HP;                  // rows per MFMA tile
    static constexpr int NT = RPT <= 4 ? 8 : 32 / RPT;   // MFMA tiles per wave
    static constexpr int NH = NT / 2;                    // tiles per half
    static constexpr int ROWS = NT * RPT;                // rows per wave
    static constexpr int OS = ROWS / 8;                  // store slots per half
    // wave-relative row of slot s of half c in lane group g, as a part that
    // depends on the lane group and a wave-uniform part:
    //   HP = 16: tile 4c + g;               HP = 8: tile 4c + 2s + (g & 1), row g >> 1;
    //   HP = 4:  tile 4c + s, row g;        HP = 2: tile 2c + s/2, row 2g + s%2;
    //   HP = 1:  tile c, row 4g + s
    static __device__ __forceinline__ int lane_row(int g) {
        if (HP == 16 || HP == 4) return g;
        if (HP == 8) return 2 * (g & 1) + (g >> 1);
        return (16 / HP / 4) * g;
    }
    static constexpr int uniform_row(int c, int s) {
        return HP == 16 ? 4 * c
             : HP == 8  ? 8 * c + 4 * s
             : HP == 4  ? 16 * c + 4 * s
             : HP == 2  ? 16 * c + 8 * (s >> 1) + (s & 1)
                        : 16 * c + s;
    }
};

// Workgroup = 4 waves x Stack<HP>::ROWS query rows of one request and one
// chunk of its keys; each wave scores its rows against every 16-key tile of
// the chunk. The row groups of one (request, chunk) are placed on one XCD,
// so their key reads meet in that XCD's L2. The tile loop has no branch:
// loads past the chunk read in-bounds keys or zeros, stores of rows and keys
// outside the output carry an offset the range check drops. Key loads run
// two tiles ahead (three register buffers), and the MFMAs of each half of
// the tiles are issued next to the other half's epilogue, which does not
// depend on them, so the matrix core and the vector ALU work side by side.
template <int FMT, int HP, bool ROT>
__global__ __launch_bounds__(256, 2) void index_score_kernel(IndexScoreParams p) {
    typedef Stack<HP> S;
    constexpr int NT = S::NT, NH = S::NH, OS = S::OS;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lg = lane >> 4;

    int bid = blockIdx.x;
    const int m = p.row_groups;
    if (m > 1) {
        const int xcd = bid & 7, k = bid >> 3;
        bid = (k / m) * 8 * m + xcd * m + (k % m);
    }
    const int rg = bid % m;
    const int bc = bid / m;
    const int ck = bc % p.chunks;
    const int b = bc / p.chunks;
    if (b >= p.batch) return;
    const int row0 = (rg * kScoreWaves + wave) * S::ROWS;
    const int n_begin = ck * p.key_chunk;
    const int n_end = min(n_begin + p.key_chunk, p.num_keys);
    if (row0 >= p.rows || n_begin >= n_end) return;

    // q (A operand) of tile j: lane (g, i) holds M-row i = (row j*RPT + i/HP,
    // head i%HP), dims [32g, 32g + 32); w of M-rows 4g .. 4g+3
    bf16x8 qa[NT][4];
    float wv[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int row = row0 + j * S::RPT + li / HP;
        const int head = li % HP;
        if (row < p.rows && head < p.heads) {
            const uint16_t* qp = p.q + (int64_t)b * p.q_stride_b + (int64_t)row * p.q_stride_row +
                                 (int64_t)head * p.q_stride_head + 32 * lg;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                qa[j][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 8 * k));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) qa[j][k] = bf16x8{};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int wrow = row0 + j * S::RPT + (4 * lg + r) / HP;
            const int whead = (4 * lg + r) % HP;
            wv[j][r] = wrow < p.rows && whead < p.heads
                           ? p.w[(int64_t)b * p.w_stride_b + (int64_t)wrow * p.w_stride_row +
                                 (int64_t)whead * p.w_stride_head]
                           : 0.0f;
        }
    }

    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(p.codes + (int64_t)b * p.codes_stride_b, p.key_bytes);
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(p.scales + (int64_t)b * p.scales_stride_b, p.scale_bytes);
    const __amdgpu_buffer_rsrc_t ors =
        make_rsrc(p.out + (int64_t)b * p.out_stride_b, p.out_bytes);
    const uint32_t kstep = 16u * (uint32_t)p.codes_stride_key;
    const uint32_t sstep = 16u * (uint32_t)p.scales_stride_key;
    uint32_t koff = (uint32_t)(n_begin + li) * (uint32_t)p.codes_stride_key +
                    (FMT == kKeysE4M3 ? 32u : 16u) * lg;
    uint32_t soff = (uint32_t)(n_begin + li) * (uint32_t)p.scales_stride_key +
                    (FMT == kKeysE4M3 ? 0u : (uint32_t)lg);
    // ROT: wave w starts 128 w keys into the chunk (whole 32-key pairs) and
    // wraps around, so the rows of a workgroup write four column regions at
    // a time instead of one; this spreads the stores of rows whose pitch is a
    // multiple of 64 KiB over more HBM channels, and the waves stay close
    // enough that each key line still comes from HBM about once. Virtual tile
    // v (v = 0, 16, ...) then holds keys key_of(v) .. + 15; without ROT
    // key_of(v) = n_begin + v.
    const int span32 = (n_end - n_begin + 31) & ~31;
    const int rot = ROT ? (128 * wave) % span32 : 0;
    auto key_of = [&](int v) { return ROT ? n_begin + (v + rot) % span32 : n_begin + v; };
    auto offs = [&](int v) {
        const uint32_t k = (uint32_t)(key_of(v) + li);
        koff = k * (uint32_t)p.codes_stride_key + (FMT == kKeysE4M3 ? 32u : 16u) * lg;
        soff = k * (uint32_t)p.scales_stride_key + (FMT == kKeysE4M3 ? 0u : (uint32_t)lg);
    };
    // byte offset of a slot's row: a per-lane part plus a wave-uniform one.
    // Rows do not overlap (row stride >= num_keys), so a row at or past
    // p.rows starts at or past the end of the request's scores and its
    // stores are dropped by the range check; the host keeps every such
    // offset below 2^31.
    const uint32_t s4 = (uint32_t)p.out_stride_row * 4u;
    // Tiles are stored in pairs (keys t .. t+31): one v_permlane16_swap of
    // a slot's even-tile and odd-tile values gives lanes 0..31 one row's 32
    // keys and lanes 32..63 another's, so every store writes whole 128-byte
    // lines (64-byte halves written apart cost extra HBM traffic). Lane
    // group g of the swapped pair holds the row of lane group g & 2 (first
    // store) or (g & 2) | 1 (second store), keys t + 16 (g & 1) + i.
    const uint32_t lb_x = (uint32_t)(row0 + S::lane_row(lg & 2)) * s4;
    const uint32_t lb_y = (uint32_t)(row0 + S::lane_row((lg & 2) | 1)) * s4;
    float hold[2][OS] = {};

    floatx4 acc0[NH], acc1[NH];
    auto mfma_half = [&](const bf16x8 (&kb)[4], int c, floatx4 (&acc)[NH]) {
#pragma unroll
        for (int t = 0; t < NH; ++t) {
            acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[NH * c + t][k], kb[k], acc[t], 0, 0, 0);
        }
    };
    // the ReLU and weights of the lane's (row, head) pairs, reduced to one
    // value per slot (one row per lane group), then stored
    auto epilogue = [&](const floatx4 (&acc)[NH], int c, float ks, auto odd_c, uint32_t ocol) {
        float v[OS];
        if constexpr (HP >= 4) {
            float s[NH];
#pragma unroll
            for (int t = 0; t < NH; ++t) {
                const float* wr = wv[NH * c + t];
                float x = relu(acc[t][0]) * wr[0];
                x = __builtin_fmaf(relu(acc[t][1]), wr[1], x);
                x = __builtin_fmaf(relu(acc[t][2]), wr[2], x);
                s[t] = __builtin_fmaf(relu(acc[t][3]), wr[3], x);
            }
            if constexpr (HP == 16) {
                v[0] = swap16_sum(swap32_sum(s[0], s[2]), swap32_sum(s[1], s[3]));
            } else if constexpr (HP == 8) {
                v[0] = swap16_sum(s[0], s[1]);
                v[1] = swap16_sum(s[2], s[3]);
            } else {
#pragma unroll
                for (int t = 0; t < NH; ++t) v[t] = s[t];
            }
        } else if constexpr (HP == 2) {
#pragma unroll
            for (int t = 0; t < NH; ++t) {
                const float* wr = wv[NH * c + t];
                v[2 * t] = __builtin_fmaf(relu(acc[t][1]), wr[1], relu(acc[t][0]) * wr[0]);
                v[2 * t + 1] = __builtin_fmaf(relu(acc[t][3]), wr[3], relu(acc[t][2]) * wr[2]);
            }
        } else {
            const float* wr = wv[c];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = relu(acc[0][r]) * wr[r];
        }
        if constexpr (!decltype(odd_c)::value) {
#pragma unroll
            for (int sl = 0; sl < OS; ++sl) hold[c][sl] = v[sl] * ks;
        } else {
#pragma unroll
            for (int sl = 0; sl < OS; ++sl) {
                const auto xy = __builtin_amdgcn_permlane16_swap(
                    __float_as_uint(hold[c][sl]), __float_as_uint(v[sl] * ks), false, false);
                const uint32_t u = (uint32_t)S::uniform_row(c, sl) * s4 + ocol;
                __builtin_amdgcn_raw_buffer_store_b32((int)xy[0], ors, (int)(lb_x + u), 0, kStoreNT);
                __builtin_amdgcn_raw_buffer_store_b32((int)xy[1], ors, (int)(lb_y + u), 0, kStoreNT);
            }
        }
    };
    // column of the lane in the swapped pair starting at key t
    auto colp = [&](int t) {
        if constexpr (ROT) {
            // t: virtual tile; the wrap never splits a pair
            const int k = key_of(t) + 16 * (lg & 1) + li;
            return t >= 0 && t < span32 && k < n_end ? (uint32_t)k * 4u : kDropped;
        } else {
            const int k = t + 16 * (lg & 1) + li;
            return k < n_end ? (uint32_t)k * 4u : kDropped;
        }
    };

    // one step: tile t's half-0 MFMAs overlap the previous tile's half-1
    // epilogue, tile t's half-1 MFMAs overlap its own half-0 epilogue; the
    // epilogue of an even tile (from the chunk's start) holds its values, that
    // of an odd tile stores the pair. The first step's previous tile is odd
    // and stores nothing (its column is the dropped offset).
    float ks_prev = 0.f;
    uint32_t ocol_prev = kDropped;
    auto step = [&](const KeyTile<FMT>& kt, int t, auto odd_c) {
        constexpr bool odd = decltype(odd_c)::value;
        bf16x8 kb[4];
        kt.widen(kb);
        const float ks = FMT == kKeysE4M3 ? kt.kscale : 1.0f;
        const uint32_t ocol = colp(t - 16);
        mfma_half(kb, 0, acc0);
        epilogue(acc1, 1, ks_prev, Parity<!odd>{}, ocol_prev);
        mfma_half(kb, 1, acc1);
        epilogue(acc0, 0, ks, odd_c, ocol);
        ks_prev = ks;
        ocol_prev = ocol;
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int t = 0; t < NH; ++t) acc1[t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // tiles n_begin, n_begin + 16, ... (with ROT virtual tiles 0, 16, ...)
    // and at least two more (their own stores all dropped) to drain the
    // pipeline and complete the last pair. Loads run two tiles ahead in three
    // buffers; the loop body is six tiles (buffer and parity both repeat),
    // then up to two three-tile bodies finish the chunk.
    KeyTile<FMT> ta, tb, tc;
    auto next = [&](int v) { offs(ROT ? v : v - n_begin); };
    auto body3 = [&](int v, auto p0) {
        constexpr bool e = decltype(p0)::value;
        next(v + 32);
        tc.load(krs, srs, koff, soff);
        step(ta, v, p0);
        next(v + 48);
        ta.load(krs, srs, koff, soff);
        step(tb, v + 16, Parity<!e>{});
        next(v + 64);
        tb.load(krs, srs, koff, soff);
        step(tc, v + 32, p0);
    };
    const int first = ROT ? 0 : n_begin;
    const int last = ROT ? span32 + 32 : n_end + 32;   // steps run while v < last
    offs(0);
    ta.load(krs, srs, koff, soff);
    next(first + 16);
    tb.load(krs, srs, koff, soff);
    int v = first;
    for (; v + 48 < last; v += 96) {
        body3(v, Parity<false>{});
        body3(v + 48, Parity<true>{});
    }
    if (v < last) body3(v, Parity<false>{});
}

template <int FMT, int HP>
hipError_t launch_score_hp(const IndexScoreParams& p, hipStream_t stream) {
    const int64_t m = p.row_groups;
    int64_t wgs = (int64_t)p.batch * p.chunks * m;
    if (m > 1) wgs = (wgs + 8 * m - 1) / (8 * m) * (8 * m);
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    if constexpr (HP <= 4) {
        if (p.rotate_keys) {
            hipLaunchKernelGGL((index_score_kernel<FMT, HP, true>), dim3((unsigned)wgs),
                               dim3(64 * kScoreWaves), 0, stream, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((index_score_kernel<FMT, HP, false>), dim3((unsigned)wgs),
                       dim3(64 * kScoreWaves), 0, stream, p);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_score(const IndexScoreParams& p, hipStream_t stream) {
    switch (index_heads_padded(p.heads)) {
        case 16: return launch_score_hp<FMT, 16>(p, stream);
        case 8: return launch_score_hp<FMT, 8>(p, stream);
        case 4: return launch_score_hp<FMT, 4>(p, stream);
        case 2: return launch_score_hp<FMT, 2>(p, stream);
        default: return launch_score_hp<FMT, 1>(p, stream);
    }
}

}  // namespace

hipError_t launch_index_keys(const IndexKeysParams& p, int key_format, hipStream_t stream) {
    const int64_t blocks = (p.num_keys + 31) / 32;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks), block(256);
    if (key_format == kKeysE4M3)
        hipLaunchKernelGGL((index_keys_kernel<kKeysE4M3>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((index_keys_kernel<kKeysMXFP4>), grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_index_keys_build(const IndexBuildParams& p, int key_format, hipStream_t stream) {
    const int64_t blocks = (p.g1 - p.g0 + 31) / 32;
    if (blocks > INT32_MAX || p.batch > 65535) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks, (unsigned)p.batch), block(256);
    if (key_format == kKeysE4M3)
        hipLaunchKernelGGL((index_keys_build_kernel<kKeysE4M3>), grid, block, 0, stream, p);
    else if (key_format == kKeysMXFP4)
        hipLaunchKernelGGL((index_keys_build_kernel<kKeysMXFP4>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((index_keys_build_kernel<kKeysBF16>), grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_index_score(const IndexScoreParams& p, int key_format, hipStream_t stream) {
    return key_format == kKeysE4M3 ? launch_score<kKeysE4M3>(p, stream)
                                   : launch_score<kKeysMXFP4>(p, stream);
}

}  // namespace fp8kv
