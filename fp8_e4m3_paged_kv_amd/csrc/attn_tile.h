// attn_tile.h -- the tile math of the decode split kernel
// (paged_decode.hip): E4M3 widening, the QK^T and PV MFMA tiles, the
// online softmax with the key scale on the score and the value scale
// folded into P; and the softmax state and lane reductions the
// chunked-prefill kernel (prefill_attn.hip) shares with it.
//
// Per 32-token tile (two 16-token halves s = 0, 1), lane l = 16*g + i:
//   QK^T  v_mfma_f32_16x16x32_bf16, A = K codes (token i, 8 head-dim slots
//         per k-step from the lane's D/4-byte chunk), B = q (row i, same
//         head-dim slots). Lane gets S[token 4g + r][row i], r = 0..3.
//   PV    v_mfma_f32_16x16x32_f16 computing O^T = V^T P^T: A = V codes
//         transposed in registers (head-dim column 8i + n for n-tile n, 8
//         tokens), B = P' (row i, the lane's 8 tokens). Lane accumulates
//         O[row i][d] for d = (D/16)(4g + r) + n: its own row, so the online
//         softmax rescale needs no cross-lane traffic.
//   P' = p * v_scale * 2^(141 - e) in fp16, where e is the running maximum
//   biased exponent of the value scales seen by the wave (floored at 15):
//   P' < 2^15 stays inside fp16's normal range, rescaling on a new exponent
//   is exact (a power of two), and the final 2^(e - 141) >= 2^-126 is a
//   normal float.
// Memory: each lane reads K as two/one 16-byte loads per token and V as 8
// (or 4) contiguous bytes per token: every 128-byte (64-byte) code row is
// read whole by 4 or 16 lanes. Tokens past a piece's end read zero through
// the buffer range check and are masked.
#pragma once

#include <hip/hip_runtime.h>

#include "fp8kv_device.h"
#include "fp8kv_internal.h"

namespace fp8kv {

constexpr float kNeg = -1.0e30f;     // "minus infinity" that keeps exp2 finite
// Cache policy of the K/V code loads: non-temporal. Every code byte is read
// once per launch; streaming them past the caches leaves L2 to the scale
// lines and block tables (decode workload: 367 -> 339 us).
constexpr int kCodesNT = 2;

__device__ __forceinline__ float pow2i(int e) {   // 2^e for e in [-126, 127]
    return __uint_as_float((uint32_t)(e + 127) << 23);
}

// Butterfly across the four 16-lane rows of a wave (xor 16, then xor 32)
// with the gfx950 row-swap instructions.
__device__ __forceinline__ float rows_max(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}


// IEEE-754 maximum (gfx950 v_maximum3_f32): unlike fmaxf it needs no
// NaN-quieting step on each operand; for the finite scores here the two
// agree (up to the sign of a zero maximum, which exp2 does not see).
__device__ __forceinline__ float fmax_fin(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float rows_max_fin(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmax_fin(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmax_fin(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Maximum over the four 16-lane rows for values that order as unsigned
// integers (non-negative floats).
__device__ __forceinline__ uint32_t rows_max_u32(uint32_t v) {
    auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max((uint32_t)a[0], (uint32_t)a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((uint32_t)b[0], (uint32_t)b[1]);
}

typedef int intx2 __attribute__((ext_vector_type(2)));
typedef int intx4 __attribute__((ext_vector_type(4)));

template <int DL>
struct VRow;
template <>
struct VRow<8> {
    typedef uint2 T;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int off) {
        intx2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCodesNT);
        return make_uint2((uint32_t)v[0], (uint32_t)v[1]);
    }
};
template <>
struct VRow<4> {
    typedef uint32_t T;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int off) {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCodesNT);
    }
};

__device__ __forceinline__ uint32_t vword(const uint2& v, int i) { return i ? v.y : v.x; }
__device__ __forceinline__ uint32_t vword(const uint32_t& v, int) { return v; }

// Per-wave online-softmax state: O^T accumulators of the lane's query row,
// running max (log2 units), partial sum of p over the lane's tokens, and the
// power-of-two range exponent of P'.
template <int DL>
struct WaveState {
    floatx4 acc[DL];
    float m_run;
    float l_run;
    int ef_run;
};

// Everything about one 32-token tile that depends on the page table: the
// buffer descriptors of its two 16-token halves (wave-uniform) and whether
// the tile needs masking. Each descriptor ends after the last token of its
// half that lies inside the partition (and never past the buffer), so loads
// for tokens beyond it return 0 without touching memory; a tile past the
// wave's last one gets empty descriptors.
struct TileAddr {
    __amdgpu_buffer_rsrc_t k[2], v[2], ks[2], vs[2];
    int t0;
    bool masked;
    int nv[2];            // selected blocks: keys of each half, from its start
};

// Loop-invariant byte offsets of the lane's loads inside a 16-token half.
// They stay entirely in the VGPR offset: the buffer range check covers the
// VGPR and immediate offsets but not the SGPR one.
struct LaneOffsets {
    int k;                // token li, head-dim bytes [lg*KB, lg*KB + KB)
    int v[4];             // token 4g + r, head-dim bytes [li*DL, li*DL + DL)
    int s;                // scale of token (4g + li) mod 16
};

// One tile's loads. The scales arrive one per lane, rotated so that lane
// r of every 16-lane row g holds token 4g + r: a row broadcast of lane r
// then gives each lane the scales of the tokens of its score registers.
template <int D>
struct TileRegs {
    static constexpr int KV4 = D / 64;      // 16-byte K loads per token
    static constexpr int DL = D / 16;
    typedef typename VRow<DL>::T VT;
    uint4 kraw[2][KV4];
    VT vraw[8];
    uint32_t ks[2], vs[2];
};

// row_newbcast:r -- every lane of a 16-lane row reads lane r of that row
template <int R>
__device__ __forceinline__ float row_bcast(uint32_t v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + R, 0xF, 0xF, false));
}

// CODES: kCodesE4M3Scaled (E4M3 codes, one fp32 scale per row), or the
// unscaled kCodesE4M3 / kCodesE5M2 (no scales are read: scale 1).
template <int D, int CODES = kCodesE4M3Scaled>
struct DecodeTile {
    static constexpr bool kScaled = CODES == kCodesE4M3Scaled;
    static constexpr int KB = D / 4;        // K code bytes per lane per token
    static constexpr int KV4 = KB / 16;     // 16-byte K loads per token
    static constexpr int KSTEPS = D / 32;   // MFMA k-steps over head_dim
    static constexpr int DL = D / 16;       // V bytes per lane per token = PV n-tiles
    typedef typename VRow<DL>::T VT;
    typedef TileRegs<D> Regs;

    // Constants of one piece's page walk (wave-uniform).
    struct WalkConsts {
        const uint8_t* kbase;     // k_cache + h * cache_stride_head
        const uint8_t* vbase;
        const float* ksbase;      // k_scale + h * scale_stride_head
        const float* vsbase;
        const int32_t* bt;        // this request's block-table row
        const int32_t* bv;        // ... and its valid-key counts (selected blocks)
        int p0, p1, ntiles, full_end, last_base;
        int nr_codes_full;        // num_records of a full half: 15*css + D
        int nr_scales_full;       // ... of its scales: 4*(15*sss + 1)
    };

    // Block-table entries of the piece's tiles k0 .. k0+31: lane j holds the
    // entry of tile k0 + j/2, half j%2. Indices are clamped to the piece's
    // last half, so every lane reads an entry the request owns.
    template <bool BSP2>
    static __device__ __forceinline__ int table_window(const DecodeParams& p, const WalkConsts& w,
                                                       const int32_t* row, int k0, int lane) {
        const int stok = min(w.p0 + 32 * (k0 + (lane >> 1)) + 16 * (lane & 1), w.last_base);
        const int bi = BSP2 ? (stok >> p.block_shift) : stok / p.block_size;
        return row[bi];
    }

    // Page walk of tile ti of the piece (wave-uniform) from its two table
    // entries. Full halves use constant bounds; a ragged tile's halves end
    // after their last token inside the piece, and a tile past the piece's
    // last one gets empty ones.
    // With selected blocks (SP), every half is bounded by the keys its block
    // holds from the half's start, and a tile with a partial half is masked.
    template <bool BSP2, bool SP>
    static __device__ __forceinline__ void address(const DecodeParams& p, const WalkConsts& w,
                                                   int ti, const int (&blk_in)[2],
                                                   const int (&valid_in)[2], TileAddr& ta) {
        const int t0 = w.p0 + (ti << 5);
        const bool live = ti < w.ntiles;
        const bool ragged = SP || !live || t0 + 32 > w.p1;
        const int bs = p.block_size;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int stok = t0 + 16 * s;
            const int tab = min(stok, w.last_base);
            const int bo = BSP2 ? (tab & (bs - 1)) : tab % bs;
            const int blk = min(max(blk_in[s], 0), p.num_blocks - 1);
            const int64_t slot = (int64_t)blk * bs + bo;
            const int64_t coff = slot * p.cache_stride_slot;
            const int64_t soff = slot * p.scale_stride_slot;
            int nrc = w.nr_codes_full, nrs = w.nr_scales_full;
            if (ragged) {
                // tokens of this half inside the piece (<= 0: none), and with
                // selected blocks only the block's keys from the half's start
                int nvalid = live ? min(16, w.p1 - stok) : 0;
                if (SP) nvalid = min(nvalid, min(max(valid_in[s], 0), bs) - bo);
                nrc = nvalid > 0 ? (nvalid - 1) * (int)p.cache_stride_slot + D : 0;
                nrs = nvalid > 0 ? 4 * ((nvalid - 1) * (int)p.scale_stride_slot + 1) : 0;
                ta.nv[s] = max(nvalid, 0);
            }
            ta.k[s] = make_rsrc(w.kbase + coff, nrc);
            ta.v[s] = make_rsrc(w.vbase + coff, nrc);
            ta.ks[s] = make_rsrc(w.ksbase + soff, nrs);
            ta.vs[s] = make_rsrc(w.vsbase + soff, nrs);
        }
        ta.t0 = t0;
        ta.masked = t0 + 32 > w.full_end || (SP && (ta.nv[0] < 16 || ta.nv[1] < 16));
    }

    // exact widening of 8 K codes to bf16 and of 2 V codes to fp16
    static __device__ __forceinline__ bf16x8 widen_k(uint32_t lo, uint32_t hi) {
        if constexpr (CODES == kCodesE5M2) return e5m2x8_to_bf16x8(lo, hi);
        else return e4m3x8_to_bf16x8(lo, hi);
    }
    template <bool HI>
    static __device__ __forceinline__ uint32_t widen_v(uint32_t w) {
        if constexpr (CODES == kCodesE5M2) return e5m2x2_to_f16x2<HI>(w);
        else return e4m3x2_to_f16x2<HI>(w);
    }

    static __device__ __forceinline__ void issue(const TileAddr& ta, const LaneOffsets& o, Regs& R) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int c = 0; c < KV4; ++c) {
                intx4 v = __builtin_amdgcn_raw_buffer_load_b128(ta.k[s], o.k + 16 * c, 0, kCodesNT);
                R.kraw[s][c] = make_uint4(v[0], v[1], v[2], v[3]);
            }
#pragma unroll
        for (int e = 0; e < 8; ++e) R.vraw[e] = VRow<DL>::load(ta.v[e >> 2], o.v[e & 3]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if constexpr (kScaled) {
                R.ks[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ta.ks[s], o.s, 0, 0);
                R.vs[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ta.vs[s], o.s, 0, 0);
            } else {
                R.ks[s] = R.vs[s] = 0x3F800000u;      // 1.0f
            }
        }
    }

    // S = K q^T, fp32 accumulate; lane holds tokens 4g + r of each half, row li.
    static __device__ __forceinline__ void qk(const Regs& R, const bf16x8 (&qv)[KSTEPS],
                                              floatx4 (&sc)[2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            sc[s] = floatx4{0.f, 0.f, 0.f, 0.f};
            const uint32_t* kw = reinterpret_cast<const uint32_t*>(R.kraw[s]);
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) {
                const bf16x8 a = widen_k(kw[2 * k], kw[2 * k + 1]);
                sc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qv[k], sc[s], 0, 0, 0);
            }
        }
    }

    // Online-softmax update of the tile's scores; returns P' = p * v_scale *
    // kappa of the lane's 8 tokens in fp16 (the B operand of PV).
    template <bool SP>
    static __device__ __forceinline__ f16x8 softmax(
        const DecodeParams& p, const TileAddr& ta, const uint32_t (&ks)[2],
        const uint32_t (&vs)[2], const floatx4 (&sc)[2], int p1, int lim, int lg,
        WaveState<DL>& st) {

        // ---- scores in log2 units, tile max, value-scale range
        float s2[2][4];
        float sv[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float sk[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            sv[s][0] = sv[s][1] = sv[s][2] = sv[s][3] = 1.0f;
            if constexpr (kScaled) {
                sk[0] = row_bcast<0>(ks[s]);
                sk[1] = row_bcast<1>(ks[s]);
                sk[2] = row_bcast<2>(ks[s]);
                sk[3] = row_bcast<3>(ks[s]);
                sv[s][0] = row_bcast<0>(vs[s]);
                sv[s][1] = row_bcast<1>(vs[s]);
                sv[s][2] = row_bcast<2>(vs[s]);
                sv[s][3] = row_bcast<3>(vs[s]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) s2[s][r] = sc[s][r] * (sk[r] * p.score_scale_log2);
        }
        if (ta.masked) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = ta.t0 + 16 * s + 4 * lg + r;
                    // a key: inside the piece (and, with selected blocks,
                    // among its block's keys); visible: not after the row
                    const bool key = SP ? (4 * lg + r < ta.nv[s]) : tok < p1;
                    s2[s][r] = (key && tok <= lim) ? s2[s][r] : kNeg;
                    sv[s][r] = key ? sv[s][r] : 0.f;
                }
        }
        float svm = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                          fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
        float mt = fmaxf(fmaxf(fmaxf(s2[0][0], s2[0][1]), fmaxf(s2[0][2], s2[0][3])),
                         fmaxf(fmaxf(s2[1][0], s2[1][1]), fmaxf(s2[1][2], s2[1][3])));
        mt = rows_max(mt);
        svm = rows_max(svm);                    // wave-uniform now
        const int ef_t = max((int)((__float_as_uint(svm) >> 23) & 0xFF), 15);
        const float m_new = fmaxf(st.m_run, mt);
        if (__any(m_new > st.m_run || ef_t > st.ef_run)) {
            const int ef_new = max(st.ef_run, ef_t);
            const float a = __builtin_amdgcn_exp2f(st.m_run - m_new);
            const float f = a * pow2i(max(st.ef_run - ef_new, -126));
#pragma unroll
            for (int n = 0; n < DL; ++n) st.acc[n] *= f;
            st.l_run *= a;
            st.m_run = m_new;
            st.ef_run = ef_new;
        }
        const float kappa = pow2i(141 - st.ef_run);

        // ---- P' = p * v_scale * kappa, fp16 (slot e = 4s + r)
        uint32_t pw[4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float e = __builtin_amdgcn_exp2f(s2[s][r] - st.m_run);
                if (ta.masked) e = s2[s][r] == kNeg ? 0.f : e;
                st.l_run += e;
                pr[r] = e * (sv[s][r] * kappa);
            }
            pw[2 * s] = pack_f16x2(pr[0], pr[1]);
            pw[2 * s + 1] = pack_f16x2(pr[2], pr[3]);
        }
        return __builtin_bit_cast(f16x8, pw);
    }

    // O^T += V^T P'^T for NT 16-row tiles from the tile's V code registers;
    // each V operand is widened once and feeds every tile's MFMA.
    template <int NT>
    static __device__ __forceinline__ void pv_tiles(const Regs& R, const f16x8 (&pbs)[NT],
                                                    WaveState<DL>* const (&sts)[NT]) {
        // ---- V^T columns of the lane's 8 tokens, then O^T += V^T P'^T.
        // Pairing two tokens' dwords byte-wise gives, in each 16-bit half, the
        // two tokens' codes of one head-dim column: the fp16 convert then
        // picks the half, so one v_perm level is enough.
#pragma unroll
        for (int w = 0; w < DL / 4; ++w) {
            uint32_t pr_lo[4], pr_hi[4];       // token pairs (0,1) (2,3) (4,5) (6,7)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t a = vword(R.vraw[2 * t], w), b = vword(R.vraw[2 * t + 1], w);
                pr_lo[t] = perm(b, a, 0x05010400u);   // a0 b0 a1 b1
                pr_hi[t] = perm(b, a, 0x07030602u);   // a2 b2 a3 b3
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t* src = c < 2 ? pr_lo : pr_hi;
                uint32_t h[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    h[t] = (c & 1) ? widen_v<true>(src[t]) : widen_v<false>(src[t]);
                const f16x8 a = __builtin_bit_cast(f16x8, h);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    sts[j]->acc[4 * w + c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        a, pbs[j], sts[j]->acc[4 * w + c], 0, 0, 0);
            }
        }
    }

    // Online-softmax update and PV with the tile's scores and V registers.
    template <bool SP>
    static __device__ __forceinline__ void rest(
        const DecodeParams& p, const TileAddr& ta, const Regs& R, const floatx4 (&sc)[2],
        int p1, int lim, int lg, WaveState<DL>& st) {
        const f16x8 pb[1] = {softmax<SP>(p, ta, R.ks, R.vs, sc, p1, lim, lg, st)};
        WaveState<DL>* const sts[1] = {&st};
        pv_tiles<1>(R, pb, sts);
    }
};

}  // namespace fp8kv
