// paged_decode.hip -- paged GQA decode attention over the E4M3 cache.
//
// Semantics (ATOM #2655 description, K/V bullet; sglang-jax #1776,
// "Modifications"): K/V codes are widened exactly to the query's 16-bit
// format before the dot products, the key scale multiplies the score of its
// key, the value scale is folded into the probability before PV, and the
// probabilities are never rounded to the cache format (they are carried in
// fp16, see below).
//
// Decomposition (persistent, evenly split). Per KV head the keys form one
// sequence of 32-token tiles: request 0's tiles, then request 1's, ...
// (U tiles in all). That sequence is cut into R equal ranges (+-1 tile) and
// one wave owns each (range, KV head) pair. By default there is one wave
// per SIMD: every wave streams the same number of tiles from start to end,
// whatever the mix of context lengths, and each SIMD holds exactly one
// stream (measured on MI355X: one stream per SIMD reads HBM faster than two
// or three, and an uneven number of waves per CU leaves a tail). A wave
// reduces each request piece of its range to a partial (normalized output,
// log-sum-exp) in the workspace; piece (request b, range r) has id b + r,
// unique because ids grow along the sequence, and a request's pieces have
// consecutive ids. A second kernel merges each request's pieces by
// log-sum-exp. The four waves of a workgroup are four KV heads of one
// range, and the workgroups of a range sit on one XCD, so a tile's K/V
// rows for all heads are read through one L2 at about the same time.
// The M = rows * G query rows that share KV head h (GQA group times MTP
// verify rows) are stacked into the 16-row dimension of the MFMA tiles, so
// each K/V byte is read from HBM once per step.
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
#include <hip/hip_runtime.h>

#include "fp8kv_device.h"
#include "fp8kv_internal.h"

namespace fp8kv {
namespace {

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
__device__ __forceinline__ float max8(const float (&v)[2][4]) {
    return fmax_fin(fmax_fin(fmax_fin(v[0][0], v[0][1]), fmax_fin(v[0][2], v[0][3])),
                    fmax_fin(fmax_fin(v[1][0], v[1][1]), fmax_fin(v[1][2], v[1][3])));
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

    // The same for NT 16-row tiles of queries: each K operand is widened
    // once and feeds every tile's MFMA chain.
    template <int NT>
    static __device__ __forceinline__ void qk_tiles(const Regs& R, const bf16x8 (&qv)[NT][KSTEPS],
                                                    floatx4 (&sc)[NT][2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int j = 0; j < NT; ++j) sc[j][s] = floatx4{0.f, 0.f, 0.f, 0.f};
            const uint32_t* kw = reinterpret_cast<const uint32_t*>(R.kraw[s]);
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) {
                const bf16x8 a = widen_k(kw[2 * k], kw[2 * k + 1]);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    sc[j][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qv[j][k], sc[j][s], 0, 0, 0);
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

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d);
        if (lane >= d) v += o;
    }
    return v;
}

// Tiles of a request of `len` cached tokens (after clamping).
__device__ __forceinline__ int request_tiles(const DecodeParams& p, int b) {
    const int len = min(max(p.context_lens[b], 0), p.max_context);
    return (len + 31) >> 5;
}

// One piece: tiles [ja, jb) of request b for KV head h, reduced to a partial
// (normalized output and log2 log-sum-exp of each of the M rows) at piece
// id `pid`.
template <int D, bool BSP2, bool SP, int CODES>
__device__ __forceinline__ void decode_piece(const DecodeParams& p, int b, int len, int ja, int jb,
                                             int h, int pid, int lane) {
    constexpr int KSTEPS = D / 32;
    constexpr int DL = D / 16;
    constexpr int KB = D / 4;
    typedef DecodeTile<D, CODES> Tile;
    typedef typename Tile::Regs Regs;
    const int li = lane & 15;
    const int lg = lane >> 4;

    const int p0 = ja << 5;
    const int p1 = min(jb << 5, len);
    const int ntiles = jb - ja;

    typename Tile::WalkConsts w;
    w.kbase = p.k_cache + (int64_t)h * p.cache_stride_head;
    w.vbase = p.v_cache + (int64_t)h * p.cache_stride_head;
    w.ksbase = p.k_scale + (int64_t)h * p.scale_stride_head;
    w.vsbase = p.v_scale + (int64_t)h * p.scale_stride_head;
    w.bt = p.block_tables + (int64_t)b * p.block_table_stride;
    w.bv = SP ? p.block_valid + (int64_t)b * p.block_valid_stride : nullptr;
    w.p0 = p0;
    w.p1 = p1;
    w.ntiles = ntiles;
    // tokens below full_end are visible to every row
    w.full_end = min(p1, len - p.rows + 1);
    w.last_base = (p1 - 1) & ~15;
    w.nr_codes_full = 15 * (int)p.cache_stride_slot + D;
    w.nr_scales_full = 4 * (15 * (int)p.scale_stride_slot + 1);

    // block-table window of tiles 0..31, and the next one when the piece is longer
    int kw = 0;
    int btw = Tile::template table_window<BSP2>(p, w, w.bt, 0, lane);
    int btn = ntiles > 32 ? Tile::template table_window<BSP2>(p, w, w.bt, 32, lane) : 0;
    int bvw = SP ? Tile::template table_window<BSP2>(p, w, w.bv, 0, lane) : 0;
    int bvn = SP && ntiles > 32 ? Tile::template table_window<BSP2>(p, w, w.bv, 32, lane) : 0;

    // q operand: row li of the stacked (verify row, query head) block
    bf16x8 qv[KSTEPS];
    int lim;                                   // last token row li sees
    if (li < p.m_rows) {
        const int r = li / p.group;
        const int hq = h * p.group + (li - r * p.group);
        const uint16_t* qp = p.q + (int64_t)b * p.q_stride_b + (int64_t)r * p.q_stride_row +
                             (int64_t)hq * p.q_stride_head + lg * (D / 4);
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k)
            qv[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 8 * k));
        lim = len - p.rows + r;
    } else {
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) qv[k] = bf16x8{};
        lim = len - 1;
    }

    WaveState<DL> st;
#pragma unroll
    for (int n = 0; n < DL; ++n) st.acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    st.m_run = kNeg;
    st.l_run = 0.f;
    st.ef_run = 15;

    // loop-invariant load offsets
    LaneOffsets lo;
    {
        const int css = (int)p.cache_stride_slot;
        const int sss = (int)p.scale_stride_slot;
        lo.k = li * css + lg * KB;
#pragma unroll
        for (int r = 0; r < 4; ++r) lo.v[r] = (4 * lg + r) * css + li * DL;
        lo.s = ((4 * lg + li) & 15) * sss * 4;
    }

    // table entries of tile k (wave-uniform k); windows move forward 32
    // tiles at a time, the next one already loaded
    auto entries = [&](int k, int (&blk)[2], int (&valid)[2]) {
        if (k - kw >= 32) {
            kw += 32;
            btw = btn;
            if (ntiles > kw + 32) btn = Tile::template table_window<BSP2>(p, w, w.bt, kw + 32, lane);
            if (SP) {
                bvw = bvn;
                if (ntiles > kw + 32) bvn = Tile::template table_window<BSP2>(p, w, w.bv, kw + 32, lane);
            }
        }
        const int j = 2 * (k - kw);
        blk[0] = __builtin_amdgcn_readlane(btw, j);
        blk[1] = __builtin_amdgcn_readlane(btw, j + 1);
        valid[0] = SP ? __builtin_amdgcn_readlane(bvw, j) : 0;
        valid[1] = SP ? __builtin_amdgcn_readlane(bvw, j + 1) : 0;
    };

    // Two tiles in flight: after a tile's QK^T has consumed its K registers,
    // the loads of the next tile are issued, then the tile's softmax and PV
    // run while they are in flight (A/B ping-pong).
    TileAddr ta_a, ta_b;
    Regs ra, rb;
    floatx4 sc[2];
    int blk[2], valid[2];
    int ti = 0;
    entries(0, blk, valid);
    Tile::template address<BSP2, SP>(p, w, 0, blk, valid, ta_a);
    Tile::issue(ta_a, lo, ra);
    while (ti < ntiles) {
        Tile::qk(ra, qv, sc);
        entries(ti + 1, blk, valid);
        Tile::template address<BSP2, SP>(p, w, ti + 1, blk, valid, ta_b);
        Tile::issue(ta_b, lo, rb);
        Tile::template rest<SP>(p, ta_a, ra, sc, p1, lim, lg, st);
        if (++ti >= ntiles) break;
        Tile::qk(rb, qv, sc);
        entries(ti + 1, blk, valid);
        Tile::template address<BSP2, SP>(p, w, ti + 1, blk, valid, ta_a);
        Tile::issue(ta_a, lo, ra);
        Tile::template rest<SP>(p, ta_b, rb, sc, p1, lim, lg, st);
        ++ti;
    }

    // the piece's partial for the lane's row
    st.l_run = rows_sum(st.l_run);
    if (li < p.m_rows) {
        const int64_t u = ((int64_t)pid * p.num_kv_heads + h) * p.m_rows + li;
        const bool any = st.l_run > 0.f;
        // undo the P' range factor 2^(141 - e) with the normalization
        const float inv = any ? pow2i(max(st.ef_run - 141, -126)) / st.l_run : 0.f;
        float* o = p.ws_o + u * D + (DL * 4) * lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float vals[DL];
#pragma unroll
            for (int n = 0; n < DL; ++n) vals[n] = st.acc[n][r] * inv;
#pragma unroll
            for (int c = 0; c < DL / 4; ++c)
                *reinterpret_cast<float4*>(o + DL * r + 4 * c) =
                    make_float4(vals[4 * c], vals[4 * c + 1], vals[4 * c + 2], vals[4 * c + 3]);
        }
        if (lg == 0) p.ws_lse[u] = any ? st.m_run + __log2f(st.l_run) : -INFINITY;
    }
}

// Workgroup = 4 waves = 4 workers; worker = (range r, KV head h). When the
// KV heads fill whole workgroups (m = Hkv / 4 of them per range), the m
// workgroups of a range are placed on one XCD: dispatch deals consecutive
// workgroup ids round-robin to the 8 XCDs.
__device__ __forceinline__ int logical_workgroup(int bid, int wgs_per_range) {
    const int m = wgs_per_range;
    if (m <= 1) return bid;
    const int xcd = bid & 7, k = bid >> 3;
    return (k / m) * 8 * m + xcd * m + (k % m);
}

template <int D, bool BSP2, bool SP, int CODES>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
    const int lane = threadIdx.x & 63;
    // wave index, provably uniform so the page walk and the buffer
    // descriptors stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int worker = logical_workgroup(blockIdx.x, p.wgs_per_range) * 4 + wave;
    const int r = worker / p.num_kv_heads;
    const int h = worker - r * p.num_kv_heads;
    if (r >= p.num_ranges) return;
    const int R = p.num_ranges;

    // total tiles U (per KV head); worker 0 also records the exclusive
    // prefix of tiles per request and U for the merge
    int U = 0;
    for (int c = 0; c < p.batch; c += 64) {
        const int n = c + lane < p.batch ? request_tiles(p, c + lane) : 0;
        const int incl = wave_scan(n, lane);
        if (worker == 0 && c + lane < p.batch) p.ws_prefix[c + lane] = U + incl - n;
        U += __builtin_amdgcn_readlane(incl, 63);
    }
    if (worker == 0 && lane == 0) p.ws_prefix[p.batch] = U;

    // this range: tiles [u0, u1) of the sequence
    const int u0 = (int)(((int64_t)r * U) / R);
    const int u1 = (int)(((int64_t)(r + 1) * U) / R);
    if (u0 >= u1) return;

    // the request holding tile u0 and the tiles before it
    int b = 0, pre = 0;
    for (int c = 0, carry = 0; c < p.batch; c += 64) {
        const int n = c + lane < p.batch ? request_tiles(p, c + lane) : 0;
        const int incl = wave_scan(n, lane) + carry;
        const uint64_t hit = __ballot(incl > u0);
        if (hit) {
            const int j = __builtin_ctzll(hit);
            b = c + j;
            pre = __builtin_amdgcn_readlane(incl - n, j);
            break;
        }
        carry = __builtin_amdgcn_readlane(incl, 63);
    }

    // walk the pieces of the range
    int u = u0;
    while (u < u1) {
        const int len = min(max(p.context_lens[b], 0), p.max_context);
        const int n = (len + 31) >> 5;
        if (n > 0) {
            const int ja = u - pre;
            const int jb = min(n, u1 - pre);
            decode_piece<D, BSP2, SP, CODES>(p, b, len, ja, jb, h, b + r, lane);
            u = pre + jb;
        }
        pre += n;
        ++b;
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

// Log-sum-exp merge of each request's pieces: one workgroup per output
// row (request b, KV head h, stacked row m). Request b's tiles are
// [pre(b), pre(b) + n(b)) of the per-head sequence; they lie in ranges
// r_first .. r_last, whose pieces have ids b + r. The workgroup first takes
// the maximum lse of those pieces, then its threads stream the pieces' rows:
// D/4 threads read one piece row (4 floats each), 256/(D/4) pieces per
// step, several steps in flight; the per-slot sums meet in LDS.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(MergeParams p) {
    constexpr int TPP = D / 4;               // threads per piece row
    constexpr int PPS = 256 / TPP;           // pieces per step
    constexpr int UNROLL = 8;
    __shared__ float lds_max[4];
    __shared__ float lds_acc[PPS][D];
    __shared__ float lds_w[PPS];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int row = blockIdx.x;
    if (row >= p.total_rows) return;
    const int m = row % p.m_rows;
    const int bh = row / p.m_rows;
    const int h = bh % p.num_kv_heads;
    const int b = bh / p.num_kv_heads;
    const int U = p.ws_prefix[p.batch];
    const int pre = p.ws_prefix[b];
    const int n = p.ws_prefix[b + 1] - pre;

    const int slot = t / TPP;
    const int col = (t % TPP) * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
    if (n > 0) {
        // range holding tile u: the r with floor(rU/R) <= u < floor((r+1)U/R)
        const int64_t R = p.num_ranges;
        const int r0 = (int)((((int64_t)pre + 1) * R - 1) / U);
        const int r1 = (int)((((int64_t)pre + n) * R - 1) / U);
        const int np = r1 - r0 + 1;
        const int64_t u0 = ((int64_t)(b + r0) * p.num_kv_heads + h) * p.m_rows + m;
        const int64_t step = (int64_t)p.num_kv_heads * p.m_rows;
        // a range with no tile (more ranges than tiles) has no piece
        auto piece_lse = [&](int q) -> float {
            const int64_t rq = r0 + q;
            if (q >= np || (rq * U) / R == ((rq + 1) * U) / R) return -INFINITY;
            return p.ws_lse[u0 + q * step];
        };

        float mx = -INFINITY;
        for (int q = t; q < np; q += 256) mx = fmaxf(mx, piece_lse(q));
        mx = wave_max(mx);
        if (lane == 0) lds_max[t >> 6] = mx;
        __syncthreads();
        mx = fmaxf(fmaxf(lds_max[0], lds_max[1]), fmaxf(lds_max[2], lds_max[3]));

        if (mx > -INFINITY) {
            const float* o = p.ws_o + u0 * D + col;
            for (int q0 = slot; q0 < np; q0 += PPS * UNROLL) {
                float w[UNROLL];
                float4 v[UNROLL];
#pragma unroll
                for (int j = 0; j < UNROLL; ++j) {
                    const int q = q0 + j * PPS;
                    const float lq = piece_lse(q);
                    w[j] = lq > -INFINITY ? exp2f(lq - mx) : 0.f;
                    v[j] = w[j] > 0.f ? *reinterpret_cast<const float4*>(o + q * step * D)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int j = 0; j < UNROLL; ++j) {
                    wsum += w[j];
                    acc.x += w[j] * v[j].x;
                    acc.y += w[j] * v[j].y;
                    acc.z += w[j] * v[j].z;
                    acc.w += w[j] * v[j].w;
                }
            }
        }
    }
    // sum the PPS slots
    *reinterpret_cast<float4*>(&lds_acc[slot][col]) = acc;
    if (col == 0) lds_w[slot] = wsum;
    __syncthreads();
    if (t < TPP) {
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        float ws = 0.f;
#pragma unroll
        for (int k = 0; k < PPS; ++k) {
            const float4 a = *reinterpret_cast<const float4*>(&lds_acc[k][col]);
            s.x += a.x; s.y += a.y; s.z += a.z; s.w += a.w;
            ws += lds_w[k];
        }
        const float inv = ws > 0.f ? 1.0f / ws : 0.f;
        const float vals[4] = {s.x * inv, s.y * inv, s.z * inv, s.w * inv};
        const int r = m / p.group;
        const int hq = h * p.group + (m - r * p.group);
        const int64_t off = (int64_t)b * p.out_stride_b + (int64_t)r * p.out_stride_row +
                            (int64_t)hq * p.out_stride_head + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (p.out_fp32) {
                static_cast<float*>(p.out)[off + i] = vals[i];
            } else {
                uint32_t bits = __float_as_uint(vals[i]);
                bits += 0x7FFFu + ((bits >> 16) & 1u);      // round to nearest even
                static_cast<uint16_t*>(p.out)[off + i] = (uint16_t)(bits >> 16);
            }
        }
    }
}

// The same merge with one wave per output row, for requests of few pieces:
// the prefix, then every piece's lse (scalar loads) and row (D/64 floats
// per lane) in one round trip per 8 pieces, with an online maximum across
// batches of 8.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_rows_kernel(MergeParams p) {
    constexpr int EPL = D / 64;              // floats per lane
    constexpr int BATCH = 8;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = blockIdx.x * 4 + wave;
    if (row >= p.total_rows) return;
    const int m = row % p.m_rows;
    const int bh = row / p.m_rows;
    const int h = bh % p.num_kv_heads;
    const int b = bh / p.num_kv_heads;
    const int U = p.ws_prefix[p.batch];
    const int pre = p.ws_prefix[b];
    const int n = p.ws_prefix[b + 1] - pre;

    float acc[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
    float wsum = 0.f;
    if (n > 0) {
        const int64_t R = p.num_ranges;
        const int r0 = (int)((((int64_t)pre + 1) * R - 1) / U);
        const int r1 = (int)((((int64_t)pre + n) * R - 1) / U);
        const int np = r1 - r0 + 1;
        const int64_t u0 = ((int64_t)(b + r0) * p.num_kv_heads + h) * p.m_rows + m;
        const int64_t step = (int64_t)p.num_kv_heads * p.m_rows;
        const float* o = p.ws_o + u0 * D + lane * EPL;
        float mx = -INFINITY;
        for (int q0 = 0; q0 < np; q0 += BATCH) {
            float lq[BATCH];
            float v[BATCH][EPL];
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
                const int q = q0 + j;
                const int64_t rq = r0 + q;
                // a range with no tile (more ranges than tiles) has no piece
                const bool live = q < np && (rq * U) / R != ((rq + 1) * U) / R;
                lq[j] = live ? p.ws_lse[u0 + q * step] : -INFINITY;
#pragma unroll
                for (int i = 0; i < EPL; ++i) v[j][i] = live ? o[q * step * D + i] : 0.f;
            }
            float cm = mx;
#pragma unroll
            for (int j = 0; j < BATCH; ++j) cm = fmaxf(cm, lq[j]);
            if (cm == -INFINITY) continue;
            if (cm > mx) {
                const float a = mx == -INFINITY ? 0.f : exp2f(mx - cm);
#pragma unroll
                for (int i = 0; i < EPL; ++i) acc[i] *= a;
                wsum *= a;
                mx = cm;
            }
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
                const float w = lq[j] > -INFINITY ? exp2f(lq[j] - mx) : 0.f;
                wsum += w;
#pragma unroll
                for (int i = 0; i < EPL; ++i) acc[i] += w * v[j][i];
            }
        }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    const int r = m / p.group;
    const int hq = h * p.group + (m - r * p.group);
    const int64_t off = (int64_t)b * p.out_stride_b + (int64_t)r * p.out_stride_row +
                        (int64_t)hq * p.out_stride_head + lane * EPL;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float val = acc[i] * inv;
        if (p.out_fp32) {
            static_cast<float*>(p.out)[off + i] = val;
        } else {
            uint32_t bits = __float_as_uint(val);
            bits += 0x7FFFu + ((bits >> 16) & 1u);      // round to nearest even
            static_cast<uint16_t*>(p.out)[off + i] = (uint16_t)(bits >> 16);
        }
    }
}

template <int D, bool BSP2, bool SP, int CODES>
hipError_t launch_split(const DecodeParams& p, hipStream_t stream) {
    const int64_t workers = (int64_t)p.num_ranges * p.num_kv_heads;
    const int64_t quantum = p.wgs_per_range > 1 ? 8 * p.wgs_per_range : 1;
    int64_t wgs = (workers + 3) / 4;
    wgs = (wgs + quantum - 1) / quantum * quantum;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_split_kernel<D, BSP2, SP, CODES>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool SP, int CODES = kCodesE4M3Scaled>
hipError_t launch_split_bs(const DecodeParams& p, hipStream_t stream) {
    return p.block_shift >= 0 ? launch_split<D, true, SP, CODES>(p, stream)
                              : launch_split<D, false, SP, CODES>(p, stream);
}

// ---------------------------------------------------------------------------
// Chunked-prefill attention over the FP8 cache: every query token of a chunk
// attends to the cached tokens up to its own position. Workgroup = (request,
// KV head, block of 4 x NT x 16/G query tokens); each of its 4 waves carries
// NT row tiles, each stacking 16/G tokens x G query heads into the 16 MFMA
// rows exactly as the decode split kernel stacks verify rows, and runs the
// decode kernel's tile math (QK^T MFMA, online softmax, P' = p * v_scale in
// fp16, PV MFMA) with the same rounding at every step. Each K and V operand
// is widened from E4M3 once per wave and feeds all NT row tiles; the
// value-scale range exponent of P' depends only on the tile, so it and
// v_scale * kappa are shared by the row tiles too.
//
// The K/V codes and scales of each 32-token tile are read from the cache
// once per workgroup into LDS (double-buffered): every loader wave moves the
// rows of 8 (head_dim 128) or 16 (head_dim 64) tokens of one 16-token half,
// whose page lookup is wave-uniform, through buffer descriptors that end
// after the chunk's last visible key, so nothing past it is read. The key
// scales go to LDS already multiplied by softmax_scale * log2(e). All 4
// waves read their operands from LDS in the decode kernel's register layout,
// the scales as four consecutive tokens per lane (no lane broadcast needed).
// Workgroups of one (request, KV head) run on one XCD, the deepest query
// blocks first.
// The prefill kernel keeps a row's running maximum until a tile's scores
// exceed it by more than kLazyMax (log2 units), so p = exp2(s - m) stays
// below 2^kLazyMax; its P' range factor is 2^(141 - kLazyMax - e), which
// keeps P' below 2^15 as in the decode kernel.
constexpr int kLazyMax = 8;

template <int D, bool BSP2, int NT>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
    constexpr int KSTEPS = D / 32;
    constexpr int DL = D / 16;
    constexpr int KB = D / 4;
    constexpr int ROW = D + 16;               // padded LDS row: conflict-free row reads
    constexpr int CPR = D / 16;               // 16-byte chunks per code row
    constexpr int TPL = 64 / CPR;             // tokens one loader wave moves
    constexpr int LOAD_WAVES = 32 / TPL;
    static_assert(TPL <= 16 && 16 % TPL == 0, "a loader wave stays inside one half");
    typedef DecodeTile<D> Tile;
    typedef typename Tile::Regs Regs;
    __shared__ __align__(16) uint8_t lds_k[2][32 * ROW];
    __shared__ __align__(16) uint8_t lds_v[2][32 * ROW];
    __shared__ __align__(16) float lds_s[2][2][32];   // [buf][k_scale * score scale | v_scale][token]

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int li = lane & 15, lg = lane >> 4;

    // XCD-contiguous numbering, deepest query block first within a group
    const int nwg = gridDim.x;
    const int L_id = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int grp = L_id / p.qblocks;
    if (grp >= p.batch * p.num_kv_heads) return;
    const int qb = p.qblocks - 1 - (L_id - grp * p.qblocks);
    const int b = grp / p.num_kv_heads;
    const int h = grp - b * p.num_kv_heads;
    const int L = min(max(p.context_lens[b], 0), p.max_context);
    const int qlen = min(min(max(p.q_lens[b], 0), p.max_q), L);
    const int TPW = p.tokens_per_wave;
    const int q0 = qb * 4 * NT * TPW;
    if (q0 >= qlen) return;
    const int P = L - qlen;                               // cached tokens before the chunk
    const int kv_end = P + min(q0 + 4 * NT * TPW, qlen);  // no row of the block sees beyond
    const int ntiles = (kv_end + 31) >> 5;

    // q operand and causal limit of row li of tile j: token tq of the chunk,
    // head hq
    const int hq = h * p.group + li % p.group;
    int tq[NT], lim[NT];
    bf16x8 qv[NT][KSTEPS];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        tq[j] = q0 + (wave * NT + j) * TPW + li / p.group;
        lim[j] = P + tq[j];
        if (tq[j] < qlen) {
            const uint16_t* qp = p.q + (int64_t)b * p.q_stride_b + (int64_t)tq[j] * p.q_stride_tok +
                                 (int64_t)hq * p.q_stride_head + lg * (D / 4);
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k)
                qv[j][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 8 * k));
        } else {
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) qv[j][k] = bf16x8{};
        }
    }
    const int wave_lim = P + q0 + wave * NT * TPW;        // smallest limit of the wave's rows

    // softmax state of each row tile; the P' range exponent is shared
    WaveState<DL> st[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int n = 0; n < DL; ++n) st[j].acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
        st[j].m_run = kNeg;
        st[j].l_run = 0.f;
    }
    int ef_run = 15;

    // cooperative tile load: lane t of a loader wave moves 16 bytes of token
    // t / CPR's K and V rows and reads the token's two scales; its chunk-0
    // lanes store the key scale, its chunk-1 lanes the value scale
    const bool loader = wave < LOAD_WAVES;
    const int ld_tok = t / CPR, ld_chunk = t % CPR;
    const int ld_half = (wave * TPL) >> 4;
    const int ld_code = (ld_tok & 15) * (int)p.cache_stride_slot + 16 * ld_chunk;
    const int ld_scale = (ld_tok & 15) * (int)p.scale_stride_slot * 4;
    const int lds_code = ld_tok * ROW + 16 * ld_chunk;
    const uint8_t* kbase = p.k_cache + (int64_t)h * p.cache_stride_head;
    const uint8_t* vbase = p.v_cache + (int64_t)h * p.cache_stride_head;
    const float* ksbase = p.k_scale + (int64_t)h * p.scale_stride_head;
    const float* vsbase = p.v_scale + (int64_t)h * p.scale_stride_head;
    const int32_t* bt = p.block_tables + (int64_t)b * p.block_table_stride;
    intx4 kr = {0, 0, 0, 0}, vr = {0, 0, 0, 0};
    float sr = 0.f;
    auto load_tile = [&](int ti) {
        // the wave's half: keys stok .. stok + nvalid - 1, all in one block
        const int stok = (ti << 5) + 16 * ld_half;
        const int nvalid = min(16, kv_end - stok);
        int64_t slot = 0;
        if (nvalid > 0) {
            const int bi = BSP2 ? (stok >> p.block_shift) : stok / p.block_size;
            const int bo = BSP2 ? (stok & (p.block_size - 1)) : stok - bi * p.block_size;
            const int blk = min(max(bt[bi], 0), p.num_blocks - 1);
            slot = (int64_t)blk * p.block_size + bo;
        }
        const int nrc = nvalid > 0 ? (nvalid - 1) * (int)p.cache_stride_slot + D : 0;
        const int nrs = nvalid > 0 ? 4 * ((nvalid - 1) * (int)p.scale_stride_slot + 1) : 0;
        const int64_t coff = slot * p.cache_stride_slot;
        const int64_t soff = slot * p.scale_stride_slot;
        kr = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(kbase + coff, nrc), ld_code, 0, 0);
        vr = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(vbase + coff, nrc), ld_code, 0, 0);
        const float ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                       make_rsrc(ksbase + soff, nrs), ld_scale, 0, 0));
        const float vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                       make_rsrc(vsbase + soff, nrs), ld_scale, 0, 0));
        sr = ld_chunk == 0 ? ks * p.score_scale_log2 : vs;
    };
    auto store_tile = [&](int buf) {
        *reinterpret_cast<intx4*>(&lds_k[buf][lds_code]) = kr;
        *reinterpret_cast<intx4*>(&lds_v[buf][lds_code]) = vr;
        if (ld_chunk < 2) lds_s[buf][ld_chunk][ld_tok] = sr;
    };

    if (loader) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int ti = 0; ti < ntiles; ++ti) {
        const int buf = ti & 1;
        if (loader && ti + 1 < ntiles) load_tile(ti + 1);
        // operands in the decode kernel's register layout
        Regs R;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int c = 0; c < Tile::KV4; ++c)
                R.kraw[s][c] = *reinterpret_cast<const uint4*>(
                    &lds_k[buf][(16 * s + li) * ROW + lg * KB + 16 * c]);
        }
        floatx4 sc[NT][2];
        Tile::template qk_tiles<NT>(R, qv, sc);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint8_t* src = &lds_v[buf][(16 * (e >> 2) + 4 * lg + (e & 3)) * ROW + li * DL];
            if constexpr (DL == 8)
                R.vraw[e] = *reinterpret_cast<const uint2*>(src);
            else
                R.vraw[e] = *reinterpret_cast<const uint32_t*>(src);
        }
        // scales of the lane's score tokens 16 s + 4 lg + r
        float sk[2][4], sv[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float4 a = *reinterpret_cast<const float4*>(&lds_s[buf][0][16 * s + 4 * lg]);
            const float4 c = *reinterpret_cast<const float4*>(&lds_s[buf][1][16 * s + 4 * lg]);
            sk[s][0] = a.x; sk[s][1] = a.y; sk[s][2] = a.z; sk[s][3] = a.w;
            sv[s][0] = c.x; sv[s][1] = c.y; sv[s][2] = c.z; sv[s][3] = c.w;
        }

        // ---- P' range of the tile (keys past the chunk have v_scale 0);
        // the scales are >= 0, so their bit patterns order as integers
        uint32_t svm = 0;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) svm = max(svm, __float_as_uint(sv[s][r]));
        svm = rows_max_u32(svm);
        const int ef_t = max((int)(svm >> 23), 15);
        const int ef_new = max(ef_run, ef_t);
        const bool ef_up = ef_new > ef_run;
        const float fe = pow2i(max(ef_run - ef_new, -126));
        ef_run = ef_new;
        const float kappa = pow2i(141 - kLazyMax - ef_run);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[s][r] *= kappa;

        // ---- online softmax of each row tile; P' = p * v_scale * kappa
        const bool masked = (ti << 5) + 31 > wave_lim;
        f16x8 pb[NT];
        WaveState<DL>* sts[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float s2[2][4];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) s2[s][r] = sc[j][s][r] * sk[s][r];
            if (masked) {
                // key 16 s + 4 lg + r of the tile is visible iff
                // 16 s + r <= lim - t0 - 4 lg
                const int d = lim[j] - (ti << 5) - 4 * lg;
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int r = 0; r < 4; ++r) s2[s][r] = 16 * s + r <= d ? s2[s][r] : kNeg;
            }
            // lazy maximum: the running maximum moves only when a score
            // exceeds it by more than kLazyMax, so most tiles skip the rescale.
            // m_run is the same in the four lanes of a row, so "some lane's
            // scores exceed it" is "some row's scores exceed it": the row
            // maximum across lanes is only needed when the branch is taken
            const float ml = max8(s2);
            if (__any(ml > st[j].m_run + kLazyMax) || ef_up) {
                const float m_new = fmax_fin(st[j].m_run, rows_max_fin(ml));
                const float a = __builtin_amdgcn_exp2f(st[j].m_run - m_new);
                const float f = a * fe;
#pragma unroll
                for (int n = 0; n < DL; ++n) st[j].acc[n] *= f;
                st[j].l_run *= a;
                st[j].m_run = m_new;
            }
            uint32_t pw[4];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                float pr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // a masked score gives exp2(kNeg - m) = 0: every row sees
                    // key 0 in the first tile, so m is a real score throughout
                    const float e = __builtin_amdgcn_exp2f(s2[s][r] - st[j].m_run);
                    st[j].l_run += e;
                    pr[r] = e * sv[s][r];
                }
                pw[2 * s] = pack_f16x2(pr[0], pr[1]);
                pw[2 * s + 1] = pack_f16x2(pr[2], pr[3]);
            }
            pb[j] = __builtin_bit_cast(f16x8, pw);
            sts[j] = &st[j];
        }
        Tile::template pv_tiles<NT>(R, pb, sts);
        if (loader && ti + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    // normalized output of row li of each tile: dims [DL*4 lg, DL*4 lg + DL*4)
    const float un = pow2i(max(ef_run - 141 + kLazyMax, -126));
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const float l_sum = rows_sum(st[j].l_run);
        if (tq[j] >= qlen) continue;
        const float inv = l_sum > 0.f ? un / l_sum : 0.f;
        const int64_t off = (int64_t)b * p.out_stride_b + (int64_t)tq[j] * p.out_stride_tok +
                            (int64_t)hq * p.out_stride_head + (DL * 4) * lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float vals[DL];
#pragma unroll
            for (int n = 0; n < DL; ++n) vals[n] = st[j].acc[n][r] * inv;
            if (p.out_fp32) {
                float* o = static_cast<float*>(p.out) + off + DL * r;
#pragma unroll
                for (int c = 0; c < DL / 4; ++c)
                    *reinterpret_cast<float4*>(o + 4 * c) =
                        make_float4(vals[4 * c], vals[4 * c + 1], vals[4 * c + 2], vals[4 * c + 3]);
            } else {
                uint16_t* o = static_cast<uint16_t*>(p.out) + off + DL * r;
                uint32_t w[DL / 2];
#pragma unroll
                for (int n = 0; n < DL / 2; ++n) {
                    const bf16x2 v2 = {(__bf16)vals[2 * n], (__bf16)vals[2 * n + 1]};
                    w[n] = __builtin_bit_cast(uint32_t, v2);
                }
                if constexpr (DL == 8)
                    *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
                else
                    *reinterpret_cast<uint2*>(o) = make_uint2(w[0], w[1]);
            }
        }
    }
}

}  // namespace

int decode_wave_slots(int device) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return 0;
    return cus * 4;                            // one wave per SIMD
}

hipError_t launch_decode_partitions(const DecodeParams& p, int head_dim, hipStream_t stream) {
    const bool sp = p.block_valid != nullptr;
    if (p.codes != kCodesE4M3Scaled) {
        // unscaled caches: the dense walk only
        if (sp) return hipErrorInvalidValue;
        const bool e5 = p.codes == kCodesE5M2;
        if (head_dim == 128)
            return e5 ? launch_split_bs<128, false, kCodesE5M2>(p, stream)
                      : launch_split_bs<128, false, kCodesE4M3>(p, stream);
        return e5 ? launch_split_bs<64, false, kCodesE5M2>(p, stream)
                  : launch_split_bs<64, false, kCodesE4M3>(p, stream);
    }
    if (head_dim == 128)
        return sp ? launch_split_bs<128, true>(p, stream) : launch_split_bs<128, false>(p, stream);
    return sp ? launch_split_bs<64, true>(p, stream) : launch_split_bs<64, false>(p, stream);
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
    const int64_t wgs = ((int64_t)p.batch * p.num_kv_heads * p.qblocks + 7) / 8 * 8;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    const bool pow2 = p.block_shift >= 0;
    dim3 grid((unsigned)wgs), block(256);
    if (head_dim == 128) {
        if (pow2) hipLaunchKernelGGL((prefill_kernel<128, true, kPrefillRowTiles>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((prefill_kernel<128, false, kPrefillRowTiles>), grid, block, 0, stream, p);
    } else {
        if (pow2) hipLaunchKernelGGL((prefill_kernel<64, true, kPrefillRowTiles>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((prefill_kernel<64, false, kPrefillRowTiles>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_decode_merge(const MergeParams& p, int head_dim, hipStream_t stream) {
    // few pieces per request on average (ranges per KV head up to 4 per
    // request): one wave per output row; else one workgroup per row
    if ((int64_t)p.num_ranges <= 4 * (int64_t)p.batch) {
        dim3 grid((unsigned)((p.total_rows + 3) / 4)), block(256);
        if (head_dim == 128)
            hipLaunchKernelGGL(decode_merge_rows_kernel<128>, grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL(decode_merge_rows_kernel<64>, grid, block, 0, stream, p);
        return hipGetLastError();
    }
    dim3 grid((unsigned)p.total_rows), block(256);
    if (head_dim == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(decode_merge_kernel<64>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace fp8kv
