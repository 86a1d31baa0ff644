// prefill_attn.hip -- chunked-prefill attention over the E4M3 cache
// (sglang-jax #1776, "Modifications": each KV tile is widened to the query
// dtype before the score dot, and P never takes the cache dtype; ATOM #2655
// description: prefill sparse GQA over the E4M3 cache). The tile math it
// shares with the decode split kernel is in attn_tile.h.
//
// Every query token of a chunk attends to the cached tokens up to its own
// position (the chunk was scattered into the cache first). Workgroup = (request,
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
// Selected blocks (SP): the page table lists the blocks a request selected,
// in position order, with a count of valid keys per entry (from the block's
// start), as in the decode over selected blocks; positions are virtual
// (offset j % bs of selected block j / bs) and the chunk is causal on them.
// A loader wave bounds its half by the block's count, so a partial block's
// tail is never read, and publishes the half's key count in LDS; a tile
// with a partial half takes the masked path, where a position past its
// block's count is no key and adds exactly nothing (a row may see no key
// in a tile, or at all: its output is then 0).
// Occupancy: the dense kernel fits 168 VGPRs, 3 waves per SIMD (each wave's
// tile chain is latency-bound, so a third wave adds throughput); the
// selected-block kernel needs more registers and runs 2 waves per SIMD.
// Key groups (KG = 3, dense head_dim 128, chosen by the host when there are
// at most 2 query blocks per CU): the workgroup is 3 groups of 4 waves; group
// g walks tiles [g T / 3, (g + 1) T / 3) of the block's T key tiles with its
// own LDS buffers, all 12 waves meeting at each tile's barrier, and the
// groups' normalized rows are merged into group 0 by their log2 sum-exp
// through LDS. A row may see no key in a group's tiles (its masked
// probabilities are zeroed and its sum-exp is kNeg, weight 0).
// The prefill kernel keeps a row's running maximum until a tile's scores
// exceed it by more than kLazyMax (log2 units), so p = exp2(s - m) stays
// below 2^kLazyMax; its P' range factor is 2^(141 - kLazyMax - e), which
// keeps P' below 2^15 as in the decode kernel.
#include <hip/hip_runtime.h>

#include "attn_tile.h"
#include "fp8kv_device.h"
#include "fp8kv_internal.h"

namespace fp8kv {
namespace {

constexpr int kLazyMax = 8;

template <int D, bool BSP2, int NT, bool SP, int KG>
__global__ __launch_bounds__(256 * KG, SP ? 2 : (KG == 1 ? 3 : 1)) void prefill_kernel(PrefillParams p) {
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
    // LDS of key group g: K and V code tiles [2][32 * ROW] each, scales
    // [2][k_scale * score scale | v_scale][32], selected-block key counts
    // [2][half]; with KG > 1 the same bytes later hold the groups' partial
    // results for the merge
    constexpr int TILE_BYTES = 4 * 32 * ROW + 2 * 2 * 32 * 4 + 16;
    constexpr int MERGE_BYTES = KG > 1 ? 4 * 64 * NT * (4 * DL + 2) * 4 : 0;
    constexpr int LDS_BYTES = KG * TILE_BYTES > MERGE_BYTES ? KG * TILE_BYTES : MERGE_BYTES;
    __shared__ __align__(16) uint8_t lds_raw[LDS_BYTES];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int kg = wv >> 2;           // key group: a third of the block's key tiles (KG = 3)
    const int wave = wv & 3;          // role in the query block: rows, loader slice
    const int li = lane & 15, lg = lane >> 4;
    uint8_t* const lds_g = lds_raw + kg * TILE_BYTES;
    auto lds_k = [&](int buf) { return lds_g + buf * 32 * ROW; };
    auto lds_v = [&](int buf) { return lds_g + (2 + buf) * 32 * ROW; };
    auto lds_s = [&](int buf, int which) {
        return reinterpret_cast<float*>(lds_g + 4 * 32 * ROW) + (2 * buf + which) * 32;
    };
    auto lds_nv = [&](int buf) {
        return reinterpret_cast<int*>(lds_g + 4 * 32 * ROW + 2 * 2 * 32 * 4) + 2 * buf;
    };

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
    // this group's tiles [tg0, tg0 + ng); the groups' counts differ by at
    // most one and every group runs nmax rounds (one barrier each)
    const int tg0 = kg * ntiles / KG;
    const int ng = (kg + 1) * ntiles / KG - tg0;
    const int nmax = (ntiles + KG - 1) / KG;

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
    const int ld_tok = (t & 255) / CPR, ld_chunk = t % CPR;
    const int ld_half = (wave * TPL) >> 4;
    const int ld_code = (ld_tok & 15) * (int)p.cache_stride_slot + 16 * ld_chunk;
    const int ld_scale = (ld_tok & 15) * (int)p.scale_stride_slot * 4;
    const int lds_code = ld_tok * ROW + 16 * ld_chunk;
    const uint8_t* kbase = p.k_cache + (int64_t)h * p.cache_stride_head;
    const uint8_t* vbase = p.v_cache + (int64_t)h * p.cache_stride_head;
    const float* ksbase = p.k_scale + (int64_t)h * p.scale_stride_head;
    const float* vsbase = p.v_scale + (int64_t)h * p.scale_stride_head;
    const int32_t* bt = p.block_tables + (int64_t)b * p.block_table_stride;
    const int32_t* bv = SP ? p.block_valid + (int64_t)b * p.block_valid_stride : nullptr;
    intx4 kr = {0, 0, 0, 0}, vr = {0, 0, 0, 0};
    float ksr = 0.f, vsr = 0.f;
    int ld_nv = 16;
    auto load_tile = [&](int ti) {
        // the wave's half: keys stok .. stok + nvalid - 1, all in one block
        // (with selected blocks: only the block's valid keys from stok)
        const int stok = (ti << 5) + 16 * ld_half;
        int nvalid = min(16, kv_end - stok);
        int64_t slot = 0;
        if (nvalid > 0) {
            const int bi = BSP2 ? (stok >> p.block_shift) : stok / p.block_size;
            const int bo = BSP2 ? (stok & (p.block_size - 1)) : stok - bi * p.block_size;
            const int blk = min(max(bt[bi], 0), p.num_blocks - 1);
            slot = (int64_t)blk * p.block_size + bo;
            if (SP) nvalid = min(nvalid, min(max(bv[bi], 0), p.block_size) - bo);
        }
        ld_nv = max(nvalid, 0);
        const int nrc = nvalid > 0 ? (nvalid - 1) * (int)p.cache_stride_slot + D : 0;
        const int nrs = nvalid > 0 ? 4 * ((nvalid - 1) * (int)p.scale_stride_slot + 1) : 0;
        const int64_t coff = slot * p.cache_stride_slot;
        const int64_t soff = slot * p.scale_stride_slot;
        kr = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(kbase + coff, nrc), ld_code, 0, 0);
        vr = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(vbase + coff, nrc), ld_code, 0, 0);
        // every lane loads both scales; they are combined when the tile is
        // stored (a multiply here would make the wave wait for all of its
        // loads in flight, the K/V codes included)
        ksr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            make_rsrc(ksbase + soff, nrs), ld_scale, 0, 0));
        vsr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            make_rsrc(vsbase + soff, nrs), ld_scale, 0, 0));
    };
    auto store_tile = [&](int buf) {
        *reinterpret_cast<intx4*>(lds_k(buf) + lds_code) = kr;
        *reinterpret_cast<intx4*>(lds_v(buf) + lds_code) = vr;
        const float sr = ld_chunk == 0 ? ksr * p.score_scale_log2 : vsr;
        if (ld_chunk < 2) lds_s(buf, ld_chunk)[ld_tok] = sr;
        if (SP && lane == 0 && ((wave * TPL) & 15) == 0) lds_nv(buf)[ld_half] = ld_nv;
    };

    if (loader && ng > 0) {
        load_tile(tg0);
        store_tile(0);
    }
    __syncthreads();
    for (int it = 0; it < nmax; ++it) {
        const int ti = tg0 + it;
        const int buf = it & 1;
        if (loader && it + 1 < ng) load_tile(ti + 1);
        if (it < ng) {
            // operands in the decode kernel's register layout
            Regs R;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int c = 0; c < Tile::KV4; ++c)
                    R.kraw[s][c] = *reinterpret_cast<const uint4*>(
                        lds_k(buf) + (16 * s + li) * ROW + lg * KB + 16 * c);
            }
            floatx4 sc[NT][2];
            Tile::template qk_tiles<NT>(R, qv, sc);
            // scales of the lane's score tokens 16 s + 4 lg + r
            float sk[2][4], sv[2][4];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const float4 a = *reinterpret_cast<const float4*>(lds_s(buf, 0) + 16 * s + 4 * lg);
                const float4 c = *reinterpret_cast<const float4*>(lds_s(buf, 1) + 16 * s + 4 * lg);
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
            int nv[2] = {16, 16};
            if (SP) {
                nv[0] = lds_nv(buf)[0];
                nv[1] = lds_nv(buf)[1];
            }
            const bool masked = (ti << 5) + 31 > wave_lim || (SP && (nv[0] < 16 || nv[1] < 16));
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
                        for (int r = 0; r < 4; ++r)
                            s2[s][r] = (16 * s + r <= d && (!SP || 4 * lg + r < nv[s])) ? s2[s][r] : kNeg;
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
                        // (with selected blocks a row may have seen no key yet, so
                        // masked positions are zeroed explicitly)
                        float e = __builtin_amdgcn_exp2f(s2[s][r] - st[j].m_run);
                        if ((SP || KG > 1) && masked) e = s2[s][r] == kNeg ? 0.f : e;
                        st[j].l_run += e;
                        pr[r] = e * sv[s][r];
                    }
                    pw[2 * s] = pack_f16x2(pr[0], pr[1]);
                    pw[2 * s + 1] = pack_f16x2(pr[2], pr[3]);
                }
                pb[j] = __builtin_bit_cast(f16x8, pw);
                sts[j] = &st[j];
            }
            // V operands read only now: not held in registers across the softmax
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint8_t* src = lds_v(buf) + (16 * (e >> 2) + 4 * lg + (e & 3)) * ROW + li * DL;
                if constexpr (DL == 8)
                    R.vraw[e] = *reinterpret_cast<const uint2*>(src);
                else
                    R.vraw[e] = *reinterpret_cast<const uint32_t*>(src);
            }
            Tile::template pv_tiles<NT>(R, pb, sts);
        }
        if (loader && it + 1 < ng) store_tile(buf ^ 1);
        __syncthreads();
    }

    // normalized output of row li of each tile: dims [DL*4 lg, DL*4 lg + DL*4)
    const float un = pow2i(max(ef_run - 141 + kLazyMax, -126));
    if constexpr (KG > 1) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            // the group's normalized rows and their log2 sum-exp (kNeg for a
            // row that saw no key in the group's tiles)
            const float l_sum = rows_sum(st[j].l_run);
            const float nrm = l_sum > 0.f ? un / l_sum : 0.f;
#pragma unroll
            for (int n = 0; n < DL; ++n) st[j].acc[n] *= nrm;
            st[j].m_run = l_sum > 0.f ? st[j].m_run + __builtin_amdgcn_logf(l_sum) : kNeg;
            st[j].l_run = 1.0f;               // weight of the rows at their own sum-exp
        }
        // merge the key groups into group 0, one group at a time through
        // LDS: rows of sum-exp lse_g weigh 2^(lse_g - max lse)
        constexpr int F = NT * (4 * DL + 1);            // floats per lane
        float* mine = reinterpret_cast<float*>(lds_raw) + wave * F * 64 + lane;
#pragma unroll
        for (int g = 1; g < KG; ++g) {
            __syncthreads();                              // the tiles, or the previous group, consumed
            if (kg == g) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
#pragma unroll
                    for (int n = 0; n < DL; ++n)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            mine[(j * (4 * DL + 1) + 4 * n + r) * 64] = st[j].acc[n][r];
                    mine[(j * (4 * DL + 1) + 4 * DL) * 64] = st[j].m_run;
                }
            }
            __syncthreads();
            if (kg == 0) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const float lo = mine[(j * (4 * DL + 1) + 4 * DL) * 64];
                    const float mx = fmaxf(st[j].m_run, lo);
                    const float a = __builtin_amdgcn_exp2f(st[j].m_run - mx);
                    const float c = __builtin_amdgcn_exp2f(lo - mx);
#pragma unroll
                    for (int n = 0; n < DL; ++n)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            st[j].acc[n][r] = __builtin_fmaf(
                                mine[(j * (4 * DL + 1) + 4 * n + r) * 64], c, st[j].acc[n][r] * a);
                    st[j].l_run = st[j].l_run * a + c;
                    st[j].m_run = mx;
                }
            }
        }
        if (kg != 0) return;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const float l_sum = rows_sum(st[j].l_run);
        if (tq[j] >= qlen) continue;
        // one key group: un / l; merged groups: the rows are normalized, l
        // is their summed weight
        const float inv = KG == 1 ? (l_sum > 0.f ? un / l_sum : 0.f) : 1.0f / st[j].l_run;
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

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
    const int64_t wgs = ((int64_t)p.batch * p.num_kv_heads * p.qblocks + 7) / 8 * 8;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    const bool pow2 = p.block_shift >= 0;
    const bool sp = p.block_valid != nullptr;
    const dim3 grid((unsigned)wgs);
    constexpr int NT = kPrefillRowTiles;
    // Dense head_dim 128 runs 3 waves per SIMD. With at most 2 query blocks
    // per CU that many waves only exist if each block's keys are split:
    // three key groups per block (12 waves), merged by log-sum-exp. With
    // more blocks, one group of 4 waves per block (the 12-wave barrier of
    // every tile costs more than the split gains).
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
    const bool groups = wgs <= 2 * (int64_t)cus;
    if (head_dim == 128) {
        if (sp) {
            if (pow2) hipLaunchKernelGGL((prefill_kernel<128, true, NT, true, 1>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((prefill_kernel<128, false, NT, true, 1>), grid, dim3(256), 0, stream, p);
        } else if (groups) {
            if (pow2) hipLaunchKernelGGL((prefill_kernel<128, true, NT, false, 3>), grid, dim3(768), 0, stream, p);
            else hipLaunchKernelGGL((prefill_kernel<128, false, NT, false, 3>), grid, dim3(768), 0, stream, p);
        } else {
            if (pow2) hipLaunchKernelGGL((prefill_kernel<128, true, NT, false, 1>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((prefill_kernel<128, false, NT, false, 1>), grid, dim3(256), 0, stream, p);
        }
    } else {
        if (sp) {
            if (pow2) hipLaunchKernelGGL((prefill_kernel<64, true, NT, true, 1>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((prefill_kernel<64, false, NT, true, 1>), grid, dim3(256), 0, stream, p);
        } else {
            if (pow2) hipLaunchKernelGGL((prefill_kernel<64, true, NT, false, 1>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((prefill_kernel<64, false, NT, false, 1>), grid, dim3(256), 0, stream, p);
        }
    }
    return hipGetLastError();
}

}  // namespace fp8kv
