// prefill_attn.hip -- chunked-prefill attention over the E4M3 cache
// (sglang-jax #1776, "Modifications": each KV tile is widened to the query
// dtype before the score dot, and P never takes the cache dtype; ATOM #2655
// description: prefill sparse GQA over the E4M3 cache). The state and
// helpers it shares with the decode split kernel are in attn_tile.h.
//
// Every query token of a chunk attends to the cached tokens up to its own
// position (the chunk was scattered into the cache first). Workgroup = (request,
// KV head, block of 4 x NT x 16/G query tokens); each of its 4 waves carries
// NT row tiles, each stacking 16/G tokens x G query heads into the 16 MFMA
// rows exactly as the decode split kernel stacks verify rows: QK^T MFMA
// (bf16), online softmax with the key scale on the score, P' = p * v_scale
// in fp16, PV MFMA (fp16). With one key group the range exponent of P' is
// fixed per workgroup before the key loop: one pass over the value scales
// of every key the workgroup will read takes their largest exponent (the
// value the decode kernel's running exponent reaches at its last tile), so
// the loader stores v_scale * kappa in LDS and the tiles do no range
// bookkeeping. Key groups keep a running exponent per group, updated per
// tile and shared by the row tiles.
//
// The K/V codes and scales of each 32-token tile are read from the cache
// once per workgroup into LDS (two buffers; with key groups four per group,
// the loader two tiles ahead): every loader wave moves the
// rows of 8 (head_dim 128) or 16 (head_dim 64) tokens of one 16-token half,
// whose page lookup is wave-uniform, through buffer descriptors that end
// after the chunk's last visible key, so nothing past it is read. The loader
// widens the codes once for the whole workgroup (exact: keys to bf16, values
// to fp16) before they go to LDS, so the 4 waves read ready MFMA operands:
// keys with 16-byte reads, values with the transposing reads of gfx950
// (ds_read_b64_tr_b16), which hand each lane 4 consecutive tokens of one
// head-dim column. The key scales go to LDS already multiplied by
// softmax_scale * log2(e); the waves read the scales as four consecutive
// tokens per lane. Workgroups of one (request, KV head) run on one XCD, the
// deepest query blocks first.
// Instruction mix: a wave hides about two cheap vector instructions behind
// each MFMA of its own instruction stream; giving the MFMA and the vector
// phases to different waves of a SIMD instead leaves each vector phase
// waiting on its own dependency chains. So each wave interleaves its own
// work: row tile j's PV MFMAs are issued between the
// exponentials of row tile j + 1, and the last row tile's between the
// loader's conversions of the next tile; the softmax's rare rescale is one
// branch for all row tiles, so the rest of a tile is one block of code.
// Occupancy: 2 waves per SIMD (the registers hold a tile's V operands).
// Selected blocks (SP): the page table lists the blocks a request selected,
// in position order, with a count of valid keys per entry (from the block's
// start), as in the decode over selected blocks; positions are virtual
// (offset j % bs of selected block j / bs) and the chunk is causal on them.
// A loader wave bounds its half by the block's count, so a partial block's
// tail is never read, and publishes the half's key count in LDS. The
// unmasked steps end at the first tile with a partial half; it and every
// later tile take the masked path, where a position past its block's count
// is no key and adds exactly nothing (a row may see no key in a tile, or
// at all: its output is then 0).
// Key groups (KG = 2, dense head_dim 128, chosen by the host when there are
// at most as many query blocks as CUs): the workgroup is 2 groups of 4 waves;
// group g walks tiles [g T / 2, (g + 1) T / 2) of the block's T key tiles
// with its own LDS buffers (four: its loader runs two tiles ahead), all 8
// waves meeting at a barrier every second tile, and the groups' normalized
// rows are merged into group 0 by their log2 sum-exp through LDS. A row may see no key in a group's tiles (its masked
// probabilities are zero and its sum-exp is kNeg, weight 0).
// The prefill kernel keeps a row's running maximum until a tile's scores
// exceed it by more than kLazyMax (log2 units), so p = exp2(s - m) stays
// below 2^kLazyMax; its P' range factor is 2^(141 - kLazyMax - e), which
// keeps P' below 2^15 as in the decode kernel. The score enters the
// exponent as one fused multiply-add, s * k_scale' - m; a key a row does
// not see gets kNeg, whose exp2 is exactly 0.
#include <hip/hip_runtime.h>

#include "attn_tile.h"
#include "fp8kv_device.h"
#include "fp8kv_internal.h"

namespace fp8kv {
namespace {

constexpr int kLazyMax = 8;

// PV A operand of a lane from the fp16 value rows: two transposing 8-byte
// reads (gfx950 ds_read_b64_tr_b16), the second `second` bytes further.
// Within each 16-lane group, lane 4 a + b receives element b of the 8-byte
// rows that lanes a, a + 4, a + 8, a + 12 address, in that order.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f16x8 read_v_operand(const uint8_t* src, int second) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    const lds_u8* p = (const lds_u8*)src;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + second));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(f16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
}

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// maximum of 8 scores as a chain of three-input maxima (4 instructions)
__device__ __forceinline__ float max8_chain(const float (&v)[2][4]) {
    const float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[0][0], v[0][1]), v[0][2]);
    const float b = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[0][3], v[1][0]), v[1][1]);
    const float c = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[1][2], v[1][3]), a);
    return __builtin_elementwise_maximum(b, c);
}

template <int D, bool BSP2, int NT, bool SP, int KG>
__global__ __launch_bounds__(256 * KG, 2 / KG) void prefill_kernel(PrefillParams p) {
    constexpr int KSTEPS = D / 32;
    constexpr int DL = D / 16;
    constexpr int LROW = 288;                 // LDS row of one key or value (16-bit values)
    constexpr int CPR = D / 16;               // 16-byte chunks per code row
    constexpr int TPL = 64 / CPR;             // tokens one loader wave moves
    constexpr int LOAD_WAVES = 32 / TPL;
    static_assert(D <= 128, "a widened row fits the 256 bytes of data of an LDS row");
    static_assert(TPL <= 16 && 16 % TPL == 0, "a loader wave stays inside one half");
    // LDS of key group g: NBUF tile buffers of the tile's keys widened to
    // bf16, then NBUF of its values widened to fp16, one 288-byte row per
    // token (head-dim columns 8 c .. 8 c + 7 in 16-byte chunk c, chunks
    // permuted per row: K chunk c of token T at c ^ ((T >> 2) & 3), V chunk c
    // at c ^ ((T >> 2) & 1)); then scales [NBUF][k_scale * score scale |
    // v_scale * kappa][32] and selected-block key counts [NBUF][half]. The row pitch
    // and permutations keep every LDS access of the loop free of bank
    // conflicts on gfx950 (the loader's 16-byte stores, the K operand reads,
    // the transposing V operand reads), and the operand addresses of a lane
    // differ only by immediate offsets. With KG > 1 the same bytes later hold
    // the groups' partial results for the merge.
    // Tile buffers: with one key group the loader stores tile t + 1 while
    // tile t is read (two buffers, a barrier every tile); with key groups it
    // stores tile t + 2 while tiles t and t + 1 are read (four buffers, a
    // barrier every second tile: the 8 waves of the workgroup then wait for
    // each other half as often; one 4-wave group per workgroup is faster with
    // a barrier every tile).
    constexpr int AHEAD = KG > 1 ? 2 : 1;
    // one key group: the P' range exponent is fixed before the key loop;
    // key groups keep a running one per group (measured faster there)
    constexpr bool FIXED_EF = KG == 1;
    constexpr int NBUF = 2 * AHEAD;
    constexpr int KT_BYTES = 32 * LROW;
    constexpr int VT_BYTES = 32 * LROW;
    constexpr int TILE_BYTES = NBUF * (KT_BYTES + VT_BYTES + 2 * 32 * 4 + 16);
    constexpr int MERGE_BYTES = KG > 1 ? 4 * 64 * NT * (4 * DL + 2) * 4 : 0;
    constexpr int LDS_BYTES = KG * TILE_BYTES > MERGE_BYTES ? KG * TILE_BYTES : MERGE_BYTES;
    __shared__ __align__(16) uint8_t lds_raw[LDS_BYTES];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int kg = wv >> 2;           // key group: a 1 / KG share of the block's key tiles
    const int wave = wv & 3;          // role in the query block: rows, loader slice
    const int li = lane & 15, lg = lane >> 4;
    uint8_t* const lds_g = lds_raw + kg * TILE_BYTES;
    auto lds_k = [&](int buf) { return lds_g + buf * KT_BYTES; };
    auto lds_v = [&](int buf) { return lds_g + NBUF * KT_BYTES + buf * VT_BYTES; };
    auto lds_s = [&](int buf, int which) {
        return reinterpret_cast<float*>(lds_g + NBUF * (KT_BYTES + VT_BYTES)) + (2 * buf + which) * 32;
    };
    auto lds_nv = [&](int buf) {
        return reinterpret_cast<int*>(lds_g + NBUF * (KT_BYTES + VT_BYTES + 2 * 32 * 4)) + 2 * buf;
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
            // k-step k of lane (i, g): head-dim slots [32 k + 8 g, 32 k + 8 g + 8)
            const uint16_t* qp = p.q + (int64_t)b * p.q_stride_b + (int64_t)tq[j] * p.q_stride_tok +
                                 (int64_t)hq * p.q_stride_head + 8 * lg;
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k)
                qv[j][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * k));
        } else {
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) qv[j][k] = bf16x8{};
        }
    }

    // softmax state of each row tile; the P' range exponent is shared
    WaveState<DL> st[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int n = 0; n < DL; ++n) st[j].acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
        st[j].m_run = kNeg;
        st[j].l_run = 0.f;
    }

    const float* ksbase = p.k_scale + (int64_t)h * p.scale_stride_head;
    const float* vsbase = p.v_scale + (int64_t)h * p.scale_stride_head;
    const int32_t* bt = p.block_tables + (int64_t)b * p.block_table_stride;
    const int32_t* bv = SP ? p.block_valid + (int64_t)b * p.block_valid_stride : nullptr;
    // P' range exponent: the largest exponent field of the value scales of
    // the keys the loader will read (tokens below kv_end; with selected
    // blocks the blocks' valid keys), at least 15; the scales are >= 0, so
    // their bit patterns order as integers. Each thread takes 8 blocks at a
    // time (their table entries first, then all their scales, so that the
    // loads are in flight together); every load stays inside its block and
    // a scale past the block's last key read counts as 0. Each wave's
    // maximum goes to LDS, and every wave takes the maximum of all of them.
    int ef_run = 15;
    if constexpr (FIXED_EF) {
        __shared__ uint32_t wave_max[4];
        constexpr int NTH = 256 * KG;
        uint32_t mx = 0;
        const int nblk = (kv_end + p.block_size - 1) / p.block_size;
        const bool dense16 = p.block_size == 16 && p.scale_stride_slot == 1 &&
                             (reinterpret_cast<uintptr_t>(vsbase) & 15) == 0;
        for (int b0 = 0; b0 < nblk; b0 += 8 * NTH) {
            int blk[8], nv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int bi = b0 + k * NTH + t;
                blk[k] = 0;
                nv[k] = 0;
                if (bi < nblk) {
                    blk[k] = min(max(bt[bi], 0), p.num_blocks - 1);
                    nv[k] = min(p.block_size, kv_end - bi * p.block_size);
                    if (SP) nv[k] = min(nv[k], min(max(bv[bi], 0), p.block_size));
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float* sp = vsbase + (int64_t)blk[k] * p.block_size * p.scale_stride_slot;
                if (dense16) {
                    // the block's 16 scales are 64 contiguous bytes
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint4 u = *reinterpret_cast<const uint4*>(sp + 4 * c);
                        mx = max(mx, 4 * c + 0 < nv[k] ? u.x : 0u);
                        mx = max(mx, 4 * c + 1 < nv[k] ? u.y : 0u);
                        mx = max(mx, 4 * c + 2 < nv[k] ? u.z : 0u);
                        mx = max(mx, 4 * c + 3 < nv[k] ? u.w : 0u);
                    }
                } else {
                    for (int j = 0; j < nv[k]; ++j)
                        mx = max(mx, __float_as_uint(sp[(int64_t)j * p.scale_stride_slot]));
                }
            }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
        mx = rows_max_u32(mx);
        if (lane == 0) wave_max[wv] = mx;
        __syncthreads();
        uint32_t all = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) all = max(all, wave_max[w]);
        ef_run = max((int)(__builtin_amdgcn_readfirstlane(all) >> 23), 15);
    }
    // P' = p * (v_scale * kappa) < 2^kLazyMax * 2^(ef_run - 126) * kappa = 2^15
    const float kappa_wg = pow2i(141 - kLazyMax - ef_run);

    // cooperative tile load, widened once for all waves: lane l of loader
    // wave w moves the 16 K and the 16 V codes of chunk l / TPL of token
    // w TPL + l % TPL (to bf16 and fp16) and reads the token's two scales; its
    // chunk-0 lanes store the key scale, its chunk-1 lanes the value scale
    const bool loader = wave < LOAD_WAVES;
    const int ld_tok = wave * TPL + lane % TPL, ld_chunk = lane / TPL;
    const int ld_half = (wave * TPL) >> 4;
    const int ld_code = (ld_tok & 15) * (int)p.cache_stride_slot + 16 * ld_chunk;
    const int ld_scale = (ld_tok & 15) * (int)p.scale_stride_slot * 4;
    const int kx = (ld_tok >> 2) & 3, vx = (ld_tok >> 2) & 1;
    const int lds_k0 = ld_tok * LROW + 16 * ((2 * ld_chunk) ^ kx);
    const int lds_k1 = ld_tok * LROW + 16 * ((2 * ld_chunk + 1) ^ kx);
    const int lds_v0 = ld_tok * LROW + 16 * ((2 * ld_chunk) ^ vx);
    const int lds_v1 = ld_tok * LROW + 16 * ((2 * ld_chunk + 1) ^ vx);
    // operand reads: K of lane (i, g), k-step k, half s at kq + 64 k + 16 LROW s
    // (token 16 s + i, chunk 4 k + g); V of n-tile n, key half e at
    // vq + 32 n + 16 LROW e (token 16 e + 4 g + i / 4, columns 16 n + 4 (i % 4)
    // .. + 3, which the transposing read hands out as column 16 n + i of the
    // tokens 16 e + 4 g .. 16 e + 4 g + 3)
    const int kq = li * LROW + 16 * (lg ^ (li >> 2));
    const int vq = (4 * lg + (li >> 2)) * LROW + 16 * (((li >> 1) & 1) ^ (lg & 1)) + 8 * (li & 1);
    const uint8_t* kbase = p.k_cache + (int64_t)h * p.cache_stride_head;
    const uint8_t* vbase = p.v_cache + (int64_t)h * p.cache_stride_head;
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
        // 16 codes -> 16 bf16 (K) / fp16 (V) in order (exact), two chunks each
        uint32_t kw[8], vw[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kw[2 * i] = e4m3x2_to_bf16x2<false>((uint32_t)kr[i]);
            kw[2 * i + 1] = e4m3x2_to_bf16x2<true>((uint32_t)kr[i]);
            vw[2 * i] = e4m3x2_to_f16x2<false>((uint32_t)vr[i]);
            vw[2 * i + 1] = e4m3x2_to_f16x2<true>((uint32_t)vr[i]);
        }
        *reinterpret_cast<uint4*>(lds_k(buf) + lds_k0) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
        *reinterpret_cast<uint4*>(lds_k(buf) + lds_k1) = make_uint4(kw[4], kw[5], kw[6], kw[7]);
        *reinterpret_cast<uint4*>(lds_v(buf) + lds_v0) = make_uint4(vw[0], vw[1], vw[2], vw[3]);
        *reinterpret_cast<uint4*>(lds_v(buf) + lds_v1) = make_uint4(vw[4], vw[5], vw[6], vw[7]);
        const float sr = ld_chunk == 0 ? ksr * p.score_scale_log2 : (FIXED_EF ? vsr * kappa_wg : vsr);
        if (ld_chunk < 2) lds_s(buf, ld_chunk)[ld_tok] = sr;
        if (SP && lane == 0 && ((wave * TPL) & 15) == 0) lds_nv(buf)[ld_half] = ld_nv;
    };

    if (loader && ng > 0) {
#pragma unroll
        for (int a = 0; a < AHEAD; ++a) {
            load_tile(tg0 + a);
            store_tile(a);
        }
    }
    __syncthreads();
    // One tile step; MASKED: the visibility test of every score (causal, and
    // with selected blocks the blocks' key counts). All waves of the
    // workgroup take the same steps, one barrier each.
    auto step = [&](int it, auto mask_c) {
        constexpr bool MASKED = decltype(mask_c)::value;
        const int ti = tg0 + it;
        // tile it in buffer it % NBUF; the loader fills buffer (it + AHEAD) %
        // NBUF, whose last readers (step it - AHEAD) passed a barrier since
        const int buf = it & (NBUF - 1);
        // one key group: the step after the last loads and stores a tile
        // with no keys (zero-length buffer ranges), which keeps the loader's
        // work in the same block as the PV MFMAs
        const bool next = KG == 1 || it + AHEAD < ng;
        if (loader && next) load_tile(ti + AHEAD);
        if (it < ng) {
            // K operands: lane (i, g) takes token 16 s + i, head-dim slots
            // [32 k + 8 g, 32 k + 8 g + 8) of k-step k (the q operand's slots)
            bf16x8 ka[KSTEPS][2];
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    ka[k][s] = *reinterpret_cast<const bf16x8*>(lds_k(buf) + kq + 64 * k + 16 * LROW * s);
            // scales of the lane's score tokens 16 s + 4 lg + r
            float sk[2][4], sv[2][4];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const float4 a = *reinterpret_cast<const float4*>(lds_s(buf, 0) + 16 * s + 4 * lg);
                const float4 c = *reinterpret_cast<const float4*>(lds_s(buf, 1) + 16 * s + 4 * lg);
                sk[s][0] = a.x; sk[s][1] = a.y; sk[s][2] = a.z; sk[s][3] = a.w;
                sv[s][0] = c.x; sv[s][1] = c.y; sv[s][2] = c.z; sv[s][3] = c.w;
            }
            // S = K q^T; the k-steps are the outer loop, so the 2 NT
            // accumulation chains take turns
            floatx4 sc[NT][2];
#pragma unroll
            for (int j = 0; j < NT; ++j) sc[j][0] = sc[j][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k)
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        sc[j][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[k][s], qv[j][k], sc[j][s], 0, 0, 0);

            // ---- key groups: P' range of the tile (keys past the chunk have
            // v_scale 0); the scales are >= 0, so their bit patterns order as
            // integers; the range bookkeeping is wave-uniform (scalar)
            bool ef_up = false;
            float fe = 1.0f;
            if constexpr (!FIXED_EF) {
                uint32_t svm = 0;
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int r = 0; r < 4; ++r) svm = max(svm, __float_as_uint(sv[s][r]));
                svm = __builtin_amdgcn_readfirstlane(rows_max_u32(svm));
                const int ef_t = max((int)(svm >> 23), 15);
                const int ef_new = max(ef_run, ef_t);
                ef_up = ef_new > ef_run;
                fe = pow2i(max(ef_run - ef_new, -126));
                ef_run = ef_new;
                const float kappa = pow2i(141 - kLazyMax - ef_run);
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sv[s][r] *= kappa;
            }

            // ---- online softmax of each row tile; P' = p * (v_scale * kappa)
            int nv[2] = {16, 16};
            if (SP) {
                nv[0] = lds_nv(buf)[0];
                nv[1] = lds_nv(buf)[1];
            }
            // key 16 s + 4 lg + r of the tile is visible to row tile j iff
            // 16 s + r <= lim[j] - t0 - 4 lg (and, with selected blocks,
            // 4 lg + r < nv[s])
            auto visible = [&](int j, int s, int r) {
                return 16 * s + r <= lim[j] - (ti << 5) - 4 * lg && (!SP || 4 * lg + r < nv[s]);
            };
            // x = score (log2 units) - running maximum, one rounding; an
            // invisible key gets kNeg, whose exp2 is exactly 0
            float x[NT][2][4];
            bool need = ef_up;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        x[j][s][r] = __builtin_fmaf(sc[j][s][r], sk[s][r], -st[j].m_run);
                        if constexpr (MASKED) x[j][s][r] = visible(j, s, r) ? x[j][s][r] : kNeg;
                    }
                need = need | __any(max8_chain(x[j]) > kLazyMax);
            }
            // lazy maximum: a row tile's running maximum moves only when a
            // score exceeds it by more than kLazyMax, so most tiles skip the
            // rescale (one branch for all row tiles). m_run is the same in the
            // four lanes of a row, so "some lane's scores exceed it" is "some
            // row's scores exceed it". A row that saw no key yet has m_run =
            // kNeg: its visible keys give x = 1e30 and take the branch.
            if (need) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    if (!(__any(max8_chain(x[j]) > kLazyMax) || ef_up)) continue;
                    float s2[2][4];
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            s2[s][r] = sc[j][s][r] * sk[s][r];
                            if constexpr (MASKED) s2[s][r] = visible(j, s, r) ? s2[s][r] : kNeg;
                        }
                    const float m_new = fmax_fin(st[j].m_run, rows_max_fin(max8_chain(s2)));
                    const float a = __builtin_amdgcn_exp2f(st[j].m_run - m_new);
                    const float f = a * fe;
#pragma unroll
                    for (int n = 0; n < DL; ++n) st[j].acc[n] *= f;
                    st[j].l_run *= a;
                    st[j].m_run = m_new;
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            x[j][s][r] = __builtin_fmaf(sc[j][s][r], sk[s][r], -m_new);
                            if constexpr (MASKED) x[j][s][r] = visible(j, s, r) ? x[j][s][r] : kNeg;
                        }
                }
            }
            // P' of row tile j in fp16 (the PV B operand); l accumulates p
            auto make_p = [&](int j) {
                uint32_t pw[4];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float pr[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float e = __builtin_amdgcn_exp2f(x[j][s][r]);
                        st[j].l_run += e;
                        pr[r] = e * sv[s][r];
                    }
                    pw[2 * s] = pack_f16x2(pr[0], pr[1]);
                    pw[2 * s + 1] = pack_f16x2(pr[2], pr[3]);
                }
                return __builtin_bit_cast(f16x8, pw);
            };
            // O^T += V^T P'^T: n-tile n of lane (i, g) is head-dim column
            // 16 n + i over the lane's 8 keys 4 g + r, 16 + 4 g + r (P's order)
            // V operands read once and kept; row tile j's PV MFMAs are
            // issued between the vector work of row tile j + 1's P' (and
            // the last row tile's between the loader's conversions), so
            // the matrix cores and the vector ALU work at the same time
            f16x8 va[DL];
#pragma unroll
            for (int n = 0; n < DL; ++n) va[n] = read_v_operand(lds_v(buf) + vq + 32 * n, 16 * LROW);
            f16x8 pb = make_p(0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const f16x8 pj = pb;
                if (j + 1 < NT) pb = make_p(j + 1);
#pragma unroll
                for (int n = 0; n < DL; ++n)
                    st[j].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[n], pj, st[j].acc[n], 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int n = 0; n < DL; ++n) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
        }
        if (loader && next) store_tile((it + AHEAD) & (NBUF - 1));
        // AHEAD = 2: tile it + 2 was stored in this step or the previous one;
        // a barrier after every odd step makes it visible before step it + 2
        // and keeps step it + 2's store behind step it's readers
        if (AHEAD == 1 || (it & 1)) __syncthreads();
    };
    // tiles every row of the block sees whole: keys up to P + q0
    const int n_clean = min(max(((P + q0 + 1) >> 5) - tg0, 0), ng);
    int it = 0;
    for (; it < n_clean; ++it) {
        if constexpr (SP) {
            // with selected blocks the unmasked steps end at the first tile
            // with a half of fewer than 16 keys (the counts the loader left
            // in LDS before the last barrier); the masked steps take the rest
            const int* nvb = lds_nv(it & (NBUF - 1));
            if (__builtin_amdgcn_readfirstlane(nvb[0] & nvb[1]) != 16) break;
        }
        step(it, BoolC<false>{});
    }
    for (; it < nmax; ++it) step(it, BoolC<true>{});

    // normalized output of row li of each tile: dims 16 n + 4 lg + r
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
                            (int64_t)hq * p.out_stride_head + 4 * lg;
#pragma unroll
        for (int n = 0; n < DL; ++n) {
            const floatx4 v = st[j].acc[n] * inv;
            if (p.out_fp32) {
                *reinterpret_cast<float4*>(static_cast<float*>(p.out) + off + 16 * n) =
                    make_float4(v[0], v[1], v[2], v[3]);
            } else {
                const bf16x2 lo = {(__bf16)v[0], (__bf16)v[1]}, hi = {(__bf16)v[2], (__bf16)v[3]};
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off + 16 * n) =
                    make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
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
    // Every instance runs 2 waves per SIMD (2 query blocks of 4 waves per
    // CU). With at most one query block per CU, dense head_dim 128 splits
    // each block's keys into two key groups (one 8-wave workgroup per CU),
    // merged by log-sum-exp, so the CU still runs 8 waves.
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
    const bool groups = wgs <= (int64_t)cus;
    if (head_dim == 128) {
        if (sp) {
            if (pow2) hipLaunchKernelGGL((prefill_kernel<128, true, NT, true, 1>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((prefill_kernel<128, false, NT, true, 1>), grid, dim3(256), 0, stream, p);
        } else if (groups) {
            if (pow2) hipLaunchKernelGGL((prefill_kernel<128, true, NT, false, 2>), grid, dim3(512), 0, stream, p);
            else hipLaunchKernelGGL((prefill_kernel<128, false, NT, false, 2>), grid, dim3(512), 0, stream, p);
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
