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
// consecutive ids. Where a range goes on into the next request, the
// loads of that piece's first tile (and its q and first block-table window)
// are issued during the current piece's last tile, so the stream does not
// stop at the boundary. A second kernel merges each request's pieces by
// log-sum-exp. The four waves of a workgroup are four KV heads of one
// range, and the workgroups of a range sit on one XCD, so a tile's K/V
// rows for all heads are read through one L2 at about the same time.
// The M = rows * G query rows that share KV head h (GQA group times MTP
// verify rows) are stacked into the 16-row dimension of the MFMA tiles, so
// each K/V byte is read from HBM once per step.
//
// The tile math (operand layouts, widening, softmax, PV) is in attn_tile.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_tile.h"
#include "fp8kv_device.h"
#include "fp8kv_internal.h"

// The decode partials of fp8kv_paged_decode_attn_fp8_noalloc: a device array
// of fixed size that every GPU the library runs on holds until the process
// ends. In host code this name is only a stand-in for the device symbol;
// its device address comes from fp8kv::noalloc_scratch().
static __device__ __align__(256) unsigned char scratch[fp8kv::kNoAllocScratchBytes];

namespace fp8kv {
namespace {


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

// Append: the new K and V rows of request b at positions [n0, n1) (verify
// row r = position - (len - rows)) for KV head h, quantized by the cache's
// row quantizer and stored at the slots the page walk reads (block ids
// clamped to the pool). Two positions per pass: DPP row g holds the K
// (g even) or V (g odd) row of position pos0 + g / 2. A pass is split into
// its loads (append_load) and its quantization and stores (append_store),
// so a wave can issue a tile's loads in between.
template <int D>
struct NewRows {
    uint32_t w[D / 32];         // the lane's D/16 bf16 of its DPP row's K or V row
    int64_t slot;
    bool live;
};

template <int D, bool BSP2>
__device__ __forceinline__ void append_load(const DecodeParams& p, const int32_t* bt, int b,
                                            int len, int pos0, int n1, int h, int lane,
                                            NewRows<D>& nr) {
    constexpr int EPL = D / 16;                 // elements per lane
    const int li = lane & 15, sub = lane >> 4;
    const bool is_v = sub & 1;
    nr.live = pos0 + (sub >> 1) < n1;
    const int pos = nr.live ? pos0 + (sub >> 1) : n1 - 1;
    const uint16_t* row =
        is_v ? p.v_new + (int64_t)b * p.vn_stride_b + (int64_t)h * p.vn_stride_head +
                   (int64_t)(pos - (len - p.rows)) * p.vn_stride_row
             : p.k_new + (int64_t)b * p.kn_stride_b + (int64_t)h * p.kn_stride_head +
                   (int64_t)(pos - (len - p.rows)) * p.kn_stride_row;
    if constexpr (EPL == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + li * EPL);
        nr.w[0] = v.x; nr.w[1] = v.y; nr.w[2] = v.z; nr.w[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(row + li * EPL);
        nr.w[0] = v.x; nr.w[1] = v.y;
    }
    const int bi = BSP2 ? (pos >> p.block_shift) : pos / p.block_size;
    const int bo = pos - bi * p.block_size;
    const int blk = min(max(bt[bi], 0), p.num_blocks - 1);
    nr.slot = (int64_t)blk * p.block_size + bo;
}

template <int D>
__device__ __forceinline__ void append_store(const DecodeParams& p, int h, int lane,
                                             const NewRows<D>& nr) {
    constexpr int EPL = D / 16;
    const int li = lane & 15;
    const bool is_v = (lane >> 4) & 1;
    float x[EPL];
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) {
        x[2 * i] = bf16_lo(nr.w[i]);
        x[2 * i + 1] = bf16_hi(nr.w[i]);
    }
    float scale;
    uint32_t packed[EPL / 4];
    quantize_row_e4m3<EPL>(x, scale, packed);
    if (nr.live) {
        uint8_t* dst = const_cast<uint8_t*>(is_v ? p.v_cache : p.k_cache) +
                       (int64_t)h * p.cache_stride_head + nr.slot * p.cache_stride_slot + li * EPL;
        if constexpr (EPL == 8)
            *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
        else
            *reinterpret_cast<uint32_t*>(dst) = packed[0];
        if (li == 0)
            const_cast<float*>(is_v ? p.v_scale : p.k_scale)[(int64_t)h * p.scale_stride_head +
                                                            nr.slot * p.scale_stride_slot] = scale;
    }
}

// The wave's own appended rows are complete before its next loads are
// issued: the stores have reached the XCD's L2 (the CU's vector L1 is kept
// coherent with the CU's own stores), so the tile loads read the new codes.
__device__ __forceinline__ void appended_rows_visible() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
}

// One piece: tiles [ja, jb) of request b for KV head h, reduced to a partial
// (normalized output and log2 log-sum-exp of each of the M rows) at piece
// id `pid`. With APPEND, the request's new rows that fall in the piece are
// first written to the cache (append_load, append_store).
// The next piece of a wave's range (request b + 1 from its first tile),
// when the range goes on into it.
struct NextPiece {
    bool valid;
    int b, len, jb;
};

// A wave's tile registers, kept across the pieces of its range: the two
// tile register sets and descriptors of the A/B pipeline and the q operand.
// When `ready`, a piece's last tile has already issued the next piece's
// first tile (into set B if `first_in_b`, else A) and loaded its q, and
// `btw` / `bvw` hold the next piece's first block-table window.
template <int D, int CODES>
struct WaveTiles {
    typename DecodeTile<D, CODES>::Regs ra, rb;
    TileAddr ta_a, ta_b;
    bf16x8 qv[D / 32];
    bool ready, first_in_b;
    int btw, bvw;
};

// Page-walk constants of piece [ja, jb) of request b (length len) for KV head h.
template <int D, int CODES>
__device__ __forceinline__ typename DecodeTile<D, CODES>::WalkConsts piece_walk(
    const DecodeParams& p, int b, int len, int ja, int jb, int h) {
    typename DecodeTile<D, CODES>::WalkConsts w;
    const int p1 = min(jb << 5, len);
    w.kbase = p.k_cache + (int64_t)h * p.cache_stride_head;
    w.vbase = p.v_cache + (int64_t)h * p.cache_stride_head;
    w.ksbase = p.k_scale + (int64_t)h * p.scale_stride_head;
    w.vsbase = p.v_scale + (int64_t)h * p.scale_stride_head;
    w.bt = p.block_tables + (int64_t)b * p.block_table_stride;
    w.bv = p.block_valid ? p.block_valid + (int64_t)b * p.block_valid_stride : nullptr;
    w.p0 = ja << 5;
    w.p1 = p1;
    w.ntiles = jb - ja;
    // tokens below full_end are visible to every row
    w.full_end = min(p1, len - p.rows + 1);
    w.last_base = (p1 - 1) & ~15;
    w.nr_codes_full = 15 * (int)p.cache_stride_slot + D;
    w.nr_scales_full = 4 * (15 * (int)p.scale_stride_slot + 1);
    return w;
}

// q operand of row li of the stacked (verify row, query head) block of
// request b, KV head h (zeros for the padding rows)
template <int D>
__device__ __forceinline__ void load_q(const DecodeParams& p, int b, int h, int li, int lg,
                                       bf16x8 (&qv)[D / 32]) {
    if (li < p.m_rows) {
        const int r = li / p.group;
        const int hq = h * p.group + (li - r * p.group);
        const uint16_t* qp = p.q + (int64_t)b * p.q_stride_b + (int64_t)r * p.q_stride_row +
                             (int64_t)hq * p.q_stride_head + lg * (D / 4);
#pragma unroll
        for (int k = 0; k < D / 32; ++k)
            qv[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 8 * k));
    } else {
#pragma unroll
        for (int k = 0; k < D / 32; ++k) qv[k] = bf16x8{};
    }
}

template <int D, bool BSP2, bool SP, int CODES, bool APPEND>
__device__ __forceinline__ void decode_piece(const DecodeParams& p, int b, int len, int ja, int jb,
                                             int h, int pid, int lane, const NextPiece& nx,
                                             WaveTiles<D, CODES>& wt) {
    constexpr int KSTEPS = D / 32;
    constexpr int DL = D / 16;
    constexpr int KB = D / 4;
    typedef DecodeTile<D, CODES> Tile;
    typedef typename Tile::Regs Regs;
    const int li = lane & 15;
    const int lg = lane >> 4;

    const typename Tile::WalkConsts w = piece_walk<D, CODES>(p, b, len, ja, jb, h);
    const int p0 = w.p0, p1 = w.p1, ntiles = w.ntiles;
    const bool ready = wt.ready;

    // new rows in the piece, positions [n0, n1): stored, and made visible
    // before the loads of the first tile that holds one (tile fence_at of
    // the piece). When that is not the first tile, the first pass's loads are
    // issued now and its stores after the first tile's loads, so the wave
    // does not wait for them before it starts streaming. (A piece whose
    // first tile holds a new row is never handed a prefetched first tile.)
    int fence_at = -1, n0 = 0, n1 = 0;
    NewRows<D> nr;
    if constexpr (APPEND) {
        n0 = max(max(len - p.rows, 0), p0);
        n1 = p1;
        if (n0 < n1) {
            fence_at = (n0 >> 5) - ja;
            append_load<D, BSP2>(p, w.bt, b, len, n0, n1, h, lane, nr);
            if (fence_at == 0) {
                append_store<D>(p, h, lane, nr);
                for (int pos0 = n0 + 2; pos0 < n1; pos0 += 2) {
                    append_load<D, BSP2>(p, w.bt, b, len, pos0, n1, h, lane, nr);
                    append_store<D>(p, h, lane, nr);
                }
            }
        }
    }

    // block-table window of tiles 0..31, and the next one when the piece is longer
    int kw = 0;
    int btw = ready ? wt.btw : Tile::template table_window<BSP2>(p, w, w.bt, 0, lane);
    int btn = ntiles > 32 ? Tile::template table_window<BSP2>(p, w, w.bt, 32, lane) : 0;
    int bvw = SP ? (ready ? wt.bvw : Tile::template table_window<BSP2>(p, w, w.bv, 0, lane)) : 0;
    int bvn = SP && ntiles > 32 ? Tile::template table_window<BSP2>(p, w, w.bv, 32, lane) : 0;

    // q operand: row li of the stacked (verify row, query head) block
    bf16x8 (&qv)[KSTEPS] = wt.qv;
    if (!ready) load_q<D>(p, b, h, li, lg, qv);
    const int lim = li < p.m_rows ? len - p.rows + li / p.group : len - 1;   // last token row li sees

    // the next piece's walk and first table window, in flight during this piece
    typename Tile::WalkConsts wn;
    int nbtw = 0, nbvw = 0;
    if (nx.valid) {
        wn = piece_walk<D, CODES>(p, nx.b, nx.len, 0, nx.jb, h);
        nbtw = Tile::template table_window<BSP2>(p, wn, wn.bt, 0, lane);
        if (SP) nbvw = Tile::template table_window<BSP2>(p, wn, wn.bv, 0, lane);
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
    // loads of tile k of the piece; after its last tile, those of the next
    // piece's first tile and its q (the last QK^T has used this piece's), or
    // with no next piece an empty tile
    auto issue_tile = [&](int k, TileAddr& ta, Regs& r) {
        int blk[2], valid[2];
        if (k < ntiles || !nx.valid) {
            entries(k, blk, valid);
            Tile::template address<BSP2, SP>(p, w, k, blk, valid, ta);
            if (APPEND && k == fence_at) appended_rows_visible();
        } else {
            blk[0] = __builtin_amdgcn_readlane(nbtw, 0);
            blk[1] = __builtin_amdgcn_readlane(nbtw, 1);
            valid[0] = SP ? __builtin_amdgcn_readlane(nbvw, 0) : 0;
            valid[1] = SP ? __builtin_amdgcn_readlane(nbvw, 1) : 0;
            Tile::template address<BSP2, SP>(p, wn, 0, blk, valid, ta);
            load_q<D>(p, nx.b, h, li, lg, qv);
        }
        Tile::issue(ta, lo, r);
    };

    // Two tiles in flight: after a tile's QK^T has consumed its K registers,
    // the loads of the next tile are issued, then the tile's softmax and PV
    // run while they are in flight (A/B ping-pong).
    TileAddr& ta_a = wt.ta_a;
    TileAddr& ta_b = wt.ta_b;
    Regs& ra = wt.ra;
    Regs& rb = wt.rb;
    floatx4 sc[2];
    int ti = 0;
    if (!ready) {
        issue_tile(0, ta_a, ra);
    } else if (wt.first_in_b) {
        ra = rb;
        ta_a = ta_b;
    }
    if (APPEND && fence_at > 0) {
        append_store<D>(p, h, lane, nr);
        for (int pos0 = n0 + 2; pos0 < n1; pos0 += 2) {
            append_load<D, BSP2>(p, w.bt, b, len, pos0, n1, h, lane, nr);
            append_store<D>(p, h, lane, nr);
        }
    }
    bool last_in_b = false;        // the tile after the last one went to set B
    while (ti < ntiles) {
        Tile::qk(ra, qv, sc);
        issue_tile(ti + 1, ta_b, rb);
        Tile::template rest<SP>(p, ta_a, ra, sc, p1, lim, lg, st);
        if (++ti >= ntiles) {
            last_in_b = true;
            break;
        }
        Tile::qk(rb, qv, sc);
        issue_tile(ti + 1, ta_a, ra);
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

    // the next piece finds its first tile and q issued, and its table window
    wt.ready = nx.valid;
    wt.first_in_b = last_in_b;
    wt.btw = nbtw;
    wt.bvw = nbvw;
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

template <int D, bool BSP2, bool SP, int CODES, bool APPEND>
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

    // walk the pieces of the range; when the range goes on into the next
    // request, its first tile is loaded during this piece's last one
    int u = u0;
    WaveTiles<D, CODES> wt;
    wt.ready = false;
    wt.first_in_b = false;
    while (u < u1) {
        const int len = min(max(p.context_lens[b], 0), p.max_context);
        const int n = (len + 31) >> 5;
        if (n > 0) {
            const int ja = u - pre;
            const int jb = min(n, u1 - pre);
            NextPiece nx{false, 0, 0, 0};
            // (not over selected blocks, whose pieces are short and whose
            // kernel measured slower with the prefetch)
            if (!SP && pre + jb < u1 && b + 1 < p.batch) {
                const int nlen = min(max(p.context_lens[b + 1], 0), p.max_context);
                const int nn = (nlen + 31) >> 5;
                const int njb = min(nn, u1 - (pre + n));
                // a first tile that holds one of the step's new rows is
                // loaded only after they are stored
                const bool fenced = APPEND && max(nlen - p.rows, 0) < min(njb << 5, nlen) &&
                                    max(nlen - p.rows, 0) < 32;
                nx = NextPiece{nn > 0 && !fenced, b + 1, nlen, njb};
            }
            decode_piece<D, BSP2, SP, CODES, APPEND>(p, b, len, ja, jb, h, b + r, lane, nx, wt);
            u = pre + jb;
        } else {
            wt.ready = false;
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

template <int D, bool BSP2, bool SP, int CODES, bool APPEND>
hipError_t launch_split(const DecodeParams& p, hipStream_t stream) {
    const int64_t workers = (int64_t)p.num_ranges * p.num_kv_heads;
    const int64_t quantum = p.wgs_per_range > 1 ? 8 * p.wgs_per_range : 1;
    int64_t wgs = (workers + 3) / 4;
    wgs = (wgs + quantum - 1) / quantum * quantum;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_split_kernel<D, BSP2, SP, CODES, APPEND>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool SP, int CODES = kCodesE4M3Scaled, bool APPEND = false>
hipError_t launch_split_bs(const DecodeParams& p, hipStream_t stream) {
    return p.block_shift >= 0 ? launch_split<D, true, SP, CODES, APPEND>(p, stream)
                              : launch_split<D, false, SP, CODES, APPEND>(p, stream);
}
}  // namespace


// Address of `scratch` on the current device: each GPU holds its own copy
// at its own address, looked up the first time a call runs on that device
// (with the device current) and cached.
hipError_t noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

int decode_wave_slots(int device) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return 0;
    return cus * 4;                            // one wave per SIMD
}

hipError_t launch_decode_partitions(const DecodeParams& p, int head_dim, hipStream_t stream) {
    const bool sp = p.block_valid != nullptr;
    if (p.k_new != nullptr) {
        // append: the dense walk over a scaled E4M3 cache only
        if (sp || p.codes != kCodesE4M3Scaled) return hipErrorInvalidValue;
        return head_dim == 128 ? launch_split_bs<128, false, kCodesE4M3Scaled, true>(p, stream)
                               : launch_split_bs<64, false, kCodesE4M3Scaled, true>(p, stream);
    }
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
