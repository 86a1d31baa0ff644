// paged_decode.hip -- paged GQA decode attention over the E4M3 cache.
//
// Semantics (ATOM #2655 description, K/V bullet; sglang-jax #1776,
// "Modifications"): K/V codes are widened exactly to the query's 16-bit
// format before the dot products, the key scale multiplies the score of its
// key, the value scale is folded into the probability before PV, and the
// probabilities are never rounded to the cache format (they are carried in
// fp16, see below).
//
// Decomposition. One workgroup per (request b, KV head h, partition of
// `partition` tokens); its NW waves take interleaved 32-token tiles and are
// merged through LDS at the end; a second kernel merges the partitions by
// log-sum-exp. The M = rows * G query rows that share KV head h (GQA group
// times MTP verify rows) are stacked into the 16-row dimension of the MFMA
// tiles, so each K/V byte is read from HBM once per step.
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
//   biased exponent of the value scales seen by the wave (floored at 14):
//   P' <= 2^15 stays inside fp16's normal range and rescaling on a new
//   exponent is exact (a power of two).
// Memory: each lane reads K as two/one 16-byte loads per token and V as 8
// (or 4) contiguous bytes per token: every 128-byte (64-byte) code row is
// read whole by 4 or 16 lanes. Tokens past the partition end are clamped
// to its last token (never beyond the caller's data) and masked.
#include <hip/hip_runtime.h>

#include "fp8kv_device.h"
#include "fp8kv_internal.h"

namespace fp8kv {
namespace {

constexpr float kNeg = -1.0e30f;     // "minus infinity" that keeps exp2 finite

__device__ __forceinline__ float pow2i(int e) {   // 2^e for e in [-126, 127]
    return __uint_as_float((uint32_t)(e + 127) << 23);
}

__device__ __forceinline__ float xor_max(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask));
}

template <int DL>
struct VRow;
template <>
struct VRow<8> { typedef uint2 T; };
template <>
struct VRow<4> { typedef uint32_t T; };

__device__ __forceinline__ uint32_t vword(const uint2& v, int i) { return i ? v.y : v.x; }
__device__ __forceinline__ uint32_t vword(const uint32_t& v, int) { return v; }

template <int D, int NW, bool SC>
__global__ __launch_bounds__(NW * 64) void decode_partition_kernel(DecodeParams p) {
    constexpr int KB = D / 4;        // K code bytes per lane per token
    constexpr int KV4 = KB / 16;     // 16-byte K loads per token
    constexpr int KSTEPS = D / 32;   // MFMA k-steps over head_dim
    constexpr int DL = D / 16;       // V bytes per lane per token = PV n-tiles
    typedef typename VRow<DL>::T VT;

    __shared__ floatx4 lds_acc[NW / 2][DL][64];
    __shared__ float lds_ml[NW / 2][2][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;
    const int lg = lane >> 4;

    // Unit of this workgroup. Consecutive (request, partition) pairs go to
    // consecutive XCDs (dispatch is round-robin over the 8 XCDs) and the
    // KV heads of one pair stay on one XCD, sharing its L2.
    const int xcd = blockIdx.x & 7;
    const int kx = blockIdx.x >> 3;
    const int pair = (kx / p.num_kv_heads) * 8 + xcd;
    const int h = kx % p.num_kv_heads;
    if (pair >= p.batch * p.num_partitions) return;
    const int b = pair / p.num_partitions;
    const int part = pair - b * p.num_partitions;
    const int len = min(max(p.context_lens[b], 0), p.max_context);
    const int p0 = part * p.partition;
    if (p0 >= len) return;
    const int p1 = min(p0 + p.partition, len);
    const int ntiles = (p1 - p0 + 31) >> 5;

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
    // tokens below full_end are visible to every row
    const int full_end = min(p1, len - p.rows + 1);

    floatx4 acc[DL];
#pragma unroll
    for (int n = 0; n < DL; ++n) acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNeg;
    float l_run = 0.f;
    int ef_run = 14;

    const int64_t h_cache = (int64_t)h * p.cache_stride_head;
    const int64_t h_scale = (int64_t)h * p.scale_stride_head;
    const int32_t* bt = p.block_tables + (int64_t)b * p.block_table_stride;
    const int last_tok = p1 - 1;
    const int last_base = last_tok & ~15;
    const int bs = p.block_size;

    for (int ti = wave; ti < ntiles; ti += NW) {
        const int t0 = p0 + (ti << 5);
        // page walk for the two 16-token halves (wave-uniform)
        int64_t sbase[2];
        int lastoff[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int st = min(t0 + 16 * s, last_base);
            int blk = bt[st / bs];
            blk = min(max(blk, 0), p.num_blocks - 1);
            sbase[s] = (int64_t)blk * bs + (st % bs);
            lastoff[s] = last_tok - st;
        }
        // K codes: token li of each half, bytes [lg*KB, lg*KB + KB)
        uint4 kraw[2][KV4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int64_t slot = sbase[s] + min(li, lastoff[s]);
            const uint8_t* kp = p.k_cache + slot * p.cache_stride_slot + h_cache + lg * KB;
#pragma unroll
            for (int c = 0; c < KV4; ++c) kraw[s][c] = *reinterpret_cast<const uint4*>(kp + 16 * c);
        }
        // V codes: tokens 4g + r of each half (slot e = 4s + r), bytes [li*DL, li*DL + DL)
        VT vraw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = e >> 2;
            const int64_t slot = sbase[s] + min(4 * lg + (e & 3), lastoff[s]);
            vraw[e] = *reinterpret_cast<const VT*>(p.v_cache + slot * p.cache_stride_slot + h_cache + li * DL);
        }
        // row scales of tokens 4g + r
        float sk[2][4], sv[2][4];
        if (SC) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int o4 = min(4 * lg, lastoff[s] & ~3);
                const int64_t idx = sbase[s] + o4 + h_scale;
                const float4 a = *reinterpret_cast<const float4*>(p.k_scale + idx);
                const float4 c = *reinterpret_cast<const float4*>(p.v_scale + idx);
                sk[s][0] = a.x; sk[s][1] = a.y; sk[s][2] = a.z; sk[s][3] = a.w;
                sv[s][0] = c.x; sv[s][1] = c.y; sv[s][2] = c.z; sv[s][3] = c.w;
            }
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t idx = (sbase[s] + min(4 * lg + r, lastoff[s])) * p.scale_stride_slot + h_scale;
                    sk[s][r] = p.k_scale[idx];
                    sv[s][r] = p.v_scale[idx];
                }
        }

        // S = K q^T (fp32 accumulate)
        floatx4 sc[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            sc[s] = floatx4{0.f, 0.f, 0.f, 0.f};
            const uint32_t* kw = reinterpret_cast<const uint32_t*>(kraw[s]);
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) {
                const bf16x8 a = e4m3x8_to_bf16x8(kw[2 * k], kw[2 * k + 1]);
                sc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qv[k], sc[s], 0, 0, 0);
            }
        }

        // scores in log2 units; mask tokens past the partition or the row
        const bool need_mask = t0 + 32 > full_end;
        float s2[2][4];
        float svm = 0.f;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s2[s][r] = sc[s][r] * sk[s][r] * p.score_scale_log2;
                if (need_mask) {
                    const int tok = t0 + 16 * s + 4 * lg + r;
                    const bool valid = tok < p1 && tok <= lim;
                    const bool any_row = tok < p1;
                    s2[s][r] = valid ? s2[s][r] : kNeg;
                    sv[s][r] = any_row ? sv[s][r] : 0.f;
                }
                svm = fmaxf(svm, sv[s][r]);
            }
        float mt = fmaxf(fmaxf(fmaxf(s2[0][0], s2[0][1]), fmaxf(s2[0][2], s2[0][3])),
                         fmaxf(fmaxf(s2[1][0], s2[1][1]), fmaxf(s2[1][2], s2[1][3])));
        mt = xor_max(xor_max(mt, 16), 32);
        svm = xor_max(xor_max(svm, 16), 32);   // wave-uniform now
        const int ef_t = max((int)((__float_as_uint(svm) >> 23) & 0xFF), 14);
        const float m_new = fmaxf(m_run, mt);
        const bool grow = m_new > m_run || ef_t > ef_run;
        if (__any(grow)) {
            const int ef_new = max(ef_run, ef_t);
            const float a = exp2f(m_run - m_new);
            const float f = a * pow2i(max(ef_run - ef_new, -126));
#pragma unroll
            for (int n = 0; n < DL; ++n) acc[n] *= f;
            l_run *= a;
            m_run = m_new;
            ef_run = ef_new;
        }
        const float kappa = pow2i(141 - ef_run);

        // probabilities; P' = p * v_scale * kappa in fp16 (slot e = 4s + r)
        uint32_t pw[4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float e = exp2f(s2[s][r] - m_run);
                if (need_mask) e = s2[s][r] == kNeg ? 0.f : e;
                l_run += e;
                pr[r] = e * (sv[s][r] * kappa);
            }
            pw[2 * s] = pack_f16x2(pr[0], pr[1]);
            pw[2 * s + 1] = pack_f16x2(pr[2], pr[3]);
        }
        const f16x8 pb = __builtin_bit_cast(f16x8, pw);

        // V^T: column c (head-dim 8i + c, or 4i + c) of the lane's 8 tokens
        uint32_t vt[DL][2];
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {              // token slots 4hs .. 4hs+3
#pragma unroll
            for (int w = 0; w < DL / 4; ++w) {        // byte columns 4w .. 4w+3
                uint32_t cols[4];
                transpose4x4(vword(vraw[4 * hs + 0], w), vword(vraw[4 * hs + 1], w),
                             vword(vraw[4 * hs + 2], w), vword(vraw[4 * hs + 3], w), cols);
#pragma unroll
                for (int c = 0; c < 4; ++c) vt[4 * w + c][hs] = cols[c];
            }
        }
#pragma unroll
        for (int n = 0; n < DL; ++n) {
            const f16x8 a = e4m3x8_to_f16x8(vt[n][0], vt[n][1]);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, acc[n], 0, 0, 0);
        }
    }

    // per-wave totals for the lane's row
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    {
        const float kinv = pow2i(max(ef_run - 141, -126));
#pragma unroll
        for (int n = 0; n < DL; ++n) acc[n] *= kinv;
    }

    // merge the NW waves pairwise through LDS (log2(NW) rounds)
#pragma unroll
    for (int half = NW / 2; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) {
            const int slot = wave - half;
#pragma unroll
            for (int n = 0; n < DL; ++n) lds_acc[slot][n][lane] = acc[n];
            lds_ml[slot][0][lane] = m_run;
            lds_ml[slot][1][lane] = l_run;
        }
        __syncthreads();
        if (wave < half) {
            const float mo = lds_ml[wave][0][lane];
            const float lo = lds_ml[wave][1][lane];
            const float mm = fmaxf(m_run, mo);
            const float fa = exp2f(m_run - mm);
            const float fb = exp2f(mo - mm);
#pragma unroll
            for (int n = 0; n < DL; ++n) acc[n] = acc[n] * fa + lds_acc[wave][n][lane] * fb;
            l_run = l_run * fa + lo * fb;
            m_run = mm;
        }
        __syncthreads();
    }

    if (wave == 0 && li < p.m_rows) {
        const int64_t u = (((int64_t)b * p.num_kv_heads + h) * p.num_partitions + part) * p.m_rows + li;
        const bool any = l_run > 0.f;
        const float inv = any ? 1.0f / l_run : 0.f;
        float* o = p.ws_o + u * D + (DL * 4) * lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float vals[DL];
#pragma unroll
            for (int n = 0; n < DL; ++n) vals[n] = acc[n][r] * inv;
#pragma unroll
            for (int c = 0; c < DL / 4; ++c)
                *reinterpret_cast<float4*>(o + DL * r + 4 * c) =
                    make_float4(vals[4 * c], vals[4 * c + 1], vals[4 * c + 2], vals[4 * c + 3]);
        }
        if (lg == 0) p.ws_lse[u] = any ? m_run + __log2f(l_run) : -INFINITY;
    }
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(MergeParams p) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.total_rows) return;
    const int m = row % p.m_rows;
    const int bh = row / p.m_rows;
    const int h = bh % p.num_kv_heads;
    const int b = bh / p.num_kv_heads;
    const int len = min(max(p.context_lens[b], 0), p.max_context);
    const int np = (len + p.partition - 1) / p.partition;
    const int64_t u0 = (int64_t)bh * p.num_partitions * p.m_rows + m;

    float mx = -INFINITY;
    for (int q = 0; q < np; ++q) mx = fmaxf(mx, p.ws_lse[u0 + (int64_t)q * p.m_rows]);
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    float wsum = 0.f;
    if (mx > -INFINITY) {
        for (int q = 0; q < np; ++q) {
            const int64_t u = u0 + (int64_t)q * p.m_rows;
            const float w = exp2f(p.ws_lse[u] - mx);
            wsum += w;
            const float* o = p.ws_o + u * D + lane * PER;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] += w * o[i];
        }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    const int r = m / p.group;
    const int hq = h * p.group + (m - r * p.group);
    const int64_t off = (int64_t)b * p.out_stride_b + (int64_t)r * p.out_stride_row +
                        (int64_t)hq * p.out_stride_head + lane * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const float v = acc[i] * inv;
        if (p.out_fp32) {
            static_cast<float*>(p.out)[off + i] = v;
        } else {
            uint32_t bits = __float_as_uint(v);
            bits += 0x7FFFu + ((bits >> 16) & 1u);      // round to nearest even
            static_cast<uint16_t*>(p.out)[off + i] = (uint16_t)(bits >> 16);
        }
    }
}

template <int D, int NW>
hipError_t launch_partitions_nw(const DecodeParams& p, bool sc, hipStream_t stream) {
    dim3 grid((unsigned)((int64_t)p.pairs_padded * p.num_kv_heads)), block(NW * 64);
    if (sc)
        hipLaunchKernelGGL((decode_partition_kernel<D, NW, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((decode_partition_kernel<D, NW, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_partitions_d(const DecodeParams& p, bool sc, hipStream_t stream) {
    // waves per workgroup: about 8+ tiles of 32 tokens per wave
    if (p.partition >= 4096) return launch_partitions_nw<D, 16>(p, sc, stream);
    if (p.partition >= 2048) return launch_partitions_nw<D, 8>(p, sc, stream);
    return launch_partitions_nw<D, 4>(p, sc, stream);
}

}  // namespace

hipError_t launch_decode_partitions(const DecodeParams& p, int head_dim,
                                    bool scale_contiguous, hipStream_t stream) {
    if (head_dim == 128) return launch_partitions_d<128>(p, scale_contiguous, stream);
    return launch_partitions_d<64>(p, scale_contiguous, stream);
}

hipError_t launch_decode_merge(const MergeParams& p, int head_dim, hipStream_t stream) {
    dim3 grid((unsigned)((p.total_rows + 3) / 4)), block(256);
    if (head_dim == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(decode_merge_kernel<64>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace fp8kv
