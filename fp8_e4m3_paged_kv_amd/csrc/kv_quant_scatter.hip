// kv_quant_scatter.hip -- fused E4M3 quantize + paged scatter of K and V
// (one launch for both; ATOM #2655 description, K/V bullet; FreeToken #354
// description and its V-pitch fix).
//
// Work unit: one (token, KV head, K-or-V) row of head_dim elements, handled
// by one 16-lane DPP row of a wave64 (head_dim/16 bf16 per lane, one 8- or
// 16-byte load). A wave covers 4 rows per step and 4 steps; all loads of a
// wave are issued before any arithmetic so 64 B per lane are in flight.
//
//   amax  = max |x|              16-lane DPP reduction, exact
//   s     = fp32(amax / 448)     IEEE division
//   c     = E4M3_rne_sat(fp32(x / s)), or E4M3(x) = +-0 when s == 0
//           (the quotient from a per-row reciprocal + one FMA correction)
//   cache[slot, h, :] = c; scale[slot, h] = s     (slot < 0 or >= num_slots:
//                                                   nothing is written)
// K and V are read at their own token/head strides.
#include <hip/hip_runtime.h>

#include "fp8kv_device.h"
#include "fp8kv_internal.h"

namespace fp8kv {
namespace {

constexpr int kQsThreads = 256;
constexpr int kQsSteps = 4;                       // row groups per wave
constexpr int kQsRowsPerWave = 4 * kQsSteps;      // 16 lanes per row
constexpr int kQsRowsPerBlock = kQsRowsPerWave * (kQsThreads / 64);

template <int D>
struct QsVec;
template <>
struct QsVec<128> {               // 8 bf16 per lane = one 16-byte load
    typedef uint4 In;
    typedef uint2 Out;            // 8 codes
};
template <>
struct QsVec<64> {                // 4 bf16 per lane = one 8-byte load
    typedef uint2 In;
    typedef uint32_t Out;         // 4 codes
};

__device__ __forceinline__ void unpack_words(const uint4& v, uint32_t w[4]) {
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
}
__device__ __forceinline__ void unpack_words(const uint2& v, uint32_t w[2]) {
    w[0] = v.x; w[1] = v.y;
}
__device__ __forceinline__ void store_codes(uint8_t* dst, const uint32_t* c, uint2*) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(c[0], c[1]);
}
__device__ __forceinline__ void store_codes(uint8_t* dst, const uint32_t* c, uint32_t*) {
    *reinterpret_cast<uint32_t*>(dst) = c[0];
}

template <int D>
__global__ __launch_bounds__(kQsThreads) void kv_quant_scatter_kernel(QuantScatterParams p) {
#pragma clang fp contract(off)
    constexpr int EPL = D / 16;          // elements per lane
    constexpr int WPL = EPL / 2;         // bf16 pairs (dwords) per lane
    typedef typename QsVec<D>::In In;
    typedef typename QsVec<D>::Out Out;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane >> 4;           // row within a 4-row group
    const int li = lane & 15;            // lane within the row
    const int64_t wave_row0 = (int64_t)blockIdx.x * kQsRowsPerBlock + wave * kQsRowsPerWave;
    const int H = p.num_kv_heads;

    uint32_t w[kQsSteps][WPL];
    int64_t slot[kQsSteps];
    int head[kQsSteps];
    int is_v[kQsSteps];

    // issue every load first
#pragma unroll
    for (int s = 0; s < kQsSteps; ++s) {
        const int64_t r = wave_row0 + 4 * s + sub;
        const bool in_range = r < p.num_rows;
        const int64_t pair = r >> 1;                 // (token, head)
        const int64_t t = in_range ? pair / H : 0;
        const int h = in_range ? (int)(pair - t * H) : 0;
        is_v[s] = (int)(r & 1);
        head[s] = h;
        slot[s] = in_range ? p.slot_ids[t] : -1;
        const uint16_t* src = is_v[s]
            ? p.v + t * p.v_stride_tok + h * p.v_stride_head
            : p.k + t * p.k_stride_tok + h * p.k_stride_head;
        In v = {};
        if (in_range) v = *reinterpret_cast<const In*>(src + li * EPL);
        unpack_words(v, w[s]);
    }

#pragma unroll
    for (int s = 0; s < kQsSteps; ++s) {
        float x[EPL];
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
            x[2 * i] = bf16_lo(w[s][i]);
            x[2 * i + 1] = bf16_hi(w[s][i]);
        }
        uint32_t amax_bits = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            amax_bits = max(amax_bits, __float_as_uint(x[i]) & 0x7FFFFFFFu);
        amax_bits = row16_max_u32(amax_bits);
        const float amax = __uint_as_float(amax_bits);
        const float scale = amax / kE4M3Max;         // IEEE binary32 division
        // x / scale, correctly rounded per element from one IEEE reciprocal
        // and one FMA correction (Markstein): q0 = x*r, e = x - q0*s (exact),
        // q = q0 + e*r, with the sign of x. Rows with a tiny scale are first
        // scaled by 2^64 (exact) so the reciprocal stays finite. Checked
        // exhaustively: for every bf16 row maximum and every bf16 element of
        // either sign up to it in magnitude, the E4M3 code equals that of the
        // IEEE quotient.
        const float f = scale < 0x1p-100f ? 0x1p64f : 1.0f;
        const float ss = scale * f;
        const float rcp = 1.0f / ss;                 // IEEE binary32 division
        uint32_t packed[EPL / 4];
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) packed[i] = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const float xs = x[i] * f;
            const float q0 = xs * rcp;
            const float e = __builtin_fmaf(-q0, ss, xs);
            // the correction turns x = -0 into +0: restore the quotient's sign
            const float qm = __builtin_copysignf(__builtin_fmaf(e, rcp, q0), x[i]);
            const float qv = scale == 0.0f ? x[i] : qm;
            packed[i / 4] |= e4m3_encode(qv) << (8 * (i % 4));
        }
        const int64_t sl = slot[s];
        if (sl >= 0 && sl < p.num_slots) {
            uint8_t* cache = is_v[s] ? p.v_cache : p.k_cache;
            float* planes = is_v[s] ? p.v_scale : p.k_scale;
            uint8_t* dst = cache + sl * p.cache_stride_slot +
                           (int64_t)head[s] * p.cache_stride_head + li * EPL;
            store_codes(dst, packed, (Out*)nullptr);
            if (li == 0)
                planes[sl * p.scale_stride_slot + (int64_t)head[s] * p.scale_stride_head] = scale;
        }
    }
}

}  // namespace

hipError_t launch_kv_quant_scatter(const QuantScatterParams& p, int head_dim,
                                   hipStream_t stream) {
    const int64_t blocks = (p.num_rows + kQsRowsPerBlock - 1) / kQsRowsPerBlock;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks), block(kQsThreads);
    if (head_dim == 128)
        hipLaunchKernelGGL(kv_quant_scatter_kernel<128>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(kv_quant_scatter_kernel<64>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace fp8kv
