// kv_quant_scatter.hip -- fused E4M3 quantize + paged scatter of K and V
// (one launch for both; ATOM #2655 description, K/V bullet; FreeToken #354
// description and its V-pitch fix).
//
// Work unit: one (token, KV head) row of head_dim elements of K or of V
// (grid y), handled by one 16-lane DPP row of a wave64 (head_dim/16 bf16 per
// lane, one 8- or 16-byte load). A wave covers 4 rows per step and 2 steps;
// all loads of a wave are issued before any arithmetic. (K and V pairs in
// one workgroup, half the workgroups with twice the loads in flight per
// lane, took 5% less on the 4096-token prefill chunk but 3-4% more on the
// cache builds.) The bf16 rows are
// read and the code rows written with the non-temporal hint (each byte is
// touched once, so they should not displace anything in L2); the 4-byte
// scale stores stay ordinary so L2 can merge neighbouring rows' scales
// into whole lines before they reach HBM.
//
//   amax  = max |x|              16-lane DPP reduction, exact
//   s     = fp32(amax / 448)     IEEE division
//   c     = E4M3_rne_sat(fp32(x / s)), or E4M3(x) = +-0 when s == 0
//           (the quotient from a per-row reciprocal + one FMA correction)
//   cache[slot, h, :] = c; scale[slot, h] = s     (slot < 0 or >= num_slots:
//                                                   nothing is written)
// K and V are read at their own token/head strides.
//
// The unscaled variants store the values themselves, with no scale:
//   c = E4M3_rne_sat(x) or E5M2_rne_sat(x) (magnitudes above the format's
//   largest finite value saturate to it).
#include <hip/hip_runtime.h>

#include "fp8kv_device.h"
#include "fp8kv_internal.h"

namespace fp8kv {
namespace {

constexpr int kQsThreads = 256;
constexpr int kQsSteps = 2;                       // row groups per wave
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_codes(uint8_t* dst, const uint32_t* c, uint2*) {
    __builtin_nontemporal_store(u32x2{c[0], c[1]}, reinterpret_cast<u32x2*>(dst));
}
__device__ __forceinline__ void store_codes(uint8_t* dst, const uint32_t* c, uint32_t*) {
    __builtin_nontemporal_store(c[0], reinterpret_cast<uint32_t*>(dst));
}

// One lane's bf16 elements of a row, non-temporal.
__device__ __forceinline__ uint4 load_row(const uint16_t* p, uint4*) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load_row(const uint16_t* p, uint2*) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v[0], v[1]);
}

// Row r of K (or of V) is (token r / H, head r % H). HSHIFT = log2(H) when
// H is a power of two (shifts), else -1 (32-bit division).
template <int HSHIFT>
__device__ __forceinline__ void split_row(uint32_t pair, uint32_t H, uint32_t& t, uint32_t& h) {
    if (HSHIFT >= 0) {
        t = pair >> HSHIFT;
        h = pair & ((1u << HSHIFT) - 1u);
    } else {
        t = pair / H;
        h = pair - t * H;
    }
}

template <int D, int HSHIFT, int CODES>
__global__ __launch_bounds__(kQsThreads) void kv_quant_scatter_kernel(QuantScatterParams p) {
#pragma clang fp contract(off)
    constexpr int EPL = D / 16;          // elements per lane
    constexpr int WPL = EPL / 2;         // bf16 pairs (dwords) per lane
    typedef typename QsVec<D>::In In;
    typedef typename QsVec<D>::Out Out;

    // blockIdx.y selects K (0) or V (1): every pointer and stride below is
    // uniform over the workgroup
    const bool is_v = blockIdx.y != 0;
    const uint16_t* src = is_v ? p.v : p.k;
    const int64_t st_tok = is_v ? p.v_stride_tok : p.k_stride_tok;
    const int64_t st_head = is_v ? p.v_stride_head : p.k_stride_head;
    uint8_t* cache = is_v ? p.v_cache : p.k_cache;
    float* planes = is_v ? p.v_scale : p.k_scale;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane >> 4;           // row within a 4-row group
    const int li = lane & 15;            // lane within the row
    // Dispatch deals consecutive workgroups round-robin to the 8 XCDs, each
    // with its own L2. Row blocks are renumbered so that every XCD takes a
    // contiguous eighth of the rows: the 4-byte scales of neighbouring slots
    // then meet in one L2 and leave it as whole lines (gridDim.x is a
    // multiple of 8).
    const uint32_t per_xcd = gridDim.x >> 3;
    const uint32_t block = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
    const uint32_t wave_row0 = block * kQsRowsPerBlock + wave * kQsRowsPerWave;
    const uint32_t H = (uint32_t)p.num_kv_heads;
    const uint32_t nrows = (uint32_t)(p.num_rows >> 1);   // (token, head) rows of K (or V)

    uint32_t w[kQsSteps][WPL];
    int64_t slot[kQsSteps];
    uint32_t head[kQsSteps];
    bool valid[kQsSteps];

    // issue every load first, without branches: rows past the end re-read
    // the last row (nrows >= 1) and are dropped at the store
#pragma unroll
    for (int s = 0; s < kQsSteps; ++s) {
        const uint32_t r = wave_row0 + 4 * s + sub;
        valid[s] = r < nrows;
        uint32_t t, h;
        split_row<HSHIFT>(min(r, nrows - 1), H, t, h);
        head[s] = h;
        slot[s] = p.slot_ids[t];
        const In v = load_row(src + (int64_t)t * st_tok + (int64_t)h * st_head + li * EPL,
                              (In*)nullptr);
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
        uint32_t packed[EPL / 4];
        float scale = 1.0f;
        if constexpr (CODES == kCodesE4M3Scaled) {
            quantize_row_e4m3<EPL>(x, scale, packed);
        } else {
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i)
                packed[i] = CODES == kCodesE5M2
                                ? e5m2x4_encode(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3])
                                : e4m3x4_encode(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
        }
        const int64_t sl = slot[s];
        if (valid[s] && sl >= 0 && sl < p.num_slots) {
            uint8_t* dst = cache + sl * p.cache_stride_slot +
                           (int64_t)head[s] * p.cache_stride_head + li * EPL;
            store_codes(dst, packed, (Out*)nullptr);
            if (CODES == kCodesE4M3Scaled && li == 0)
                planes[sl * p.scale_stride_slot + (int64_t)head[s] * p.scale_stride_head] = scale;
        }
    }
}

}  // namespace

hipError_t launch_kv_quant_scatter(const QuantScatterParams& p, int head_dim,
                                   hipStream_t stream) {
    // rows are numbered in 32 bits; K rows on grid y = 0, V rows on y = 1
    const int64_t kv_rows = p.num_rows / 2;
    if (kv_rows > 0x7FFFFFFF - 8 * kQsRowsPerBlock) return hipErrorInvalidValue;
    // whole multiples of 8 workgroups (the XCD renumbering); the extra ones
    // find no rows
    const int64_t blocks = (kv_rows + 8 * kQsRowsPerBlock - 1) / (8 * kQsRowsPerBlock) * 8;
    dim3 grid((unsigned)blocks, 2), block(kQsThreads);
    const int H = p.num_kv_heads;
    const int hs = (H & (H - 1)) == 0 ? __builtin_ctz((unsigned)H) : -1;
#define FP8KV_QS_LAUNCH(DIM, HS) \
    hipLaunchKernelGGL((kv_quant_scatter_kernel<DIM, HS, kCodesE4M3Scaled>), grid, block, 0, stream, p)
#define FP8KV_QS_DISPATCH(DIM)                                   \
    switch (hs) {                                                \
        case 0: FP8KV_QS_LAUNCH(DIM, 0); break;                  \
        case 1: FP8KV_QS_LAUNCH(DIM, 1); break;                  \
        case 2: FP8KV_QS_LAUNCH(DIM, 2); break;                  \
        case 3: FP8KV_QS_LAUNCH(DIM, 3); break;                  \
        case 4: FP8KV_QS_LAUNCH(DIM, 4); break;                  \
        default: FP8KV_QS_LAUNCH(DIM, -1); break;                \
    }
    if (p.codes != kCodesE4M3Scaled) {
        // unscaled codes: the generic row split only
        const bool e5 = p.codes == kCodesE5M2;
        if (head_dim == 128) {
            if (e5) hipLaunchKernelGGL((kv_quant_scatter_kernel<128, -1, kCodesE5M2>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((kv_quant_scatter_kernel<128, -1, kCodesE4M3>), grid, block, 0, stream, p);
        } else {
            if (e5) hipLaunchKernelGGL((kv_quant_scatter_kernel<64, -1, kCodesE5M2>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((kv_quant_scatter_kernel<64, -1, kCodesE4M3>), grid, block, 0, stream, p);
        }
    } else if (head_dim == 128) {
        FP8KV_QS_DISPATCH(128)
    } else {
        FP8KV_QS_DISPATCH(64)
    }
#undef FP8KV_QS_DISPATCH
#undef FP8KV_QS_LAUNCH
    return hipGetLastError();
}

}  // namespace fp8kv
