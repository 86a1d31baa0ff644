// hbm_probes.hip -- measurement kernels (libfp8kv_probes.so, used by the
// benchmark only, not part of the cache library): plain HBM streams that
// bound what the cache kernels can reach on this GPU, and an empty kernel
// for the launch floor of a replayed HIP graph.
//
//   kind 0  read:   sum of `bytes` (16-byte non-temporal loads)
//   kind 1  copy:   dst = a                      (1:1 read:write)
//   kind 2  2:1:    dst = a ^ b, a and b `bytes` each, dst `bytes`
//   kind 3  write:  dst = pattern                (write only)
//   kind 4  empty:  a kernel that does nothing
//   kind 5  paged read: sum of the 2 KiB blocks of `a` in the order of the
//           int32 block ids `b` (bytes / 2048 of them; a 16-token block of
//           one KV head's 128-byte code rows), one block per wave, one pass
//   kind 6, 7  the same blocks read by one wave per SIMD, each wave walking
//           its share of the ids in groups of U = 4 or 8 blocks (8 or 16
//           KiB: U = 4 is one 32-token tile of K and V codes), the next
//           group's loads issued before the current group is consumed
// fp8kv_probe_ops: instruction-cost probes (no memory traffic but one value
// and one cycle count per wave): every wave runs `iters` iterations of 8
// independent chains of one operation, or of 8 independent 16x16x32 bf16
// MFMA chains with K vector FMAs (or one exp2) beside each MFMA in the same
// instruction stream, or (variant 8) MFMA-only and FMA-only waves
// alternating on each SIMD; see fp8kv_probe_ops below for the variants.
// fp8kv_probe_scatter: the prefill-chunk store's memory traffic without its
// arithmetic (head_dim 128): each (token, KV head) row of K and of V is read
// from its strided source (256 bytes), and 128 bytes (the two 16-byte halves
// of each 32-byte piece xor-ed) go to the row's slot in a head-major code
// pool with the non-temporal hint, plus one ordinary 4-byte store to the
// row's scale plane; 8 lanes per row, 2 row pieces per thread. `mode`
// leaves parts out to attribute the time: bit 0 no code stores, bit 1 no
// scale stores, bit 2 rows read from a dense source (row r at r x 256
// bytes of k, which must then hold 2 x tokens x heads rows) instead of the
// strided slices.
// Every thread moves 2 x 16 bytes: loads carry the non-temporal hint, stores
// are ordinary; the grid covers the buffer once (no grid-stride loop), so
// each wave's loads and stores are 1 KiB contiguous. Of the shapes measured
// over 2 GiB on MI355X (2 to 16 x 16 bytes per thread; grids of 1, 2 or 4
// workgroups per CU looping, or one pass; non-temporal or ordinary
// stores), this one is the fastest for every stream: read 6.96, copy 5.76,
// 2:1 5.71, write 6.58 TB/s (8 x 16 bytes at 2 workgroups per CU with
// non-temporal stores: 6.58, 4.69, 5.11, 5.24).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 2;

__global__ __launch_bounds__(kThreads) void probe_read(const u32x4* a, size_t n, uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    u32x4 acc = {0, 0, 0, 0};
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + u * stride;
            v[u] = j < n ? __builtin_nontemporal_load(a + j) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    // never true for the buffers the bench passes; keeps the loads alive
    if ((acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu) sink[0] = acc.x;
}

__global__ __launch_bounds__(kThreads) void probe_copy(const u32x4* a, u32x4* d, size_t n) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + u * stride;
            if (j < n) v[u] = __builtin_nontemporal_load(a + j);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + u * stride;
            if (j < n) d[j] = v[u];
        }
    }
}

__global__ __launch_bounds__(kThreads) void probe_read2_write1(const u32x4* a, const u32x4* b,
                                                               u32x4* d, size_t n) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride * kUnroll) {
        u32x4 v[kUnroll], w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + u * stride;
            if (j < n) {
                v[u] = __builtin_nontemporal_load(a + j);
                w[u] = __builtin_nontemporal_load(b + j);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + u * stride;
            if (j < n) d[j] = v[u] ^ w[u];
        }
    }
}

__global__ __launch_bounds__(kThreads) void probe_write(u32x4* d, size_t n) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride * kUnroll) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + u * stride;
            if (j < n) d[j] = u32x4{(uint32_t)j, 1u, 2u, 3u};
        }
    }
}

__global__ void probe_empty() {}

// one 2 KiB block per wave; ids are clamped to the buffer's blocks
__global__ __launch_bounds__(kThreads) void probe_paged_read(const u32x4* a, const int32_t* ids,
                                                             uint32_t nblk, uint32_t* sink) {
    const uint32_t w = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    u32x4 acc = {0, 0, 0, 0};
    if (w < nblk) {
        const uint32_t id = min((uint32_t)ids[w], nblk - 1);
        const u32x4* q = a + (size_t)id * 128 + lane;
        acc = __builtin_nontemporal_load(q) ^ __builtin_nontemporal_load(q + 64);
    }
    if ((acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu) sink[0] = acc.x;
}

template <int U>
struct BlockGroup {
    u32x4 v[U][2];
    __device__ __forceinline__ void load(const u32x4* a, const int32_t* ids, uint32_t i, uint32_t b1,
                                         uint32_t nblk, int lane) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t id = min((uint32_t)ids[min(i + u, b1 - 1)], nblk - 1);
            const u32x4* q = a + (size_t)id * 128 + lane;
            v[u][0] = __builtin_nontemporal_load(q);
            v[u][1] = __builtin_nontemporal_load(q + 64);
        }
    }
    __device__ __forceinline__ void consume(u32x4& acc) const {
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1];
    }
};

// one wave per SIMD; the wave's share of the ids in groups of U blocks,
// the next group's loads issued before the current group is consumed (the
// decode kernel's one-tile-ahead pipeline without its arithmetic)
template <int U>
__global__ __launch_bounds__(kThreads) void probe_paged_read_persistent(const u32x4* a,
                                                                        const int32_t* ids,
                                                                        uint32_t nblk,
                                                                        uint32_t* sink) {
    const uint32_t waves = gridDim.x * (kThreads / 64);
    const uint32_t w = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t per = (nblk + waves - 1) / waves;
    const uint32_t b0 = min(w * per, nblk), b1 = min(b0 + per, nblk);
    u32x4 acc = {0, 0, 0, 0};
    if (b0 < b1) {
        BlockGroup<U> g0, g1;
        g0.load(a, ids, b0, b1, nblk, lane);
        uint32_t i = b0;
        for (;;) {
            if (i + U >= b1) { g0.consume(acc); break; }
            g1.load(a, ids, i + U, b1, nblk, lane);
            g0.consume(acc);
            i += U;
            if (i + U >= b1) { g1.consume(acc); break; }
            g0.load(a, ids, i + U, b1, nblk, lane);
            g1.consume(acc);
            i += U;
        }
    }
    if ((acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu) sink[0] = acc.x;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// OP: 0 exp2 f32 (+ multiply), 1 exp2 f16 (+ multiply), 2 FMA;
// MF: MFMA chains, with K FMAs (OP 2) or K exp2 (OP 0) per MFMA in the same
// wave; SPLIT (8-wave workgroups, one per CU): waves 4..7 run only the FMAs
// (K per MFMA slot), waves 0..3 only the MFMAs, so each SIMD holds one wave
// of each kind (the role is wave-uniform: each wave issues one kind)
template <int OP, bool MF, int K, bool SPLIT>
__global__ __launch_bounds__(512) void probe_ops(float* out, unsigned long long* cyc, int iters) {
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    bf16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (t + i));
        b[i] = (__bf16)(0.002f * (t - i));
    }
    floatx4_t acc[8];
    for (int c = 0; c < 8; ++c) acc[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    float x[8];
    _Float16 hx[8];
    for (int k = 0; k < 8; ++k) {
        x[k] = 0.001f * (t + k);
        hx[k] = (_Float16)(0.001f * (t + k));
    }
    const float y = 0.9999f, z = 0.0001f;
    auto valu_op = [&](int k) {
        if (OP == 0) x[k] = __builtin_amdgcn_exp2f(x[k]) * 0.5f;
        else if (OP == 1) hx[k] = __builtin_exp2f16(hx[k]) * (_Float16)0.5f;
        else x[k] = __builtin_fmaf(x[k], y, z);
    };
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    if (SPLIT && wave >= 4) {
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < 8 * K; ++c) valu_op(c & 7);
    } else {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (MF) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
                if (!SPLIT) {
                    constexpr int per = MF ? K : 1;
#pragma unroll
                    for (int j = 0; j < per; ++j) valu_op((c * per + j) & 7);
                }
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    float s = 0.f;
    for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    for (int k = 0; k < 8; ++k) s += x[k] + (float)hx[k];
    const int w = blockIdx.x * (blockDim.x >> 6) + (t >> 6);
    if ((t & 63) == 0) {
        out[w] = s;
        cyc[w] = t1 - t0;
    }
}

struct ScatterArgs {
    const uint16_t* k;
    const uint16_t* v;
    int64_t tok_stride, head_stride;     // source strides, elements
    const int64_t* slots;
    uint8_t* kpool;
    uint8_t* vpool;
    int64_t pool_head_stride, pool_slot_stride;   // bytes
    float* kplane;
    float* vplane;
    int64_t plane_head_stride, plane_slot_stride; // elements
    int64_t num_slots;
    uint32_t units;                      // 2 x tokens x heads x 8
    uint32_t heads, kv_rows;             // kv_rows = tokens x heads
    uint32_t mode;
};

__global__ __launch_bounds__(kThreads) void probe_scatter_rows(ScatterArgs a) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t j = blockIdx.x * kThreads * kUnroll + u * kThreads + threadIdx.x;
        if (j >= a.units) continue;
        const uint32_t row = j >> 3, piece = j & 7;
        const bool is_v = row >= a.kv_rows;
        const uint32_t r = is_v ? row - a.kv_rows : row;
        const uint32_t t = r / a.heads, h = r - t * a.heads;
        const int64_t slot = min(max(a.slots[t], (int64_t)0), a.num_slots - 1);
        const uint16_t* src = (a.mode & 4) ? a.k + (int64_t)row * 128 + 16 * piece
                                            : (is_v ? a.v : a.k) + (int64_t)t * a.tok_stride +
                                                  (int64_t)h * a.head_stride + 16 * piece;
        const u32x4 x0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        const u32x4 x1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + 1);
        uint8_t* dst = (is_v ? a.vpool : a.kpool) + (int64_t)h * a.pool_head_stride +
                       slot * a.pool_slot_stride + 16 * piece;
        if (!(a.mode & 1)) __builtin_nontemporal_store(x0 ^ x1, reinterpret_cast<u32x4*>(dst));
        if (piece == 0 && !(a.mode & 2))
            (is_v ? a.vplane : a.kplane)[(int64_t)h * a.plane_head_stride + slot * a.plane_slot_stride] =
                __uint_as_float(x0.x & 0x3FFFFFFFu);
    }
}

}  // namespace

extern "C" {

// Enqueue one probe kernel on `stream`. bytes: the size of each buffer (a
// multiple of 16). Returns 0, or -1 for a bad argument, -2 for a launch
// error.
int fp8kv_probe(int kind, const void* a, const void* b, void* dst, size_t bytes, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind == 4) {
        hipLaunchKernelGGL(probe_empty, dim3(1), dim3(64), 0, s);
        return hipGetLastError() == hipSuccess ? 0 : -2;
    }
    if (bytes % 16 != 0 || bytes == 0) return -1;
    if (kind >= 5 && kind <= 7) {
        // b: bytes / 2048 int32 block ids
        if (!a || !b || !dst || bytes % 2048 != 0 || bytes / 2048 > 0x7FFFFFFFu) return -1;
        const uint32_t nblk = (uint32_t)(bytes / 2048);
        const int32_t* ids = static_cast<const int32_t*>(b);
        uint32_t* sink = static_cast<uint32_t*>(dst);
        const u32x4* va = static_cast<const u32x4*>(a);
        if (kind == 5) {
            const uint32_t wgs = (nblk + kThreads / 64 - 1) / (kThreads / 64);
            hipLaunchKernelGGL(probe_paged_read, dim3(wgs), dim3(kThreads), 0, s, va, ids, nblk, sink);
        } else {
            int dev = 0, cus = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                cus <= 0)
                return -2;
            if (kind == 6)
                hipLaunchKernelGGL(probe_paged_read_persistent<4>, dim3(cus), dim3(kThreads), 0, s, va, ids,
                                   nblk, sink);
            else
                hipLaunchKernelGGL(probe_paged_read_persistent<8>, dim3(cus), dim3(kThreads), 0, s, va, ids,
                                   nblk, sink);
        }
        return hipGetLastError() == hipSuccess ? 0 : -2;
    }
    const size_t n = bytes / 16;
    const size_t per_block = (size_t)kThreads * kUnroll;
    const size_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFu) return -1;
    const dim3 grid((unsigned)blocks), block(kThreads);
    const u32x4* va = static_cast<const u32x4*>(a);
    switch (kind) {
        case 0:
            if (!a || !dst) return -1;
            hipLaunchKernelGGL(probe_read, grid, block, 0, s, va, n, static_cast<uint32_t*>(dst));
            break;
        case 1:
            if (!a || !dst) return -1;
            hipLaunchKernelGGL(probe_copy, grid, block, 0, s, va, static_cast<u32x4*>(dst), n);
            break;
        case 2:
            if (!a || !b || !dst) return -1;
            hipLaunchKernelGGL(probe_read2_write1, grid, block, 0, s, va,
                               static_cast<const u32x4*>(b), static_cast<u32x4*>(dst), n);
            break;
        case 3:
            if (!dst) return -1;
            hipLaunchKernelGGL(probe_write, grid, block, 0, s, static_cast<u32x4*>(dst), n);
            break;
        default:
            return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Instruction-cost probe `variant` over `blocks` workgroups of 4 waves
// (blocks = CUs x waves per SIMD; variants 8 and 9 take blocks / 2
// workgroups of 8 waves, blocks even); out and cyc hold blocks x 4 entries.
//   0  8 exp2 f32 chains        1  8 exp2 f16 chains      2  8 FMA chains
//   3  8 MFMA chains            4  + 2 FMA per MFMA       5  + 4 FMA per MFMA
//   6  + 1 exp2 per MFMA        7  + 3 FMA per MFMA
//   8  MFMA-only waves and FMA-only waves (2 FMAs per MFMA slot) alternating,
//   9  FMA-only waves of variant 8 alone (16 FMA chains' worth per iteration)
// Returns 0, -1 for a bad argument, -2 for a launch error.
int fp8kv_probe_ops(int variant, float* out, unsigned long long* cyc, int iters, int blocks, void* stream) {
    if (!out || !cyc || iters <= 0 || blocks <= 0) return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g((unsigned)blocks), b(256);
    switch (variant) {
        case 0: hipLaunchKernelGGL((probe_ops<0, false, 1, false>), g, b, 0, s, out, cyc, iters); break;
        case 1: hipLaunchKernelGGL((probe_ops<1, false, 1, false>), g, b, 0, s, out, cyc, iters); break;
        case 2: hipLaunchKernelGGL((probe_ops<2, false, 1, false>), g, b, 0, s, out, cyc, iters); break;
        case 3: hipLaunchKernelGGL((probe_ops<2, true, 0, false>), g, b, 0, s, out, cyc, iters); break;
        case 4: hipLaunchKernelGGL((probe_ops<2, true, 2, false>), g, b, 0, s, out, cyc, iters); break;
        case 5: hipLaunchKernelGGL((probe_ops<2, true, 4, false>), g, b, 0, s, out, cyc, iters); break;
        case 6: hipLaunchKernelGGL((probe_ops<0, true, 1, false>), g, b, 0, s, out, cyc, iters); break;
        case 7: hipLaunchKernelGGL((probe_ops<2, true, 3, false>), g, b, 0, s, out, cyc, iters); break;
        case 8:
        case 9:
            if (blocks % 2) return -1;
            if (variant == 8)
                hipLaunchKernelGGL((probe_ops<2, true, 2, true>), dim3((unsigned)blocks / 2), dim3(512), 0, s,
                                   out, cyc, iters);
            else
                hipLaunchKernelGGL((probe_ops<2, false, 2, true>), dim3((unsigned)blocks / 2), dim3(512), 0, s,
                                   out, cyc, iters);
            break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// The prefill-chunk store's traffic (see probe_scatter_rows) for `tokens`
// tokens of `heads` KV heads, head_dim 128, parts left out by `mode`. Returns 0, -1 for a bad argument,
// -2 for a launch error.
int fp8kv_probe_scatter(const void* k, const void* v, int64_t tok_stride, int64_t head_stride,
                        const int64_t* slots, int tokens, int heads, void* kpool, void* vpool,
                        int64_t pool_head_stride, int64_t pool_slot_stride, void* kplane,
                        void* vplane, int64_t plane_head_stride, int64_t plane_slot_stride,
                        int64_t num_slots, int mode, void* stream) {
    if (!k || !v || !slots || !kpool || !vpool || !kplane || !vplane || tokens <= 0 || heads <= 0 ||
        num_slots <= 0 || (int64_t)tokens * heads * 16 > 0x7FFFFFFF)
        return -1;
    ScatterArgs a{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), tok_stride,
                  head_stride, slots, static_cast<uint8_t*>(kpool), static_cast<uint8_t*>(vpool),
                  pool_head_stride, pool_slot_stride, static_cast<float*>(kplane),
                  static_cast<float*>(vplane), plane_head_stride, plane_slot_stride, num_slots,
                  (uint32_t)tokens * (uint32_t)heads * 16u, (uint32_t)heads,
                  (uint32_t)tokens * (uint32_t)heads, (uint32_t)mode};
    const uint32_t per_block = kThreads * kUnroll;
    const uint32_t blocks = (a.units + per_block - 1) / per_block;
    hipLaunchKernelGGL(probe_scatter_rows, dim3(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
