// fp8kv_api.cpp -- the C ABI of libfp8kv.so: host-side O(1) validation,
// grid sizing and kernel launches. Nothing here touches device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <utility>
#include <vector>

#include "../../include/fp8kv.h"
#include "fp8kv_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return FP8KV_OK;
}

bool aligned(const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

constexpr int kMaxStackedRows = 16; // MFMA M dimension
constexpr int kMaxRanges = 1 << 20;  // bound of the decode split

struct DecodeShape {
    int32_t num_ranges = 0;
    int32_t group = 0;
    int32_t m_rows = 0;
    int64_t pieces = 0;             // batch + num_ranges - 1
    int64_t lse_offset_bytes = 0;
    int64_t prefix_offset_bytes = 0;
    int64_t ws_bytes = 0;
};

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Ranges the library picks for num_ranges == 0: one wave per (range, KV
// head) and one wave per SIMD of the current device.
int auto_ranges(int32_t num_kv_heads, int32_t* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(FP8KV_E_LAUNCH, "no HIP device to size the decode split for");
    const int waves = fp8kv::decode_wave_slots(dev);
    if (waves <= 0)
        return fail(FP8KV_E_LAUNCH, "cannot query the CU count of device %d", dev);
    *out = waves / num_kv_heads > 1 ? waves / num_kv_heads : 1;
    return FP8KV_OK;
}

// Shape rules shared by the workspace query and the calls.
int decode_shape(int32_t batch, int32_t rows, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, int32_t num_ranges,
                 DecodeShape* s) {
    if (head_dim != 64 && head_dim != 128)
        return fail(FP8KV_E_UNSUPPORTED, "head_dim %d: only 64 and 128 are supported", head_dim);
    if (batch < 0)
        return fail(FP8KV_E_SHAPE, "batch (%d) must be >= 0", batch);
    if (rows < 1 || num_q_heads < 1 || num_kv_heads < 1)
        return fail(FP8KV_E_SHAPE, "rows, num_q_heads and num_kv_heads must be >= 1");
    if (num_q_heads % num_kv_heads != 0)
        return fail(FP8KV_E_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    num_q_heads, num_kv_heads);
    const int32_t group = num_q_heads / num_kv_heads;
    if ((int64_t)rows * group > kMaxStackedRows)
        return fail(FP8KV_E_UNSUPPORTED,
                    "rows * (num_q_heads / num_kv_heads) = %d exceeds the %d-row tile",
                    rows * group, kMaxStackedRows);
    if (num_ranges < 0 || num_ranges > kMaxRanges)
        return fail(FP8KV_E_SHAPE, "num_ranges %d: must be 0 (auto) or 1..%d", num_ranges, kMaxRanges);
    int32_t R = num_ranges;
    if (R == 0) {
        const int st = auto_ranges(num_kv_heads, &R);
        if (st != FP8KV_OK) return st;
    }
    s->num_ranges = R;
    s->group = group;
    s->m_rows = rows * group;
    s->pieces = (int64_t)batch + R - 1;
    const int64_t units = s->pieces * num_kv_heads * s->m_rows;
    if (units * head_dim > INT64_C(1) << 40)
        return fail(FP8KV_E_SHAPE, "decode workspace of %lld partial rows is too large",
                    (long long)units);
    s->lse_offset_bytes = round_up(units * head_dim * 4, 256);
    s->prefix_offset_bytes = s->lse_offset_bytes + round_up(units * 4, 256);
    s->ws_bytes = s->prefix_offset_bytes + round_up(((int64_t)batch + 1) * 4, 256);
    return FP8KV_OK;
}

int check_out_dtype(int32_t out_dtype) {
    if (out_dtype != FP8KV_DTYPE_BF16 && out_dtype != FP8KV_DTYPE_FP32)
        return fail(FP8KV_E_UNSUPPORTED, "out_dtype %d: only BF16 and FP32 outputs", out_dtype);
    return FP8KV_OK;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess)
        return fail(FP8KV_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// ---------------------------------------------------------------------------
// Checked mode (fp8kv_set_checked): before a launch, every pointer argument
// must be device memory of the current device, and the device-resident ids
// are copied to the host and range-checked. It synchronizes the stream, so
// it is refused under graph capture. Off by default.
std::atomic<int> g_checked{0};

bool checked() { return g_checked.load(std::memory_order_relaxed) != 0; }

int checked_begin(void* stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) != hipSuccess) {
        (void)hipGetLastError();
        return fail(FP8KV_E_LAUNCH, "checked mode: cannot query the stream's capture state");
    }
    if (cs != hipStreamCaptureStatusNone)
        return fail(FP8KV_E_UNSUPPORTED,
                    "checked mode synchronizes the stream and cannot run under graph capture");
    return FP8KV_OK;
}

int check_device_ptr(const void* ptr, const char* name) {
    if (!ptr) return FP8KV_OK;             // required pointers were refused as NULL before
    hipPointerAttribute_t a;
    const hipError_t e = hipPointerGetAttributes(&a, ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FP8KV_E_NOT_DEVICE, "%s (%p) is not memory the HIP runtime knows", name, ptr);
    }
    if (a.type == hipMemoryTypeManaged || a.isManaged) return FP8KV_OK;
    if (a.type != hipMemoryTypeDevice)
        return fail(FP8KV_E_NOT_DEVICE, "%s (%p) is host memory, not device memory", name, ptr);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(FP8KV_E_LAUNCH, "checked mode: no current HIP device");
    }
    if (a.device != dev)
        return fail(FP8KV_E_NOT_DEVICE, "%s (%p) is on device %d, the current device is %d", name,
                    ptr, a.device, dev);
    return FP8KV_OK;
}

int check_device_ptrs(std::initializer_list<std::pair<const void*, const char*>> ptrs) {
    for (const auto& x : ptrs) {
        const int st = check_device_ptr(x.first, x.second);
        if (st != FP8KV_OK) return st;
    }
    return FP8KV_OK;
}

// Host copy of n device elements once the stream's earlier work is done.
template <class T>
int fetch(std::vector<T>& h, const T* d, int64_t n, void* stream) {
    h.resize(static_cast<size_t>(n));
    if (n == 0) return FP8KV_OK;
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
        e = hipMemcpy(h.data(), d, static_cast<size_t>(n) * sizeof(T), hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FP8KV_E_LAUNCH, "checked mode: reading device ids failed: %s",
                    hipGetErrorString(e));
    }
    return FP8KV_OK;
}

// Context lengths within [0, max_context] and, for every request, the
// table entries of the blocks that hold its tokens within [0, num_blocks);
// with selected blocks also each valid count within [0, block_size] (an
// entry with no valid key is never read, so its id is not checked).
int check_tables(const int32_t* context_lens, const int32_t* block_tables, int64_t bt_stride,
                 const int32_t* block_valid, int64_t bv_stride, int32_t batch,
                 int32_t block_size, int64_t num_blocks, int32_t max_context, void* stream,
                 std::vector<int32_t>* lens_out) {
    std::vector<int32_t> lens, ids, valid;
    int st = fetch(lens, context_lens, batch, stream);
    if (st != FP8KV_OK) return st;
    for (int32_t b = 0; b < batch; ++b) {
        if (lens[b] < 0 || lens[b] > max_context)
            return fail(FP8KV_E_RANGE, "context_lens[%d] = %d is outside [0, max_context = %d]",
                        b, lens[b], max_context);
        const int64_t nb = ((int64_t)lens[b] + block_size - 1) / block_size;
        if ((st = fetch(ids, block_tables + b * bt_stride, nb, stream)) != FP8KV_OK) return st;
        if (block_valid &&
            (st = fetch(valid, block_valid + b * bv_stride, nb, stream)) != FP8KV_OK)
            return st;
        for (int64_t i = 0; i < nb; ++i) {
            if (block_valid) {
                if (valid[i] < 0 || valid[i] > block_size)
                    return fail(FP8KV_E_RANGE, "block_valid[%d][%lld] = %d is outside [0, %d]", b,
                                (long long)i, valid[i], block_size);
                if (valid[i] == 0) continue;
            }
            if (ids[i] < 0 || ids[i] >= num_blocks)
                return fail(FP8KV_E_RANGE, "block_tables[%d][%lld] = %d is outside [0, %lld)", b,
                            (long long)i, ids[i], (long long)num_blocks);
        }
    }
    if (lens_out) *lens_out = std::move(lens);
    return FP8KV_OK;
}

// New K/V rows of fp8kv_paged_decode_append_attn_fp8 (k == nullptr: none).
struct AppendRows {
    const void* k = nullptr;
    int64_t k_sb = 0, k_sr = 0, k_sh = 0;
    const void* v = nullptr;
    int64_t v_sb = 0, v_sr = 0, v_sh = 0;
};

static int decode_partials(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype, const uint8_t* k_cache,
    const uint8_t* v_cache, int64_t cache_stride_slot,
    int64_t cache_stride_head, const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* block_valid, int64_t block_valid_stride,
    const int32_t* context_lens, int32_t batch, int32_t rows,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges,
    int32_t max_context, void* workspace, size_t workspace_bytes,
    int32_t codes, void* stream, const AppendRows& app = AppendRows()) {
    DecodeShape s;
    int st = decode_shape(batch, rows, num_q_heads, num_kv_heads, head_dim, num_ranges, &s);
    if (st != FP8KV_OK) return st;
    const bool scaled = codes == fp8kv::kCodesE4M3Scaled;
    if (q_dtype != FP8KV_DTYPE_BF16)
        return fail(FP8KV_E_UNSUPPORTED, "q_dtype %d: only BF16 queries", q_dtype);
    if (block_size < 16 || block_size % 16 != 0)
        return fail(FP8KV_E_UNSUPPORTED, "block_size %d: must be a positive multiple of 16", block_size);
    if (max_context < 0)
        return fail(FP8KV_E_SHAPE, "max_context (%d) must be >= 0", max_context);
    if ((int64_t)batch * ((max_context + 31) / 32) > INT32_MAX)
        return fail(FP8KV_E_SHAPE, "batch * max_context too large for 32-bit tile counts");
    // no request: nothing is read or written, any pointer may be NULL
    if (batch == 0) return ok();
    if (!q || !k_cache || !v_cache || (scaled && (!k_scale || !v_scale)) || !block_tables ||
        !context_lens)
        return fail(FP8KV_E_NULL, "paged_decode: a required pointer is NULL");
    if (!workspace)
        return fail(FP8KV_E_WORKSPACE, "paged_decode: workspace is NULL");
    if ((int64_t)workspace_bytes < s.ws_bytes)
        return fail(FP8KV_E_WORKSPACE, "workspace %zu bytes < required %lld",
                    workspace_bytes, (long long)s.ws_bytes);
    if (app.k || app.v) {
        // the new rows: bf16 [B, rows, Hkv, D], rows on head_dim/8-byte
        // boundaries (the quantizer's one 16- or 8-byte load per lane)
        const int64_t el = head_dim / 16;
        if (!app.k || !app.v)
            return fail(FP8KV_E_NULL, "paged_decode_append: k_new or v_new is NULL");
        if (app.k_sb < 0 || app.k_sr < 0 || app.k_sh < 0 || app.v_sb < 0 || app.v_sr < 0 ||
            app.v_sh < 0)
            return fail(FP8KV_E_STRIDE, "paged_decode_append: negative new-row stride");
        if (!aligned(app.k, 2 * el) || !aligned(app.v, 2 * el) || app.k_sb % el ||
            app.k_sr % el || app.k_sh % el || app.v_sb % el || app.v_sr % el || app.v_sh % el)
            return fail(FP8KV_E_ALIGN, "new K/V rows must start on %lld-byte boundaries",
                        (long long)(2 * el));
    }
    if (q_stride_b < 0 || q_stride_row < 0 || q_stride_head < 0 ||
        cache_stride_slot < 0 || cache_stride_head < 0 ||
        scale_stride_slot < 0 || scale_stride_head < 0 ||
        block_table_stride < 0 || block_valid_stride < 0)
        return fail(FP8KV_E_STRIDE, "paged_decode: negative stride");
    if (!aligned(q, 16) || q_stride_b % 8 || q_stride_row % 8 || q_stride_head % 8)
        return fail(FP8KV_E_ALIGN, "q rows must start on 16-byte boundaries");
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        cache_stride_slot % 16 || cache_stride_head % 16)
        return fail(FP8KV_E_ALIGN, "cache rows must start on 16-byte boundaries");
    if ((scaled && (!aligned(k_scale, 4) || !aligned(v_scale, 4))) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
        !aligned(block_valid, 4) || !aligned(workspace, 256))
        return fail(FP8KV_E_ALIGN, "scale planes, tables or workspace misaligned");
    const int64_t num_blocks = num_slots / block_size;
    if (batch > 0 && max_context > 0 && num_blocks < 1)
        return fail(FP8KV_E_SHAPE, "num_slots %lld holds no block of %d",
                    (long long)num_slots, block_size);
    if (num_blocks > INT32_MAX)
        return fail(FP8KV_E_SHAPE, "num_slots / block_size exceeds int32 block ids");
    // in-block offsets are 32-bit: 16 slots of codes / scales must fit
    if (cache_stride_slot > (INT32_MAX / 16) || scale_stride_slot > (INT32_MAX / 64))
        return fail(FP8KV_E_SHAPE, "slot stride too large for 32-bit in-block offsets");
    if (checked()) {
        if ((st = checked_begin(stream)) != FP8KV_OK) return st;
        st = check_device_ptrs({{q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"},
                                {k_scale, "k_scale"}, {v_scale, "v_scale"},
                                {block_tables, "block_tables"}, {block_valid, "block_valid"},
                                {context_lens, "context_lens"}, {workspace, "workspace"},
                                {app.k, "k_new"}, {app.v, "v_new"}});
        if (st != FP8KV_OK) return st;
        st = check_tables(context_lens, block_tables, block_table_stride, block_valid,
                          block_valid_stride, batch, block_size, num_blocks, max_context, stream,
                          nullptr);
        if (st != FP8KV_OK) return st;
    }

    fp8kv::DecodeParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.q_stride_b = q_stride_b;
    p.q_stride_row = q_stride_row;
    p.q_stride_head = q_stride_head;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.cache_stride_slot = cache_stride_slot;
    p.cache_stride_head = cache_stride_head;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.scale_stride_slot = scale_stride_slot;
    p.scale_stride_head = scale_stride_head;
    p.block_tables = block_tables;
    p.block_table_stride = block_table_stride;
    p.block_valid = block_valid;
    p.block_valid_stride = block_valid_stride;
    p.context_lens = context_lens;
    p.batch = batch;
    p.rows = rows;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = s.group;
    p.m_rows = s.m_rows;
    p.block_size = block_size;
    p.block_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
    p.max_context = max_context;
    p.num_blocks = (int32_t)(num_blocks > 0 ? num_blocks : 1);
    p.num_ranges = s.num_ranges;
    p.wgs_per_range = (num_kv_heads % 4 == 0 && num_kv_heads > 4) ? num_kv_heads / 4 : 1;
    p.score_scale_log2 = softmax_scale * 1.4426950408889634f;
    p.codes = codes;
    char* ws = static_cast<char*>(workspace);
    p.ws_o = reinterpret_cast<float*>(ws);
    p.ws_lse = reinterpret_cast<float*>(ws + s.lse_offset_bytes);
    p.ws_prefix = reinterpret_cast<int32_t*>(ws + s.prefix_offset_bytes);
    p.k_new = static_cast<const uint16_t*>(app.k);
    p.v_new = static_cast<const uint16_t*>(app.v);
    p.kn_stride_b = app.k_sb;
    p.kn_stride_row = app.k_sr;
    p.kn_stride_head = app.k_sh;
    p.vn_stride_b = app.v_sb;
    p.vn_stride_row = app.v_sr;
    p.vn_stride_head = app.v_sh;
    return launched(fp8kv::launch_decode_partitions(p, head_dim, (hipStream_t)stream),
                    "paged_decode_partials");
}

}  // namespace

extern "C" {

int fp8kv_abi_version(void) { return FP8KV_ABI_VERSION; }

const char* fp8kv_status_string(int status) {
    switch (status) {
        case FP8KV_OK: return "ok";
        case FP8KV_E_NULL: return "null pointer";
        case FP8KV_E_SHAPE: return "bad shape";
        case FP8KV_E_STRIDE: return "bad stride";
        case FP8KV_E_ALIGN: return "misaligned pointer or stride";
        case FP8KV_E_UNSUPPORTED: return "unsupported combination";
        case FP8KV_E_WORKSPACE: return "workspace too small";
        case FP8KV_E_LAUNCH: return "kernel launch failed";
        case FP8KV_E_NOT_DEVICE: return "pointer is not device memory (checked mode)";
        case FP8KV_E_RANGE: return "device id out of range (checked mode)";
        default: return "unknown status";
    }
}

const char* fp8kv_last_error(void) { return g_last_error; }

int fp8kv_set_checked(int enabled) {
    return g_checked.exchange(enabled ? 1 : 0);
}

static int quant_scatter(
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    int32_t in_dtype, int32_t num_tokens, int32_t num_kv_heads,
    int32_t head_dim, const int64_t* slot_ids, uint8_t* k_cache,
    uint8_t* v_cache, int64_t cache_stride_slot, int64_t cache_stride_head,
    float* k_scale, float* v_scale, int64_t scale_stride_slot,
    int64_t scale_stride_head, int64_t num_slots, int32_t codes, void* stream) {
    const bool scaled = codes == fp8kv::kCodesE4M3Scaled;
    if (in_dtype != FP8KV_DTYPE_BF16)
        return fail(FP8KV_E_UNSUPPORTED, "in_dtype %d: only BF16 K/V inputs", in_dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(FP8KV_E_UNSUPPORTED, "head_dim %d: only 64 and 128 are supported", head_dim);
    if (num_tokens < 0 || num_kv_heads < 1 || num_slots < 0)
        return fail(FP8KV_E_SHAPE, "num_tokens %d, num_kv_heads %d, num_slots %lld",
                    num_tokens, num_kv_heads, (long long)num_slots);
    // nothing to store: nothing is read or written, any pointer may be NULL
    if (num_tokens == 0) return ok();
    if (!k || !v || !slot_ids || !k_cache || !v_cache || (scaled && (!k_scale || !v_scale)))
        return fail(FP8KV_E_NULL, "kv_quant_scatter: a required pointer is NULL");
    if (k_stride_tok < 0 || k_stride_head < 0 || v_stride_tok < 0 ||
        v_stride_head < 0 || cache_stride_slot < 0 || cache_stride_head < 0 ||
        scale_stride_slot < 0 || scale_stride_head < 0)
        return fail(FP8KV_E_STRIDE, "kv_quant_scatter: negative stride");
    // each lane moves head_dim/16 bf16 (8 or 16 bytes) and writes
    // head_dim/16 codes; rows must start on those boundaries
    const int64_t in_vec = head_dim / 16;
    if (!aligned(k, in_vec * 2) || !aligned(v, in_vec * 2) ||
        k_stride_tok % in_vec || k_stride_head % in_vec ||
        v_stride_tok % in_vec || v_stride_head % in_vec)
        return fail(FP8KV_E_ALIGN, "K/V rows must start on %lld-byte boundaries",
                    (long long)(in_vec * 2));
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        cache_stride_slot % 16 || cache_stride_head % 16)
        return fail(FP8KV_E_ALIGN, "cache rows must start on 16-byte boundaries");
    if ((scaled && (!aligned(k_scale, 4) || !aligned(v_scale, 4))) || !aligned(slot_ids, 8))
        return fail(FP8KV_E_ALIGN, "scale planes / slot ids misaligned");
    if (checked()) {
        int st = checked_begin(stream);
        if (st != FP8KV_OK) return st;
        st = check_device_ptrs({{k, "k"}, {v, "v"}, {slot_ids, "slot_ids"}, {k_cache, "k_cache"},
                                {v_cache, "v_cache"}, {k_scale, "k_scale"}, {v_scale, "v_scale"}});
        if (st != FP8KV_OK) return st;
        std::vector<int64_t> slots;
        if ((st = fetch(slots, slot_ids, num_tokens, stream)) != FP8KV_OK) return st;
        for (int32_t t = 0; t < num_tokens; ++t)
            if (slots[t] >= num_slots)
                return fail(FP8KV_E_RANGE, "slot_ids[%d] = %lld is not below num_slots = %lld", t,
                            (long long)slots[t], (long long)num_slots);
    }

    fp8kv::QuantScatterParams p;
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.k_stride_tok = k_stride_tok;
    p.k_stride_head = k_stride_head;
    p.v_stride_tok = v_stride_tok;
    p.v_stride_head = v_stride_head;
    p.slot_ids = slot_ids;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.cache_stride_slot = cache_stride_slot;
    p.cache_stride_head = cache_stride_head;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.scale_stride_slot = scale_stride_slot;
    p.scale_stride_head = scale_stride_head;
    p.num_slots = num_slots;
    p.num_tokens = num_tokens;
    p.num_kv_heads = num_kv_heads;
    p.num_rows = (int64_t)num_tokens * num_kv_heads * 2;
    p.codes = codes;
    return launched(fp8kv::launch_kv_quant_scatter(p, head_dim, (hipStream_t)stream),
                    "kv_quant_scatter");
}

int fp8kv_kv_quant_scatter(
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    int32_t in_dtype, int32_t num_tokens, int32_t num_kv_heads,
    int32_t head_dim, const int64_t* slot_ids, uint8_t* k_cache,
    uint8_t* v_cache, int64_t cache_stride_slot, int64_t cache_stride_head,
    float* k_scale, float* v_scale, int64_t scale_stride_slot,
    int64_t scale_stride_head, int64_t num_slots, void* stream) {
    return quant_scatter(k, k_stride_tok, k_stride_head, v, v_stride_tok, v_stride_head,
                         in_dtype, num_tokens, num_kv_heads, head_dim, slot_ids, k_cache,
                         v_cache, cache_stride_slot, cache_stride_head, k_scale, v_scale,
                         scale_stride_slot, scale_stride_head, num_slots,
                         fp8kv::kCodesE4M3Scaled, stream);
}

// FP8KV_CODES_* of the public header -> the kernels' unscaled formats
static int unscaled_codes(int32_t code_format, int32_t* codes) {
    if (code_format == FP8KV_CODES_E4M3) *codes = fp8kv::kCodesE4M3;
    else if (code_format == FP8KV_CODES_E5M2) *codes = fp8kv::kCodesE5M2;
    else return fail(FP8KV_E_UNSUPPORTED, "code_format %d: E4M3 (0) or E5M2 (1)", code_format);
    return FP8KV_OK;
}

int fp8kv_kv_quant_scatter_unscaled(
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    int32_t in_dtype, int32_t num_tokens, int32_t num_kv_heads,
    int32_t head_dim, const int64_t* slot_ids, uint8_t* k_cache,
    uint8_t* v_cache, int64_t cache_stride_slot, int64_t cache_stride_head,
    int64_t num_slots, int32_t code_format, void* stream) {
    int32_t codes = 0;
    const int st = unscaled_codes(code_format, &codes);
    if (st != FP8KV_OK) return st;
    return quant_scatter(k, k_stride_tok, k_stride_head, v, v_stride_tok, v_stride_head,
                         in_dtype, num_tokens, num_kv_heads, head_dim, slot_ids, k_cache,
                         v_cache, cache_stride_slot, cache_stride_head, nullptr, nullptr, 0, 0,
                         num_slots, codes, stream);
}

int64_t fp8kv_paged_decode_workspace_bytes(
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_ranges) {
    DecodeShape s;
    int st = decode_shape(batch, rows, num_q_heads, num_kv_heads, head_dim, num_ranges, &s);
    if (st != FP8KV_OK) return st;
    return s.ws_bytes;
}

int32_t fp8kv_paged_decode_num_ranges(int32_t num_kv_heads, int32_t num_ranges) {
    if (num_kv_heads < 1) return fail(FP8KV_E_SHAPE, "num_kv_heads must be >= 1");
    DecodeShape s;
    int st = decode_shape(0, 1, num_kv_heads, num_kv_heads, 128, num_ranges, &s);
    if (st != FP8KV_OK) return st;
    return s.num_ranges;
}

int fp8kv_paged_decode_partials(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype, const uint8_t* k_cache,
    const uint8_t* v_cache, int64_t cache_stride_slot,
    int64_t cache_stride_head, const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int32_t batch, int32_t rows,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges,
    int32_t max_context, void* workspace, size_t workspace_bytes,
    void* stream) {
    return decode_partials(q, q_stride_b, q_stride_row, q_stride_head, q_dtype, k_cache,
                           v_cache, cache_stride_slot, cache_stride_head, k_scale, v_scale,
                           scale_stride_slot, scale_stride_head, num_slots, block_tables,
                           block_table_stride, nullptr, 0, context_lens, batch, rows,
                           num_q_heads, num_kv_heads, head_dim, block_size, softmax_scale,
                           num_ranges, max_context, workspace, workspace_bytes,
                           fp8kv::kCodesE4M3Scaled, stream);
}

int fp8kv_sparse_decode_partials(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype, const uint8_t* k_cache,
    const uint8_t* v_cache, int64_t cache_stride_slot,
    int64_t cache_stride_head, const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* block_valid, int64_t block_valid_stride,
    const int32_t* context_lens, int32_t batch, int32_t rows,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges,
    int32_t max_context, void* workspace, size_t workspace_bytes,
    void* stream) {
    if (!block_valid && batch > 0)
        return fail(FP8KV_E_NULL, "sparse_decode: block_valid is NULL");
    return decode_partials(q, q_stride_b, q_stride_row, q_stride_head, q_dtype, k_cache,
                           v_cache, cache_stride_slot, cache_stride_head, k_scale, v_scale,
                           scale_stride_slot, scale_stride_head, num_slots, block_tables,
                           block_table_stride, block_valid, block_valid_stride, context_lens,
                           batch, rows, num_q_heads, num_kv_heads, head_dim, block_size,
                           softmax_scale, num_ranges, max_context, workspace,
                           workspace_bytes, fp8kv::kCodesE4M3Scaled, stream);
}

int fp8kv_paged_decode_partials_unscaled(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype, const uint8_t* k_cache,
    const uint8_t* v_cache, int64_t cache_stride_slot,
    int64_t cache_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int32_t batch, int32_t rows,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges,
    int32_t max_context, void* workspace, size_t workspace_bytes,
    int32_t code_format, void* stream) {
    int32_t codes = 0;
    const int st = unscaled_codes(code_format, &codes);
    if (st != FP8KV_OK) return st;
    return decode_partials(q, q_stride_b, q_stride_row, q_stride_head, q_dtype, k_cache,
                           v_cache, cache_stride_slot, cache_stride_head, nullptr, nullptr, 0, 0,
                           num_slots, block_tables, block_table_stride, nullptr, 0, context_lens,
                           batch, rows, num_q_heads, num_kv_heads, head_dim, block_size,
                           softmax_scale, num_ranges, max_context, workspace, workspace_bytes,
                           codes, stream);
}

int fp8kv_paged_decode_merge(
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_ranges, const void* workspace,
    size_t workspace_bytes, void* out, int64_t out_stride_b,
    int64_t out_stride_row, int64_t out_stride_head, int32_t out_dtype,
    void* stream) {
    DecodeShape s;
    int st = decode_shape(batch, rows, num_q_heads, num_kv_heads, head_dim, num_ranges, &s);
    if (st != FP8KV_OK) return st;
    if ((st = check_out_dtype(out_dtype)) != FP8KV_OK) return st;
    // no request: nothing is read or written, any pointer may be NULL
    if (batch == 0) return ok();
    if (!out) return fail(FP8KV_E_NULL, "paged_decode_merge: out is NULL");
    if (!workspace)
        return fail(FP8KV_E_WORKSPACE, "paged_decode_merge: workspace is NULL");
    if ((int64_t)workspace_bytes < s.ws_bytes)
        return fail(FP8KV_E_WORKSPACE, "workspace %zu bytes < required %lld",
                    workspace_bytes, (long long)s.ws_bytes);
    if (out_stride_b < 0 || out_stride_row < 0 || out_stride_head < 0)
        return fail(FP8KV_E_STRIDE, "paged_decode_merge: negative stride");
    const int esz = out_dtype == FP8KV_DTYPE_FP32 ? 4 : 2;
    if (!aligned(out, esz) || !aligned(workspace, 256))
        return fail(FP8KV_E_ALIGN, "out or workspace misaligned");
    if (checked()) {
        if ((st = checked_begin(stream)) != FP8KV_OK) return st;
        if ((st = check_device_ptrs({{workspace, "workspace"}, {out, "out"}})) != FP8KV_OK)
            return st;
    }
    fp8kv::MergeParams p;
    const char* ws = static_cast<const char*>(workspace);
    p.ws_o = reinterpret_cast<const float*>(ws);
    p.ws_lse = reinterpret_cast<const float*>(ws + s.lse_offset_bytes);
    p.ws_prefix = reinterpret_cast<const int32_t*>(ws + s.prefix_offset_bytes);
    p.out = out;
    p.out_stride_b = out_stride_b;
    p.out_stride_row = out_stride_row;
    p.out_stride_head = out_stride_head;
    p.out_fp32 = out_dtype == FP8KV_DTYPE_FP32;
    p.batch = batch;
    p.num_kv_heads = num_kv_heads;
    p.group = s.group;
    p.m_rows = s.m_rows;
    p.num_ranges = s.num_ranges;
    p.total_rows = batch * num_kv_heads * s.m_rows;
    return launched(fp8kv::launch_decode_merge(p, head_dim, (hipStream_t)stream),
                    "paged_decode_merge");
}

int fp8kv_paged_decode_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype, const uint8_t* k_cache,
    const uint8_t* v_cache, int64_t cache_stride_slot,
    int64_t cache_stride_head, const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int32_t batch, int32_t rows,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges,
    int32_t max_context, void* workspace, size_t workspace_bytes, void* out,
    int64_t out_stride_b, int64_t out_stride_row, int64_t out_stride_head,
    int32_t out_dtype, void* stream) {
    // validate everything before enqueueing anything
    int st = check_out_dtype(out_dtype);
    if (st != FP8KV_OK) return st;
    if (!out && batch > 0) return fail(FP8KV_E_NULL, "paged_decode: out is NULL");
    if (out_stride_b < 0 || out_stride_row < 0 || out_stride_head < 0)
        return fail(FP8KV_E_STRIDE, "paged_decode: negative out stride");
    if (!aligned(out, out_dtype == FP8KV_DTYPE_FP32 ? 4 : 2))
        return fail(FP8KV_E_ALIGN, "out misaligned");
    if (checked() && batch > 0 && (st = check_device_ptr(out, "out")) != FP8KV_OK) return st;
    st = fp8kv_paged_decode_partials(
        q, q_stride_b, q_stride_row, q_stride_head, q_dtype, k_cache, v_cache,
        cache_stride_slot, cache_stride_head, k_scale, v_scale,
        scale_stride_slot, scale_stride_head, num_slots, block_tables,
        block_table_stride, context_lens, batch, rows, num_q_heads,
        num_kv_heads, head_dim, block_size, softmax_scale, num_ranges,
        max_context, workspace, workspace_bytes, stream);
    if (st != FP8KV_OK) return st;
    return fp8kv_paged_decode_merge(
        batch, rows, num_q_heads, num_kv_heads, head_dim, num_ranges,
        workspace, workspace_bytes, out, out_stride_b, out_stride_row,
        out_stride_head, out_dtype, stream);
}

int fp8kv_paged_decode_append_partials(
    const void* q, int64_t q_stride_b, int64_t q_stride_row, int64_t q_stride_head,
    int32_t q_dtype, const void* k_new, int64_t k_new_stride_b, int64_t k_new_stride_row,
    int64_t k_new_stride_head, const void* v_new, int64_t v_new_stride_b,
    int64_t v_new_stride_row, int64_t v_new_stride_head, int32_t new_dtype, uint8_t* k_cache,
    uint8_t* v_cache, int64_t cache_stride_slot, int64_t cache_stride_head, float* k_scale,
    float* v_scale, int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride, const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes, void* stream);

int fp8kv_paged_decode_append_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_row, int64_t q_stride_head,
    int32_t q_dtype, const void* k_new, int64_t k_new_stride_b, int64_t k_new_stride_row,
    int64_t k_new_stride_head, const void* v_new, int64_t v_new_stride_b,
    int64_t v_new_stride_row, int64_t v_new_stride_head, int32_t new_dtype, uint8_t* k_cache,
    uint8_t* v_cache, int64_t cache_stride_slot, int64_t cache_stride_head, float* k_scale,
    float* v_scale, int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride, const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes, void* out, int64_t out_stride_b,
    int64_t out_stride_row, int64_t out_stride_head, int32_t out_dtype, void* stream) {
    // validate everything before enqueueing anything
    int st = check_out_dtype(out_dtype);
    if (st != FP8KV_OK) return st;
    if (new_dtype != FP8KV_DTYPE_BF16)
        return fail(FP8KV_E_UNSUPPORTED, "new_dtype %d: only BF16 K/V rows", new_dtype);
    if (!out && batch > 0) return fail(FP8KV_E_NULL, "paged_decode_append: out is NULL");
    if (out_stride_b < 0 || out_stride_row < 0 || out_stride_head < 0)
        return fail(FP8KV_E_STRIDE, "paged_decode_append: negative out stride");
    if (!aligned(out, out_dtype == FP8KV_DTYPE_FP32 ? 4 : 2))
        return fail(FP8KV_E_ALIGN, "out misaligned");
    if (checked() && batch > 0 && (st = check_device_ptr(out, "out")) != FP8KV_OK) return st;
    st = fp8kv_paged_decode_append_partials(
        q, q_stride_b, q_stride_row, q_stride_head, q_dtype, k_new, k_new_stride_b,
        k_new_stride_row, k_new_stride_head, v_new, v_new_stride_b, v_new_stride_row,
        v_new_stride_head, new_dtype, k_cache, v_cache, cache_stride_slot, cache_stride_head,
        k_scale, v_scale, scale_stride_slot, scale_stride_head, num_slots, block_tables,
        block_table_stride, context_lens, batch, rows, num_q_heads, num_kv_heads, head_dim,
        block_size, softmax_scale, num_ranges, max_context, workspace, workspace_bytes, stream);
    if (st != FP8KV_OK) return st;
    return fp8kv_paged_decode_merge(
        batch, rows, num_q_heads, num_kv_heads, head_dim, num_ranges,
        workspace, workspace_bytes, out, out_stride_b, out_stride_row,
        out_stride_head, out_dtype, stream);
}

int fp8kv_paged_decode_append_partials(
    const void* q, int64_t q_stride_b, int64_t q_stride_row, int64_t q_stride_head,
    int32_t q_dtype, const void* k_new, int64_t k_new_stride_b, int64_t k_new_stride_row,
    int64_t k_new_stride_head, const void* v_new, int64_t v_new_stride_b,
    int64_t v_new_stride_row, int64_t v_new_stride_head, int32_t new_dtype, uint8_t* k_cache,
    uint8_t* v_cache, int64_t cache_stride_slot, int64_t cache_stride_head, float* k_scale,
    float* v_scale, int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride, const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes, void* stream) {
    if (new_dtype != FP8KV_DTYPE_BF16)
        return fail(FP8KV_E_UNSUPPORTED, "new_dtype %d: only BF16 K/V rows", new_dtype);
    if (batch > 0 && (!k_new || !v_new))
        return fail(FP8KV_E_NULL, "paged_decode_append: k_new or v_new is NULL");
    AppendRows app;
    app.k = batch > 0 ? k_new : nullptr;
    app.k_sb = k_new_stride_b;
    app.k_sr = k_new_stride_row;
    app.k_sh = k_new_stride_head;
    app.v = batch > 0 ? v_new : nullptr;
    app.v_sb = v_new_stride_b;
    app.v_sr = v_new_stride_row;
    app.v_sh = v_new_stride_head;
    return decode_partials(q, q_stride_b, q_stride_row, q_stride_head, q_dtype, k_cache, v_cache,
                           cache_stride_slot, cache_stride_head, k_scale, v_scale,
                           scale_stride_slot, scale_stride_head, num_slots, block_tables,
                           block_table_stride, nullptr, 0, context_lens, batch, rows,
                           num_q_heads, num_kv_heads, head_dim, block_size, softmax_scale,
                           num_ranges, max_context, workspace, workspace_bytes,
                           fp8kv::kCodesE4M3Scaled, stream, app);
}

int fp8kv_paged_decode_attn_fp8_noalloc(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype, const uint8_t* k_cache,
    const uint8_t* v_cache, int64_t cache_stride_slot,
    int64_t cache_stride_head, const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int32_t batch, int32_t rows,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges,
    int32_t max_context, void* out, int64_t out_stride_b,
    int64_t out_stride_row, int64_t out_stride_head, int32_t out_dtype,
    void* stream) {
    // the partials must fit the library's scratch: refuse before any HIP call
    DecodeShape s;
    int st = decode_shape(batch, rows, num_q_heads, num_kv_heads, head_dim, num_ranges, &s);
    if (st != FP8KV_OK) return st;
    if (s.ws_bytes > (int64_t)FP8KV_NOALLOC_SCRATCH_BYTES)
        return fail(FP8KV_E_WORKSPACE,
                    "paged_decode_noalloc: the partials need %lld bytes, more than the "
                    "%lld-byte library scratch; use fp8kv_paged_decode_attn_fp8 with a workspace",
                    (long long)s.ws_bytes, (long long)FP8KV_NOALLOC_SCRATCH_BYTES);
    static_assert(fp8kv::kNoAllocScratchBytes == FP8KV_NOALLOC_SCRATCH_BYTES,
                  "header and library agree on the scratch size");
    void* scratch = nullptr;
    if (batch > 0) {
        const hipError_t e = fp8kv::noalloc_scratch(&scratch);
        if (e != hipSuccess)
            return fail(FP8KV_E_LAUNCH, "paged_decode_noalloc: scratch address: %s",
                        hipGetErrorString(e));
    }
    // the scratch holds only the split's partials, each written before the
    // merge reads it: nothing needs clearing between calls
    return fp8kv_paged_decode_attn_fp8(
        q, q_stride_b, q_stride_row, q_stride_head, q_dtype, k_cache, v_cache,
        cache_stride_slot, cache_stride_head, k_scale, v_scale,
        scale_stride_slot, scale_stride_head, num_slots, block_tables,
        block_table_stride, context_lens, batch, rows, num_q_heads,
        num_kv_heads, head_dim, block_size, softmax_scale, num_ranges,
        max_context, scratch, batch > 0 ? (size_t)FP8KV_NOALLOC_SCRATCH_BYTES : 0, out,
        out_stride_b, out_stride_row, out_stride_head, out_dtype, stream);
}

int fp8kv_sparse_decode_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype, const uint8_t* k_cache,
    const uint8_t* v_cache, int64_t cache_stride_slot,
    int64_t cache_stride_head, const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* block_valid, int64_t block_valid_stride,
    const int32_t* context_lens, int32_t batch, int32_t rows,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges,
    int32_t max_context, void* workspace, size_t workspace_bytes, void* out,
    int64_t out_stride_b, int64_t out_stride_row, int64_t out_stride_head,
    int32_t out_dtype, void* stream) {
    // validate everything before enqueueing anything
    int st = check_out_dtype(out_dtype);
    if (st != FP8KV_OK) return st;
    if (!out && batch > 0) return fail(FP8KV_E_NULL, "sparse_decode: out is NULL");
    if (out_stride_b < 0 || out_stride_row < 0 || out_stride_head < 0)
        return fail(FP8KV_E_STRIDE, "sparse_decode: negative out stride");
    if (!aligned(out, out_dtype == FP8KV_DTYPE_FP32 ? 4 : 2))
        return fail(FP8KV_E_ALIGN, "out misaligned");
    if (checked() && batch > 0 && (st = check_device_ptr(out, "out")) != FP8KV_OK) return st;
    st = fp8kv_sparse_decode_partials(
        q, q_stride_b, q_stride_row, q_stride_head, q_dtype, k_cache, v_cache,
        cache_stride_slot, cache_stride_head, k_scale, v_scale,
        scale_stride_slot, scale_stride_head, num_slots, block_tables,
        block_table_stride, block_valid, block_valid_stride, context_lens, batch, rows,
        num_q_heads, num_kv_heads, head_dim, block_size, softmax_scale, num_ranges,
        max_context, workspace, workspace_bytes, stream);
    if (st != FP8KV_OK) return st;
    return fp8kv_paged_decode_merge(
        batch, rows, num_q_heads, num_kv_heads, head_dim, num_ranges,
        workspace, workspace_bytes, out, out_stride_b, out_stride_row,
        out_stride_head, out_dtype, stream);
}

int fp8kv_paged_decode_attn_unscaled(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype, const uint8_t* k_cache,
    const uint8_t* v_cache, int64_t cache_stride_slot,
    int64_t cache_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int32_t batch, int32_t rows,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float softmax_scale, int32_t num_ranges,
    int32_t max_context, void* workspace, size_t workspace_bytes, void* out,
    int64_t out_stride_b, int64_t out_stride_row, int64_t out_stride_head,
    int32_t out_dtype, int32_t code_format, void* stream) {
    // validate everything before enqueueing anything
    int st = check_out_dtype(out_dtype);
    if (st != FP8KV_OK) return st;
    if (!out && batch > 0) return fail(FP8KV_E_NULL, "paged_decode: out is NULL");
    if (out_stride_b < 0 || out_stride_row < 0 || out_stride_head < 0)
        return fail(FP8KV_E_STRIDE, "paged_decode: negative out stride");
    if (!aligned(out, out_dtype == FP8KV_DTYPE_FP32 ? 4 : 2))
        return fail(FP8KV_E_ALIGN, "out misaligned");
    if (checked() && batch > 0 && (st = check_device_ptr(out, "out")) != FP8KV_OK) return st;
    st = fp8kv_paged_decode_partials_unscaled(
        q, q_stride_b, q_stride_row, q_stride_head, q_dtype, k_cache, v_cache,
        cache_stride_slot, cache_stride_head, num_slots, block_tables, block_table_stride,
        context_lens, batch, rows, num_q_heads, num_kv_heads, head_dim, block_size,
        softmax_scale, num_ranges, max_context, workspace, workspace_bytes, code_format, stream);
    if (st != FP8KV_OK) return st;
    return fp8kv_paged_decode_merge(
        batch, rows, num_q_heads, num_kv_heads, head_dim, num_ranges,
        workspace, workspace_bytes, out, out_stride_b, out_stride_row,
        out_stride_head, out_dtype, stream);
}

static int prefill(
    const void* q, int64_t q_stride_b, int64_t q_stride_tok, int64_t q_stride_head,
    int32_t q_dtype, const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head, const float* k_scale,
    const float* v_scale, int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* block_valid, int64_t block_valid_stride,
    const int32_t* context_lens, const int32_t* q_lens, int32_t batch, int32_t max_q,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float softmax_scale, int32_t max_context, void* out, int64_t out_stride_b,
    int64_t out_stride_tok, int64_t out_stride_head, int32_t out_dtype, void* stream,
    bool selected) {
    if (head_dim != 64 && head_dim != 128)
        return fail(FP8KV_E_UNSUPPORTED, "head_dim %d: only 64 and 128 are supported", head_dim);
    if (q_dtype != FP8KV_DTYPE_BF16)
        return fail(FP8KV_E_UNSUPPORTED, "q_dtype %d: only BF16 queries", q_dtype);
    int st = check_out_dtype(out_dtype);
    if (st != FP8KV_OK) return st;
    if (batch < 0 || max_q < 0 || max_context < 0 || num_q_heads < 1 || num_kv_heads < 1)
        return fail(FP8KV_E_SHAPE, "batch %d, max_q %d, max_context %d, heads %d/%d", batch,
                    max_q, max_context, num_q_heads, num_kv_heads);
    if (num_q_heads % num_kv_heads != 0)
        return fail(FP8KV_E_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    num_q_heads, num_kv_heads);
    const int32_t group = num_q_heads / num_kv_heads;
    if (group > kMaxStackedRows || kMaxStackedRows % group != 0)
        return fail(FP8KV_E_UNSUPPORTED, "GQA group %d: must divide %d", group, kMaxStackedRows);
    if (block_size < 16 || block_size % 16 != 0)
        return fail(FP8KV_E_UNSUPPORTED, "block_size %d: must be a positive multiple of 16", block_size);
    // no query row: nothing is read or written, any pointer may be NULL
    if (batch == 0 || max_q == 0) return ok();
    if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !block_tables || !context_lens ||
        !q_lens || !out || (selected && !block_valid))
        return fail(FP8KV_E_NULL, "prefill: a required pointer is NULL");
    if (q_stride_b < 0 || q_stride_tok < 0 || q_stride_head < 0 || cache_stride_slot < 0 ||
        cache_stride_head < 0 || scale_stride_slot < 0 || scale_stride_head < 0 ||
        block_table_stride < 0 || block_valid_stride < 0 || out_stride_b < 0 ||
        out_stride_tok < 0 || out_stride_head < 0)
        return fail(FP8KV_E_STRIDE, "prefill: negative stride");
    if (!aligned(q, 16) || q_stride_b % 8 || q_stride_tok % 8 || q_stride_head % 8)
        return fail(FP8KV_E_ALIGN, "q rows must start on 16-byte boundaries");
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || cache_stride_slot % 16 ||
        cache_stride_head % 16)
        return fail(FP8KV_E_ALIGN, "cache rows must start on 16-byte boundaries");
    const int oal = out_dtype == FP8KV_DTYPE_FP32 ? 16 : 8;     // vector row stores
    const int oel = out_dtype == FP8KV_DTYPE_FP32 ? 4 : 2;
    if (!aligned(out, oal) || (out_stride_b * oel) % oal || (out_stride_tok * oel) % oal ||
        (out_stride_head * oel) % oal)
        return fail(FP8KV_E_ALIGN, "out rows must start on %d-byte boundaries", oal);
    if (!aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(block_tables, 4) ||
        !aligned(block_valid, 4) || !aligned(context_lens, 4) || !aligned(q_lens, 4))
        return fail(FP8KV_E_ALIGN, "scale planes or tables misaligned");
    const int64_t num_blocks = num_slots / block_size;
    if (batch > 0 && max_context > 0 && num_blocks < 1)
        return fail(FP8KV_E_SHAPE, "num_slots %lld holds no block of %d", (long long)num_slots,
                    block_size);
    if (num_blocks > INT32_MAX)
        return fail(FP8KV_E_SHAPE, "num_slots / block_size exceeds int32 block ids");
    if (cache_stride_slot > (INT32_MAX / 16) || scale_stride_slot > (INT32_MAX / 64))
        return fail(FP8KV_E_SHAPE, "slot stride too large for 32-bit in-block offsets");
    if (checked()) {
        if ((st = checked_begin(stream)) != FP8KV_OK) return st;
        st = check_device_ptrs({{q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"},
                                {k_scale, "k_scale"}, {v_scale, "v_scale"},
                                {block_tables, "block_tables"}, {block_valid, "block_valid"},
                                {context_lens, "context_lens"}, {q_lens, "q_lens"}, {out, "out"}});
        if (st != FP8KV_OK) return st;
        std::vector<int32_t> lens, qls;
        st = check_tables(context_lens, block_tables, block_table_stride, block_valid,
                          block_valid_stride, batch, block_size, num_blocks, max_context, stream,
                          &lens);
        if (st != FP8KV_OK) return st;
        if ((st = fetch(qls, q_lens, batch, stream)) != FP8KV_OK) return st;
        for (int32_t b = 0; b < batch; ++b)
            if (qls[b] < 0 || qls[b] > max_q || qls[b] > lens[b])
                return fail(FP8KV_E_RANGE, "q_lens[%d] = %d is outside [0, min(max_q = %d, "
                            "context_lens[%d] = %d)]", b, qls[b], max_q, b, lens[b]);
    }
    fp8kv::PrefillParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.q_stride_b = q_stride_b;
    p.q_stride_tok = q_stride_tok;
    p.q_stride_head = q_stride_head;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.cache_stride_slot = cache_stride_slot;
    p.cache_stride_head = cache_stride_head;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.scale_stride_slot = scale_stride_slot;
    p.scale_stride_head = scale_stride_head;
    p.block_tables = block_tables;
    p.block_table_stride = block_table_stride;
    p.block_valid = selected ? block_valid : nullptr;
    p.block_valid_stride = block_valid_stride;
    p.context_lens = context_lens;
    p.q_lens = q_lens;
    p.out = out;
    p.out_stride_b = out_stride_b;
    p.out_stride_tok = out_stride_tok;
    p.out_stride_head = out_stride_head;
    p.out_fp32 = out_dtype == FP8KV_DTYPE_FP32;
    p.batch = batch;
    p.max_q = max_q;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = group;
    p.tokens_per_wave = kMaxStackedRows / group;
    const int block_tokens = 4 * fp8kv::kPrefillRowTiles * p.tokens_per_wave;
    p.qblocks = (max_q + block_tokens - 1) / block_tokens;
    p.block_size = block_size;
    p.block_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
    p.num_blocks = (int32_t)(num_blocks > 0 ? num_blocks : 1);
    p.max_context = max_context;
    p.score_scale_log2 = softmax_scale * 1.4426950408889634f;
    return launched(fp8kv::launch_prefill(p, head_dim, (hipStream_t)stream), "prefill_attn");
}

int fp8kv_prefill_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_tok, int64_t q_stride_head,
    int32_t q_dtype, const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head, const float* k_scale,
    const float* v_scale, int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, const int32_t* q_lens, int32_t batch, int32_t max_q,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float softmax_scale, int32_t max_context, void* out, int64_t out_stride_b,
    int64_t out_stride_tok, int64_t out_stride_head, int32_t out_dtype, void* stream) {
    return prefill(q, q_stride_b, q_stride_tok, q_stride_head, q_dtype, k_cache, v_cache,
                   cache_stride_slot, cache_stride_head, k_scale, v_scale, scale_stride_slot,
                   scale_stride_head, num_slots, block_tables, block_table_stride, nullptr, 0,
                   context_lens, q_lens, batch, max_q, num_q_heads, num_kv_heads, head_dim,
                   block_size, softmax_scale, max_context, out, out_stride_b, out_stride_tok,
                   out_stride_head, out_dtype, stream, false);
}

int fp8kv_sparse_prefill_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_tok, int64_t q_stride_head,
    int32_t q_dtype, const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head, const float* k_scale,
    const float* v_scale, int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* block_valid, int64_t block_valid_stride,
    const int32_t* context_lens, const int32_t* q_lens, int32_t batch, int32_t max_q,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float softmax_scale, int32_t max_context, void* out, int64_t out_stride_b,
    int64_t out_stride_tok, int64_t out_stride_head, int32_t out_dtype, void* stream) {
    return prefill(q, q_stride_b, q_stride_tok, q_stride_head, q_dtype, k_cache, v_cache,
                   cache_stride_slot, cache_stride_head, k_scale, v_scale, scale_stride_slot,
                   scale_stride_head, num_slots, block_tables, block_table_stride, block_valid,
                   block_valid_stride, context_lens, q_lens, batch, max_q, num_q_heads,
                   num_kv_heads, head_dim, block_size, softmax_scale, max_context, out,
                   out_stride_b, out_stride_tok, out_stride_head, out_dtype, stream, true);
}

int fp8kv_index_keys_quantize(
    const void* keys, int64_t key_stride, int64_t num_keys, int32_t head_dim,
    int32_t key_format, uint8_t* codes, int64_t code_stride,
    void* scales, int64_t scale_stride, void* stream) {
    if (head_dim != fp8kv::kIndexDim)
        return fail(FP8KV_E_UNSUPPORTED, "index keys: head_dim %d, only 128", head_dim);
    if (key_format != FP8KV_KEYS_MXFP4 && key_format != FP8KV_KEYS_E4M3)
        return fail(FP8KV_E_UNSUPPORTED, "key_format %d", key_format);
    if (num_keys < 0 || num_keys > (INT64_C(1) << 36))
        return fail(FP8KV_E_SHAPE, "num_keys %lld", (long long)num_keys);
    if (num_keys == 0) return ok();      // nothing read or written, any pointer may be NULL
    if (!keys || !codes || !scales)
        return fail(FP8KV_E_NULL, "index_keys_quantize: a required pointer is NULL");
    if (key_stride < 0 || code_stride < 0 || scale_stride < 0)
        return fail(FP8KV_E_STRIDE, "index_keys_quantize: negative stride");
    if (!aligned(keys, 16) || key_stride % 8)
        return fail(FP8KV_E_ALIGN, "key rows must start on 16-byte boundaries");
    const bool e4m3 = key_format == FP8KV_KEYS_E4M3;
    if (!aligned(codes, e4m3 ? 8 : 4) || code_stride % (e4m3 ? 8 : 4))
        return fail(FP8KV_E_ALIGN, "code rows must start on %d-byte boundaries", e4m3 ? 8 : 4);
    if (e4m3 && !aligned(scales, 4))
        return fail(FP8KV_E_ALIGN, "fp32 key scales misaligned");
    if (checked()) {
        int st = checked_begin(stream);
        if (st != FP8KV_OK) return st;
        st = check_device_ptrs({{keys, "keys"}, {codes, "codes"}, {scales, "scales"}});
        if (st != FP8KV_OK) return st;
    }
    fp8kv::IndexKeysParams p;
    p.keys = static_cast<const uint16_t*>(keys);
    p.key_stride = key_stride;
    p.codes = codes;
    p.code_stride = code_stride;
    p.scales = scales;
    p.scale_stride = scale_stride;
    p.num_keys = num_keys;
    return launched(fp8kv::launch_index_keys(p, key_format, (hipStream_t)stream),
                    "index_keys_quantize");
}

int fp8kv_index_keys_build(
    const void* raw, int64_t raw_stride_b, int64_t raw_stride_tok, int32_t batch,
    int64_t g0, int64_t g1, int32_t head_dim, int32_t key_format, uint8_t* codes,
    int64_t code_stride_b, int64_t code_stride_key, void* scales,
    int64_t scale_stride_b, int64_t scale_stride_key, void* stream) {
    if (head_dim != fp8kv::kIndexDim)
        return fail(FP8KV_E_UNSUPPORTED, "index keys: head_dim %d, only 128", head_dim);
    if (key_format != FP8KV_KEYS_MXFP4 && key_format != FP8KV_KEYS_E4M3 &&
        key_format != FP8KV_KEYS_BF16)
        return fail(FP8KV_E_UNSUPPORTED, "key_format %d", key_format);
    if (batch < 0 || batch > 65535 || g0 < 0 || g1 < g0 || g1 - g0 > (INT64_C(1) << 36))
        return fail(FP8KV_E_SHAPE, "batch %d, groups [%lld, %lld)", batch, (long long)g0,
                    (long long)g1);
    const bool bf16 = key_format == FP8KV_KEYS_BF16;
    if (batch == 0 || g1 == g0) return ok();     // nothing read or written, pointers may be NULL
    if (!raw || !codes || (!scales && !bf16))
        return fail(FP8KV_E_NULL, "index_keys_build: a required pointer is NULL");
    if (raw_stride_b < 0 || raw_stride_tok < 0 || code_stride_b < 0 || code_stride_key < 0 ||
        scale_stride_b < 0 || scale_stride_key < 0)
        return fail(FP8KV_E_STRIDE, "index_keys_build: negative stride");
    if (!aligned(raw, 16) || raw_stride_b % 8 || raw_stride_tok % 8)
        return fail(FP8KV_E_ALIGN, "raw key rows must start on 16-byte boundaries");
    const int cal = bf16 ? 16 : key_format == FP8KV_KEYS_E4M3 ? 8 : 4;
    if (!aligned(codes, cal) || code_stride_b % cal || code_stride_key % cal)
        return fail(FP8KV_E_ALIGN, "code rows must start on %d-byte boundaries", cal);
    if (key_format == FP8KV_KEYS_E4M3 && !aligned(scales, 4))
        return fail(FP8KV_E_ALIGN, "fp32 key scales misaligned");
    if (checked()) {
        int st = checked_begin(stream);
        if (st != FP8KV_OK) return st;
        st = check_device_ptrs({{raw, "raw"}, {codes, "codes"}, {scales, "scales"}});
        if (st != FP8KV_OK) return st;
    }
    fp8kv::IndexBuildParams p;
    p.raw = static_cast<const uint16_t*>(raw);
    p.raw_stride_b = raw_stride_b;
    p.raw_stride_tok = raw_stride_tok;
    p.g0 = g0;
    p.g1 = g1;
    p.codes = codes;
    p.code_stride_b = code_stride_b;
    p.code_stride_key = code_stride_key;
    p.scales = scales;
    p.scale_stride_b = scale_stride_b;
    p.scale_stride_key = scale_stride_key;
    p.batch = batch;
    return launched(fp8kv::launch_index_keys_build(p, key_format, (hipStream_t)stream),
                    "index_keys_build");
}

int fp8kv_index_score_mxfp4(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const float* w, int64_t w_stride_b, int64_t w_stride_row, int64_t w_stride_head,
    int32_t key_format, const uint8_t* codes, int64_t codes_stride_b,
    int64_t codes_stride_key, const void* scales, int64_t scales_stride_b,
    int64_t scales_stride_key, int32_t batch, int32_t rows, int32_t num_heads,
    int32_t head_dim, int32_t num_keys, int32_t key_chunk,
    float* out, int64_t out_stride_b, int64_t out_stride_row, void* stream) {
    if (head_dim != fp8kv::kIndexDim)
        return fail(FP8KV_E_UNSUPPORTED, "index scorer: head_dim %d, only 128", head_dim);
    if (q_dtype != FP8KV_DTYPE_BF16)
        return fail(FP8KV_E_UNSUPPORTED, "q_dtype %d: only BF16 queries", q_dtype);
    if (key_format != FP8KV_KEYS_MXFP4 && key_format != FP8KV_KEYS_E4M3)
        return fail(FP8KV_E_UNSUPPORTED, "key_format %d", key_format);
    if (num_heads < 1 || num_heads > fp8kv::kIndexMaxHeads)
        return fail(FP8KV_E_UNSUPPORTED, "num_heads %d: 1..%d index heads", num_heads,
                    fp8kv::kIndexMaxHeads);
    if (batch < 0 || rows < 1 || num_keys < 0)
        return fail(FP8KV_E_SHAPE, "batch %d, rows %d, num_keys %d", batch, rows, num_keys);
    if (key_chunk < 0 || key_chunk % 16)
        return fail(FP8KV_E_SHAPE, "key_chunk %d: 0 (auto) or a positive multiple of 16", key_chunk);
    if (batch == 0 || num_keys == 0) return ok();     // nothing read or written, pointers may be NULL
    if (!q || !w || !codes || !scales || !out)
        return fail(FP8KV_E_NULL, "index_score: a required pointer is NULL");
    if (q_stride_b < 0 || q_stride_row < 0 || q_stride_head < 0 || w_stride_b < 0 ||
        w_stride_row < 0 || w_stride_head < 0 || codes_stride_b < 0 || codes_stride_key < 0 ||
        scales_stride_b < 0 || scales_stride_key < 0 || out_stride_b < 0 || out_stride_row < 0)
        return fail(FP8KV_E_STRIDE, "index_score: negative stride");
    if (!aligned(q, 16) || q_stride_b % 8 || q_stride_row % 8 || q_stride_head % 8)
        return fail(FP8KV_E_ALIGN, "q rows must start on 16-byte boundaries");
    if (!aligned(codes, 16) || codes_stride_b % 16 || codes_stride_key % 16)
        return fail(FP8KV_E_ALIGN, "key code rows must start on 16-byte boundaries");
    const bool e4m3 = key_format == FP8KV_KEYS_E4M3;
    if (!aligned(w, 4) || !aligned(out, 4) || (e4m3 && !aligned(scales, 4)))
        return fail(FP8KV_E_ALIGN, "w, out or key scales misaligned");
    if (checked()) {
        int st = checked_begin(stream);
        if (st != FP8KV_OK) return st;
        st = check_device_ptrs({{q, "q"}, {w, "w"}, {codes, "codes"}, {scales, "scales"},
                                {out, "out"}});
        if (st != FP8KV_OK) return st;
    }

    const int32_t rows_per_block = fp8kv::index_rows_per_block(num_heads);
    const int32_t row_groups = (rows + rows_per_block - 1) / rows_per_block;
    int32_t chunk = key_chunk;
    if (chunk == 0) {
        // two waves per SIMD, every workgroup a (request, row group, chunk)
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return fail(FP8KV_E_LAUNCH, "no HIP device to size the index scorer for");
        const int slots = fp8kv::decode_wave_slots(dev);
        if (slots <= 0) return fail(FP8KV_E_LAUNCH, "cannot query the CU count of device %d", dev);
        const int64_t wgs_wanted = 2 * (int64_t)slots / 4;
        const int64_t per_chunk = (int64_t)batch * row_groups;
        const int64_t chunks = (wgs_wanted + per_chunk - 1) / per_chunk;
        chunk = (int32_t)round_up((num_keys + chunks - 1) / chunks, 16);
    }
    const int64_t chunks = ((int64_t)num_keys + chunk - 1) / chunk;
    if ((int64_t)batch * chunks * row_groups > INT32_MAX / 2)
        return fail(FP8KV_E_SHAPE, "index scorer grid too large");
    // each request's keys, scales and scores are addressed with 32-bit
    // byte offsets below 2^30
    const int64_t scale_key_bytes = e4m3 ? scales_stride_key * 4 : scales_stride_key;
    const int64_t key_bytes = (int64_t)(num_keys - 1) * codes_stride_key + (e4m3 ? 128 : 64);
    const int64_t scale_bytes = (int64_t)(num_keys - 1) * scale_key_bytes + 4;
    const int64_t out_bytes = ((int64_t)(rows - 1) * out_stride_row + num_keys) * 4;
    // score rows must not overlap: the kernel drops the stores of rows past
    // `rows` by the range check, which needs each row to start past the
    // previous row's last key (a single row's stride is never used); rows
    // up to 31 past the end (a wave's last rows) stay below 2^31 bytes
    const int64_t row_stride = rows > 1 ? out_stride_row : num_keys;
    if (row_stride < num_keys)
        return fail(FP8KV_E_STRIDE, "index scorer: out rows overlap (out_stride_row %lld < "
                                    "num_keys %d)", (long long)out_stride_row, num_keys);
    if (((int64_t)(rows + 31) * row_stride + num_keys) * 4 >= (INT64_C(1) << 31))
        return fail(FP8KV_E_SHAPE, "index scorer: score rows span 2^31 bytes or more");
    if (key_bytes >= (INT64_C(1) << 30) || scale_bytes >= (INT64_C(1) << 30) ||
        out_bytes >= (INT64_C(1) << 30))
        return fail(FP8KV_E_SHAPE, "index scorer: one request's keys, scales or scores "
                                   "span 2^30 bytes or more");

    fp8kv::IndexScoreParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.q_stride_b = q_stride_b;
    p.q_stride_row = q_stride_row;
    p.q_stride_head = q_stride_head;
    p.w = w;
    p.w_stride_b = w_stride_b;
    p.w_stride_row = w_stride_row;
    p.w_stride_head = w_stride_head;
    p.codes = codes;
    p.codes_stride_b = codes_stride_b;
    p.codes_stride_key = codes_stride_key;
    p.scales = static_cast<const uint8_t*>(scales);
    p.scales_stride_b = e4m3 ? scales_stride_b * 4 : scales_stride_b;
    p.scales_stride_key = e4m3 ? scales_stride_key * 4 : scales_stride_key;
    p.out = out;
    p.out_stride_b = out_stride_b;
    p.out_stride_row = row_stride;
    p.batch = batch;
    p.rows = rows;
    p.heads = num_heads;
    p.num_keys = num_keys;
    p.key_chunk = chunk;
    p.chunks = (int32_t)chunks;
    p.row_groups = row_groups;
    // rows whose pitch is a multiple of 64 KiB write their scores to the
    // same HBM channels at the same column; at 4 heads or fewer (one score
    // per 4 or more MFMA rows) those stores set the pace, so the waves of a
    // workgroup start at different columns (128 keys apart)
    p.rotate_keys = fp8kv::index_heads_padded(num_heads) <= 4 && ((int64_t)row_stride * 4) % 65536 == 0;
    p.key_bytes = (int32_t)key_bytes;
    p.scale_bytes = (int32_t)scale_bytes;
    p.out_bytes = (int32_t)out_bytes;
    return launched(fp8kv::launch_index_score(p, key_format, (hipStream_t)stream),
                    "index_score");
}

}  // extern "C"
