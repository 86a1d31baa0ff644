// fp8kv_internal.h -- kernel parameter blocks and launchers shared by the
// C-ABI layer (fp8kv_api.cpp) and the kernel translation units. Not part of
// the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8kv {

// Cache code formats: E4M3 codes with one fp32 scale per (token, KV head)
// row (the default), or codes without scales (the value itself, scale 1)
// in E4M3 or E5M2.
constexpr int kCodesE4M3Scaled = 0;
constexpr int kCodesE4M3 = 1;
constexpr int kCodesE5M2 = 2;

struct QuantScatterParams {
    const uint16_t* k;         // bf16 bits
    const uint16_t* v;
    int64_t k_stride_tok, k_stride_head;
    int64_t v_stride_tok, v_stride_head;
    const int64_t* slot_ids;
    uint8_t* k_cache;
    uint8_t* v_cache;
    int64_t cache_stride_slot, cache_stride_head;
    float* k_scale;
    float* v_scale;
    int64_t scale_stride_slot, scale_stride_head;
    int64_t num_slots;
    int32_t num_tokens, num_kv_heads;
    int64_t num_rows;          // num_tokens * num_kv_heads * 2
    int32_t codes;             // kCodes*: unscaled formats write no scales
};

hipError_t launch_kv_quant_scatter(const QuantScatterParams& p, int head_dim,
                                   hipStream_t stream);

struct DecodeParams {
    const uint16_t* q;         // bf16 bits
    int64_t q_stride_b, q_stride_row, q_stride_head;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    int64_t cache_stride_slot, cache_stride_head;
    const float* k_scale;
    const float* v_scale;
    int64_t scale_stride_slot, scale_stride_head;
    const int32_t* block_tables;
    int64_t block_table_stride;
    const int32_t* block_valid;   // selected blocks: valid keys per entry, or null (dense)
    int64_t block_valid_stride;
    const int32_t* context_lens;
    int32_t batch, rows, num_q_heads, num_kv_heads, group, m_rows;
    int32_t block_size, max_context;
    int32_t block_shift;       // log2(block_size) when a power of two, else -1
    int32_t num_blocks;        // physical blocks: ids are clamped below it
    int32_t num_ranges;        // R: equal ranges of each KV head's tile sequence
    int32_t wgs_per_range;     // Hkv / 4 when that is a whole number > 1, else 1
    float score_scale_log2;    // softmax_scale * log2(e)
    int32_t codes;             // kCodes*: unscaled formats read no scales
    float* ws_o;               // [(batch + R - 1) * Hkv * M, head_dim]
    float* ws_lse;             // [(batch + R - 1) * Hkv * M]
    int32_t* ws_prefix;        // [batch + 1]: tiles before each request, then U
    // append (fp8kv_paged_decode_append_attn_fp8): the new K and V rows of
    // each request's last `rows` positions (bf16 [B, rows, Hkv, D] at these
    // element strides), quantized into the cache before they are read; null
    // for the other calls
    const uint16_t* k_new;
    const uint16_t* v_new;
    int64_t kn_stride_b, kn_stride_row, kn_stride_head;
    int64_t vn_stride_b, vn_stride_row, vn_stride_head;
};

struct MergeParams {
    const float* ws_o;
    const float* ws_lse;
    const int32_t* ws_prefix;
    void* out;
    int64_t out_stride_b, out_stride_row, out_stride_head;
    int32_t out_fp32;          // 1: fp32 output, 0: bf16
    int32_t batch, num_kv_heads, group, m_rows, num_ranges;
    int32_t total_rows;        // batch * num_kv_heads * m_rows
};

struct PrefillParams {
    const uint16_t* q;         // bf16 bits [B, max_q, Hq, D]
    int64_t q_stride_b, q_stride_tok, q_stride_head;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    int64_t cache_stride_slot, cache_stride_head;
    const float* k_scale;
    const float* v_scale;
    int64_t scale_stride_slot, scale_stride_head;
    const int32_t* block_tables;
    int64_t block_table_stride;
    const int32_t* block_valid;    // selected blocks: valid keys per entry, or null (dense)
    int64_t block_valid_stride;
    const int32_t* context_lens;   // cached tokens of request b, the chunk included
    const int32_t* q_lens;         // query tokens of request b: its last q_lens[b] tokens
    void* out;                     // [B, max_q, Hq, D]
    int64_t out_stride_b, out_stride_tok, out_stride_head;
    int32_t out_fp32;
    int32_t batch, max_q, num_q_heads, num_kv_heads, group;
    int32_t tokens_per_wave;       // per 16-row tile: 16 / group
    int32_t qblocks;               // ceil(max_q / (4 * kPrefillRowTiles * tokens_per_wave))
    int32_t block_size, block_shift, num_blocks, max_context;
    float score_scale_log2;
};

// 16-row MFMA tiles of query rows per prefill wave.
constexpr int kPrefillRowTiles = 2;

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream);

// Wave slots the decode split fills by default: one per SIMD (4 per CU),
// 0 if the device query fails.
int decode_wave_slots(int device);

hipError_t launch_decode_partitions(const DecodeParams& p, int head_dim, hipStream_t stream);

// Library-held device scratch of the decode entry point that allocates
// nothing: its size, and its address on the current device (looked up once
// per device with hipGetSymbolAddress, then cached).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_decode_merge(const MergeParams& p, int head_dim,
                               hipStream_t stream);

// Compressed index keys (head_dim 128).
constexpr int kKeysMXFP4 = 0;
constexpr int kKeysE4M3 = 1;
constexpr int kKeysBF16 = 2;           // the builder's unquantized output
constexpr int kIndexDim = 128;
constexpr int kIndexMaxHeads = 16;     // MFMA M dimension
// The scorer stacks rows x heads into the 16 MFMA rows: the heads are
// padded up to a power of two HP, and 16 / HP rows share one MFMA tile.
constexpr int index_heads_padded(int heads) {
    return heads <= 1 ? 1 : heads <= 2 ? 2 : heads <= 4 ? 4 : heads <= 8 ? 8 : 16;
}
// Query rows per scorer workgroup (4 waves; a wave carries 8 MFMA tiles, or
// 32 rows when the tiles stack more than 4 rows each).
constexpr int index_rows_per_block(int heads) {
    const int rpt = 16 / index_heads_padded(heads);
    const int tiles = rpt <= 4 ? 8 : 32 / rpt;
    return 4 * tiles * rpt;
}

struct IndexKeysParams {
    const uint16_t* keys;      // bf16 bits [num_keys, 128], row stride key_stride elements
    int64_t key_stride;
    uint8_t* codes;            // E4M3 [., 128] / packed E2M1 [., 64]; row stride in bytes
    int64_t code_stride;
    void* scales;              // E4M3: fp32 [.], MXFP4: E8M0 bytes [., 4]; row stride in elements
    int64_t scale_stride;
    int64_t num_keys;
};

struct IndexScoreParams {
    const uint16_t* q;         // bf16 bits [B, rows, heads, 128]
    int64_t q_stride_b, q_stride_row, q_stride_head;
    const float* w;            // [B, rows, heads]
    int64_t w_stride_b, w_stride_row, w_stride_head;
    const uint8_t* codes;      // per request, keys at codes_stride_key bytes
    int64_t codes_stride_b, codes_stride_key;
    const uint8_t* scales;     // per request; strides in bytes
    int64_t scales_stride_b, scales_stride_key;
    float* out;                // [B, rows, num_keys], key stride 1
    int64_t out_stride_b, out_stride_row;
    int32_t batch, rows, heads, num_keys;
    int32_t key_chunk;         // keys per workgroup, a multiple of 16
    int32_t chunks;            // ceil(num_keys / key_chunk)
    int32_t row_groups;        // ceil(rows / index_rows_per_block(heads))
    int32_t key_bytes;         // per request: extent of the key codes in bytes
    int32_t scale_bytes;       // per request: extent of the key scales in bytes
    int32_t out_bytes;         // per request: (rows - 1) * out_stride_row * 4 + num_keys * 4
    int32_t rotate_keys;       // 1: each wave of a workgroup starts at its own quarter of the chunk
};

struct IndexBuildParams {
    const uint16_t* raw;       // bf16 bits [B, L, 128]: raw index keys by position
    int64_t raw_stride_b, raw_stride_tok;
    int64_t g0, g1;            // compressed keys g0 .. g1-1 (raw keys 4*g0 .. 4*g1-1)
    uint8_t* codes;            // [B, N, bytes]: strides in bytes
    int64_t code_stride_b, code_stride_key;
    void* scales;              // [B, N(, 4)]: strides in elements
    int64_t scale_stride_b, scale_stride_key;
    int32_t batch;
};

hipError_t launch_index_keys(const IndexKeysParams& p, int key_format, hipStream_t stream);
hipError_t launch_index_keys_build(const IndexBuildParams& p, int key_format, hipStream_t stream);
hipError_t launch_index_score(const IndexScoreParams& p, int key_format, hipStream_t stream);

}  // namespace fp8kv
