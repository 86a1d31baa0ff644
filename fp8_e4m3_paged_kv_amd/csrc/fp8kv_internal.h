// fp8kv_internal.h -- kernel parameter blocks and launchers shared by the
// C-ABI layer (fp8kv_api.cpp) and the kernel translation units. Not part of
// the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8kv {

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
    const int32_t* context_lens;
    int32_t batch, rows, num_q_heads, num_kv_heads, group, m_rows;
    int32_t block_size, max_context;
    int32_t block_shift;       // log2(block_size) when a power of two, else -1
    int32_t num_blocks;        // physical blocks: ids are clamped below it
    int32_t num_ranges;        // R: equal ranges of each KV head's tile sequence
    int32_t wgs_per_range;     // Hkv / 4 when that is a whole number > 1, else 1
    float score_scale_log2;    // softmax_scale * log2(e)
    float* ws_o;               // [(batch + R - 1) * Hkv * M, head_dim]
    float* ws_lse;             // [(batch + R - 1) * Hkv * M]
    int32_t* ws_prefix;        // [batch + 1]: tiles before each request, then U
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

// Wave slots the decode split fills by default: one per SIMD (4 per CU),
// 0 if the device query fails.
int decode_wave_slots(int device);

hipError_t launch_decode_partitions(const DecodeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_merge(const MergeParams& p, int head_dim,
                               hipStream_t stream);

}  // namespace fp8kv
