/*
 * fp8kv.h -- C ABI of the MI355X (gfx950) FP8 E4M3 paged KV cache library
 * (libfp8kv.so).
 *
 * The cache format ("feat(kvcache): store the KV cache as fp8 e4m3 codes",
 * FreeToken #354, description; "fix(qwen4-exp): register the QSA FP8 scale
 * planes for KV offload", ROCm/ATOM #2655, description, K/V bullet):
 *   - every (token, KV head) row of K, and separately of V, is head_dim
 *     OCP E4M3FN codes (max 448) kept in a plain uint8 buffer that has the
 *     geometry of the 16-bit cache -- only the element type changes;
 *   - plus ONE fp32 symmetric scale per row, scale = row amax / 448, held in
 *     a separate fp32 "scale plane" per cache (k_scale, v_scale). Anything
 *     that moves codes must move both planes with them.
 *
 * Conventions shared by every call:
 *   - Pointers marked (device) are device memory owned by the caller. The
 *     library never allocates, frees, synchronizes or reads device memory
 *     from the host; every call only enqueues kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream), so every call
 *     may be captured into a HIP graph.
 *   - Strides are in ELEMENTS of the pointed-to type. The innermost
 *     (head_dim) stride is always 1; every other stride is free, and K and V
 *     inputs carry their OWN strides (the FreeToken V-pitch fix: a K view of
 *     a fused qkv slice and a densely materialized V have different row
 *     pitches and must each be read at their own).
 *   - The compute dtype (what q, K/V inputs and outputs are) is an argument;
 *     the store dtype is always E4M3 in uint8 (FreeToken #354, description:
 *     pool.dtype vs pool.store_dtype).
 *   - Unsupported combinations are refused with a status, never ignored
 *     (FreeToken #354, description: fp8 is refused at startup where the row
 *     scales cannot be applied). Functions return FP8KV_OK (0) or a negative
 *     fp8kv_status and never abort or throw across the ABI. On failure
 *     nothing has been enqueued, except for FP8KV_E_LAUNCH.
 *   - Checks are host-side and O(1): sizes, strides, alignment, dtypes.
 *     Device-resident ids (slot ids, block tables, context lengths) are not
 *     read by the host; the kernels bound every id they use (see each call)
 *     so a bad id never reads or writes outside the buffers described by the
 *     arguments.
 *   - A call with nothing to do (no token to store, no request, no query
 *     row, no key) returns FP8KV_OK after its shape and dtype checks,
 *     enqueues nothing, and accepts NULL for every pointer (empty tensors
 *     have no storage).
 *   - fp8kv_last_error() returns a thread-local description of the most
 *     recent failure on the calling thread.
 *   - An optional checked mode (fp8kv_set_checked) adds pointer-kind and
 *     id-range checks that synchronize; it is off by default.
 */
#ifndef FP8KV_H
#define FP8KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8KV_ABI_VERSION 11

typedef enum fp8kv_status {
    FP8KV_OK = 0,
    FP8KV_E_NULL = -1,         /* a required pointer is NULL                */
    FP8KV_E_SHAPE = -2,        /* a size is out of range or inconsistent    */
    FP8KV_E_STRIDE = -3,       /* an inner stride is not 1, or a stride is  */
                               /* negative                                  */
    FP8KV_E_ALIGN = -4,        /* a pointer or stride breaks the alignment  */
                               /* the vector loads/stores need              */
    FP8KV_E_UNSUPPORTED = -5,  /* dtype / head_dim / grouping not supported */
    FP8KV_E_WORKSPACE = -6,    /* workspace NULL or smaller than required   */
    FP8KV_E_LAUNCH = -7,       /* the HIP runtime reported a launch error   */
    FP8KV_E_NOT_DEVICE = -8,   /* checked mode: a pointer is not device     */
                               /* memory of the current device              */
    FP8KV_E_RANGE = -9         /* checked mode: a device-resident id or     */
                               /* length is out of range                    */
} fp8kv_status;

typedef enum fp8kv_dtype {
    FP8KV_DTYPE_BF16 = 1,
    FP8KV_DTYPE_FP16 = 2,
    FP8KV_DTYPE_FP32 = 3
} fp8kv_dtype;

int fp8kv_abi_version(void);
const char* fp8kv_status_string(int status);
const char* fp8kv_last_error(void);

/*
 * fp8kv_set_checked -- switch the process-wide checked mode on (enabled !=
 * 0) or off; returns the previous setting (0 or 1). Off by default.
 *
 * The pages report a CPU tensor reaching the kernel as a real failure, and
 * out-of-range ids as undefined on the fast path ("feat(kvcache): store the
 * KV cache as fp8 e4m3 codes", FreeToken #354, review thread). In checked
 * mode every call, after its O(1) checks and before it enqueues anything:
 *   - refuses, with FP8KV_E_NOT_DEVICE, a pointer argument that is not
 *     device (or managed) memory of the current device
 *     (hipPointerGetAttributes);
 *   - synchronizes `stream`, copies the device-resident ids to the host and
 *     refuses, with FP8KV_E_RANGE: a slot id >= num_slots (ids < 0 stay
 *     padding); a context length outside [0, max_context]; a block-table
 *     entry of a request's tokens outside [0, num_slots / block_size); a
 *     selected block's valid count outside [0, block_size] (an entry with
 *     count 0 is never read and its id is not checked); a prefill q_lens
 *     entry outside [0, min(max_q, context length)].
 * Because it synchronizes, checked mode refuses to run under graph capture
 * (FP8KV_E_UNSUPPORTED), and it breaks the "never synchronizes or reads
 * device memory" convention above by design; the fast path (the default)
 * keeps it, bounding every id inside the kernels instead.
 */
int fp8kv_set_checked(int enabled);

/*
 * fp8kv_kv_quant_scatter -- quantize K and V rows to E4M3 + fp32 row scales
 * and scatter them to cache slots, K and V in ONE launch (ATOM #2655,
 * description, K/V bullet; FreeToken #354, description: one launch under
 * graph capture with the slot ids arriving as a device tensor).
 *
 * For every token t < num_tokens, KV head h < num_kv_heads and each of K, V:
 *   x[d]   = input[t * stride_tok + h * stride_head + d], d < head_dim
 *   s      = fp32(max_d |x[d]| / 448)                (IEEE division)
 *   c[d]   = E4M3(fp32(x[d] / s)) round-to-nearest-even, saturating;
 *            when s == 0 (all-zero row) c[d] = E4M3(x[d]) = +-0
 *   cache[slot * cache_stride_slot + h * cache_stride_head + d] = c[d]
 *   scale[slot * scale_stride_slot + h * scale_stride_head]      = s
 * with slot = slot_ids[t]. A slot id < 0 (padding) or >= num_slots writes
 * nothing for that token. Two tokens with the same slot id race (undefined
 * which row lands).
 *
 * k, v        (device) inputs of dtype in_dtype (FP8KV_DTYPE_BF16 only),
 *             element (t, h, d) at t*stride_tok + h*stride_head + d. Each
 *             row starts on a head_dim/8-byte boundary (16 bytes at 128, 8
 *             at 64): pointer and strides multiples of head_dim/16 elements.
 * slot_ids    (device) int64[num_tokens].
 * k_cache, v_cache (device) uint8 code buffers sharing the cache strides;
 *             pointers and cache strides multiples of 16 bytes.
 * k_scale, v_scale (device) fp32 scale planes sharing the scale strides.
 * head_dim    64 or 128. num_tokens may be 0 (nothing is launched).
 * Errors: E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_UNSUPPORTED, E_LAUNCH.
 */
int fp8kv_kv_quant_scatter(
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    int32_t in_dtype, int32_t num_tokens, int32_t num_kv_heads,
    int32_t head_dim,
    const int64_t* slot_ids,
    uint8_t* k_cache, uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    float* k_scale, float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots, void* stream);

/*
 * Paged GQA decode attention over the E4M3 cache (ATOM #2655, description,
 * K/V bullet: the attention kernel works on E4M3 tiles, scales each key's
 * score by that key's scale and weights each value row's probability by
 * the value's scale ahead of the PV product; sglang-jax #1776,
 * "Modifications": K/V tiles are widened to the query
 * dtype before the score dot and the probabilities are never rounded to the
 * cache dtype).
 *
 * Rows: request b < batch, verify row r < rows, query head hq < num_q_heads.
 * G = num_q_heads / num_kv_heads; query head hq reads KV head hq / G. With
 * L = min(context_lens[b], max_context), row r sees cache tokens
 * 0 .. L - rows + r (the rows are causal among themselves; rows == 1 sees
 * all L). Token j of request b lives in slot
 *     block_tables[b * block_table_stride + j / block_size] * block_size
 *     + j % block_size.
 *   score_j = (q . dec(k_code_j)) * k_scale_j * softmax_scale
 *   out     = sum_j softmax(score)_j * v_scale_j * dec(v_code_j)
 * A row that sees no token gets out = 0.
 *
 * Split. Per KV head the visible keys of all requests form one sequence
 * of 32-token tiles (request 0's ceil(L/32) tiles, then request 1's, ...;
 * U tiles in all). It is cut into num_ranges equal ranges (range r holds
 * tiles [floor(r*U/R), floor((r+1)*U/R))), each reduced by one wave per KV
 * head, so the work per wave does not depend on how the lengths are mixed.
 * Each piece (request b, range r) of a range becomes a partial (normalized
 * output, log2 log-sum-exp) in the workspace, and a merge kernel combines
 * each request's pieces by log-sum-exp. num_ranges = 0 lets the library
 * choose (4 * the current device's CU count / num_kv_heads: one wave per
 * SIMD). The
 * grid depends only on host values, so the launch is graph-capturable with
 * any context_lens; max_context is the bound the lengths are clamped to.
 *
 * q           (device) FP8KV_DTYPE_BF16, element (b, r, hq, d) at
 *             b*q_stride_b + r*q_stride_row + hq*q_stride_head + d;
 *             16-byte aligned rows.
 * k_cache, v_cache, k_scale, v_scale  (device) as written by
 *             fp8kv_kv_quant_scatter; num_slots bounds every slot used.
 *             Pointers and cache strides multiples of 16 bytes.
 * block_tables (device) int32; context_lens (device) int32[batch].
 * Bounding: block ids are clamped into [0, num_slots / block_size) and
 *             context lengths into [0, max_context] before use, so
 *             invalid ids read wrong rows, never out-of-bounds memory.
 * head_dim 64 or 128; block_size a multiple of 16; rows * G <= 16;
 * num_q_heads % num_kv_heads == 0.
 * out         (device) dtype out_dtype (BF16, round-to-nearest-even, or
 *             FP32), element (b, r, hq, d) at b*out_stride_b +
 *             r*out_stride_row + hq*out_stride_head + d.
 * workspace   (device) at least fp8kv_paged_decode_workspace_bytes(...)
 *             bytes, 256-byte aligned; no initialization needed. Calls
 *             that share a workspace must be ordered on one stream.
 * Errors: E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_UNSUPPORTED, E_WORKSPACE,
 *         E_LAUNCH.
 */
int fp8kv_paged_decode_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale,
    int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes,
    void* out, int64_t out_stride_b, int64_t out_stride_row,
    int64_t out_stride_head, int32_t out_dtype,
    void* stream);

/*
 * fp8kv_paged_decode_append_attn_fp8 -- one decode step: the store of each
 * request's new tokens and the attention over the cache that includes them,
 * in the decode's two launches ("feat(kvcache): store the KV cache as fp8
 * e4m3 codes", FreeToken #354, description: the store is one launch under
 * graph capture, its slots known on the device; ATOM #2655, description,
 * K/V bullet: the row quantizer).
 *
 * The last `rows` positions of request b (positions L - rows .. L - 1,
 * L = min(context_lens[b], max_context); those below 0 are skipped) are
 * its new tokens, already counted in context_lens. Their K and V rows,
 *   k_new[b*k_new_stride_b + r*k_new_stride_row + h*k_new_stride_head + d]
 *   (row r = position - (L - rows), d < head_dim; v_new likewise at its own
 *   strides), are quantized exactly as fp8kv_kv_quant_scatter quantizes
 *   them and stored at the slot the page walk reads for that position
 *   (block_tables[b][pos / block_size], clamped to the pool, times
 *   block_size plus pos % block_size); then the decode attention of
 *   fp8kv_paged_decode_attn_fp8 runs over the cache. The result equals
 *   fp8kv_kv_quant_scatter with those slots followed by
 *   fp8kv_paged_decode_attn_fp8 with the same num_ranges, bit for bit (codes,
 *   scales and output). The wave that reads a new token's tile writes it,
 *   and waits for its own stores before reading that tile.
 * k_new, v_new (device) new_dtype FP8KV_DTYPE_BF16; rows on head_dim/8-byte
 *             boundaries (pointers and strides multiples of head_dim/16).
 * k_cache, v_cache, k_scale, v_scale (device) written as well as read.
 * Everything else as fp8kv_paged_decode_attn_fp8 (same workspace).
 * Errors: as fp8kv_paged_decode_attn_fp8; E_NULL for k_new / v_new,
 *         E_UNSUPPORTED for new_dtype.
 */
int fp8kv_paged_decode_append_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const void* k_new, int64_t k_new_stride_b, int64_t k_new_stride_row,
    int64_t k_new_stride_head,
    const void* v_new, int64_t v_new_stride_b, int64_t v_new_stride_row,
    int64_t v_new_stride_head, int32_t new_dtype,
    uint8_t* k_cache, uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    float* k_scale, float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale,
    int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes,
    void* out, int64_t out_stride_b, int64_t out_stride_row,
    int64_t out_stride_head, int32_t out_dtype,
    void* stream);

/* Split phase of fp8kv_paged_decode_append_attn_fp8 (the new rows' store
 * and the partials); merge with fp8kv_paged_decode_merge. */
int fp8kv_paged_decode_append_partials(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const void* k_new, int64_t k_new_stride_b, int64_t k_new_stride_row,
    int64_t k_new_stride_head,
    const void* v_new, int64_t v_new_stride_b, int64_t v_new_stride_row,
    int64_t v_new_stride_head, int32_t new_dtype,
    uint8_t* k_cache, uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    float* k_scale, float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale,
    int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8kv_paged_decode_attn_fp8_noalloc -- fp8kv_paged_decode_attn_fp8 for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * rules and results (bit for bit, for the same num_ranges) without the
 * workspace: the partials go to a device array the library holds, of
 * FP8KV_NOALLOC_SCRATCH_BYTES per GPU, kept by each GPU the library runs on
 * until the process ends.
 *   - The call allocates and frees nothing; its first call on a device looks
 *     up that device's copy of the array (hipGetSymbolAddress).
 *   - A call whose partials need more (fp8kv_paged_decode_workspace_bytes of
 *     its sizes > FP8KV_NOALLOC_SCRATCH_BYTES) is refused with
 *     FP8KV_E_WORKSPACE before anything else happens. 16 MiB covers, e.g.,
 *     64 requests x 32 query heads / 8 KV heads and 4 requests x 4 verify
 *     rows x 16 / 4 heads at the default split on a 256-CU device.
 *   - Every call on one GPU shares its array, and the array keeps the last
 *     call's partials: calls that overlap on one GPU (two streams, or two
 *     host threads without ordering) race. Order them on one stream. No
 *     clearing is needed between calls: the split writes every partial the
 *     merge reads.
 * Errors: as fp8kv_paged_decode_attn_fp8; E_WORKSPACE as above.
 */
#define FP8KV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int fp8kv_paged_decode_attn_fp8_noalloc(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale,
    int32_t num_ranges, int32_t max_context,
    void* out, int64_t out_stride_b, int64_t out_stride_row,
    int64_t out_stride_head, int32_t out_dtype,
    void* stream);

/*
 * Workspace bytes fp8kv_paged_decode_attn_fp8 / _partials / _merge need for
 * these sizes (same num_ranges rule: 0 = library choice). Returns a
 * negative fp8kv_status for an unsupported combination.
 *
 * Layout, with R the resolved num_ranges, P = batch + R - 1 piece ids,
 * M = rows * G and row m = r * G + (hq % G): P*Hkv*M*head_dim floats of
 * normalized partial outputs o[(id*Hkv + h)*M + m][d], then (256-byte
 * aligned) P*Hkv*M floats of log2-domain log-sum-exp
 * lse[(id*Hkv + h)*M + m] (-inf when the piece holds no token the row
 * sees), then (256-byte aligned) batch + 1 int32: the tiles before each
 * request and, last, U. Piece (b, r) has id b + r; request b's pieces are
 * those of the non-empty ranges r holding its tiles.
 */
int64_t fp8kv_paged_decode_workspace_bytes(
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_ranges);

/* The number of ranges used for num_kv_heads (resolves num_ranges == 0 on
 * the current device), or a negative fp8kv_status. */
int32_t fp8kv_paged_decode_num_ranges(int32_t num_kv_heads, int32_t num_ranges);

/*
 * The two phases of fp8kv_paged_decode_attn_fp8, callable separately: the
 * split phase (page walk, KV streaming, scores, online softmax, PV,
 * partials to the workspace) and the log-sum-exp merge of the partials into
 * `out`. Same arguments and rules as the fused call; the merge reads only
 * the workspace (and must use the num_ranges of the partials). Running
 * _partials then _merge on one stream equals one
 * fp8kv_paged_decode_attn_fp8 call bit for bit.
 */
int fp8kv_paged_decode_partials(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale,
    int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes, void* stream);

int fp8kv_paged_decode_merge(
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_ranges,
    const void* workspace, size_t workspace_bytes,
    void* out, int64_t out_stride_b, int64_t out_stride_row,
    int64_t out_stride_head, int32_t out_dtype,
    void* stream);

/*
 * fp8kv_sparse_decode_attn_fp8 -- the decode attention over SELECTED blocks
 * only ([ATOM] "fix(qwen4-exp): register the QSA FP8 scale planes for KV
 * offload", ROCm/ATOM #2655, description, K/V bullet: the sparse GQA kernel
 * works on E4M3 tiles with the same key- and value-scale handling;
 * "feat(kvcache): store the KV cache as fp8 e4m3 codes", FreeToken #354,
 * description: block selection uses 16-bit keys, and the codes of the
 * chosen rows are all that is fetched from the cache).
 *
 * Same arguments, rules and workspace as fp8kv_paged_decode_attn_fp8,
 * except:
 * block_tables  (device) int32: row b lists the blocks request b selected,
 *               in position order (the selection is its page table).
 * block_valid   (device) int32, entry (b, i) at b*block_valid_stride + i:
 *               how many tokens of the i-th selected block, from its start,
 *               are keys (clamped to [0, block_size]); the rest are neither
 *               read nor attended. Must not be NULL.
 * context_lens  (device) int32: virtual positions of request b, where
 *               position j is offset j % block_size of selected block
 *               j / block_size; verify row r of R attends the keys at
 *               positions 0 .. context_lens[b] - R + r (causal on virtual
 *               positions). Typically (n_selected - 1) * block_size +
 *               block_valid of the last block, which holds the newest
 *               tokens. Clamped to [0, max_context].
 * A row with no key outputs 0. With every block selected and full counts
 * this is fp8kv_paged_decode_attn_fp8.
 * Errors: as fp8kv_paged_decode_attn_fp8; E_NULL for block_valid.
 */
int fp8kv_sparse_decode_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* block_valid, int64_t block_valid_stride,
    const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale,
    int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes,
    void* out, int64_t out_stride_b, int64_t out_stride_row,
    int64_t out_stride_head, int32_t out_dtype,
    void* stream);

/* Split phase of fp8kv_sparse_decode_attn_fp8; merge with
 * fp8kv_paged_decode_merge. */
int fp8kv_sparse_decode_partials(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head,
    int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* block_valid, int64_t block_valid_stride,
    const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale,
    int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Unscaled FP8 caches ("feat(dsa): implement fp8 KV cache (e4m3) with a
 * bf16 indexer cache", sglang-jax #1776, description and "Three design
 * points": new K/V are cast to the cache dtype with no scale, since fp8
 * precision is relative and the cached values are O(1); e4m3 is preferred
 * over e5m2 for its extra mantissa bit, at about half the error).
 *
 * The cache holds the values themselves as codes, with the same geometry as
 * the scaled cache and no scale planes:
 *   c[d] = E4M3 or E5M2 of x[d], round to nearest even; magnitudes above the
 *          format's largest finite value (448 / 57344) saturate to it
 * and attention reads them with scale 1. The calls mirror
 * fp8kv_kv_quant_scatter and fp8kv_paged_decode_attn_fp8 /
 * fp8kv_paged_decode_partials (same arguments, conventions, constraints and
 * errors) without the scale planes; the split phase merges with
 * fp8kv_paged_decode_merge.
 * code_format  FP8KV_CODES_E4M3 or FP8KV_CODES_E5M2 (else E_UNSUPPORTED).
 */
typedef enum fp8kv_code_format {
    FP8KV_CODES_E4M3 = 0,   /* OCP E4M3FN, max 448                        */
    FP8KV_CODES_E5M2 = 1    /* OCP E5M2, max 57344                        */
} fp8kv_code_format;

int fp8kv_kv_quant_scatter_unscaled(
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    int32_t in_dtype, int32_t num_tokens, int32_t num_kv_heads,
    int32_t head_dim,
    const int64_t* slot_ids,
    uint8_t* k_cache, uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    int64_t num_slots, int32_t code_format, void* stream);

int fp8kv_paged_decode_attn_unscaled(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale,
    int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes,
    void* out, int64_t out_stride_b, int64_t out_stride_row,
    int64_t out_stride_head, int32_t out_dtype,
    int32_t code_format, void* stream);

int fp8kv_paged_decode_partials_unscaled(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens,
    int32_t batch, int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale,
    int32_t num_ranges, int32_t max_context,
    void* workspace, size_t workspace_bytes,
    int32_t code_format, void* stream);

/*
 * fp8kv_prefill_attn_fp8 -- chunked-prefill attention over the FP8 cache
 * ("feat(dsa): implement fp8 KV cache (e4m3) with a bf16 indexer cache",
 * sglang-jax #1776, "Modifications", qblock prefill bullet: the KV tile is
 * upcast to the query dtype once before the score dot and P never goes to
 * the cache dtype; ATOM #2655 description, K/V bullet: key scale applied to
 * each score, value scale to each probability weight).
 *
 * Request b has context_lens[b] cached tokens, the last q_lens[b] of which
 * are its chunk (already written with fp8kv_kv_quant_scatter); its query
 * token i < q_lens[b] (position P + i, P = context_lens[b] - q_lens[b])
 * attends to the cached tokens 0 .. P + i:
 *   out[b, i, hq, :] = softmax_j(softmax_scale * q . dec(kc_j) * ks_j)
 *                      weighted sum of dec(vc_j) * vs_j
 * with the cache, strides and GQA mapping of fp8kv_paged_decode_attn_fp8.
 * q         (device) bf16 [B, max_q, Hq, D] at (b, i, hq) strides; 16-byte rows.
 * q_lens    (device) int32 [B], clamped to [0, min(max_q, context_lens[b])].
 * out       (device) bf16 or fp32, element (b, i, hq, d) at b*out_stride_b +
 *           i*out_stride_tok + hq*out_stride_head + d; rows aligned to 8
 *           (bf16) or 16 (fp32) bytes. Rows i >= q_lens[b] are not written.
 * Constraints: head_dim 64 or 128; num_q_heads / num_kv_heads divides 16;
 * block_size a multiple of 16. No workspace.
 * Launch shape: one workgroup per block of query rows up to max_q, so a
 * max_q near the longest chunk avoids workgroups with no rows; when there
 * are at most as many blocks as compute units (head_dim 128) each block's
 * keys are split over two groups of waves and merged (same result within
 * the floating-point bar; the split rounds differently).
 * Errors: E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_UNSUPPORTED, E_LAUNCH.
 */
int fp8kv_prefill_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_tok, int64_t q_stride_head,
    int32_t q_dtype, const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, const int32_t* q_lens,
    int32_t batch, int32_t max_q, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale, int32_t max_context,
    void* out, int64_t out_stride_b, int64_t out_stride_tok, int64_t out_stride_head,
    int32_t out_dtype, void* stream);

/*
 * fp8kv_sparse_prefill_attn_fp8 -- chunked-prefill attention over SELECTED
 * blocks only ([ATOM] "fix(qwen4-exp): register the QSA FP8 scale planes for
 * KV offload", ROCm/ATOM #2655, description, MI355X results: the sparse GQA
 * prefill over the E4M3 cache; "feat(kvcache): store the KV cache as fp8
 * e4m3 codes", FreeToken #354, description: the codes of the chosen rows
 * are all that is fetched from the cache).
 *
 * fp8kv_prefill_attn_fp8 over the selection of fp8kv_sparse_decode_attn_fp8:
 * block_tables  (device) int32: row b lists the blocks request b selected,
 *               in position order; the chunk's own tokens are among them.
 * block_valid   (device) int32, entry (b, i) at b*block_valid_stride + i:
 *               how many tokens of the i-th selected block, from its start,
 *               are keys (clamped to [0, block_size]). Must not be NULL.
 * context_lens  (device) int32: virtual positions of request b (position j
 *               is offset j % block_size of selected block j / block_size);
 *               its last q_lens[b] positions are the chunk, and chunk token i
 *               attends the keys at positions 0 .. context_lens[b] -
 *               q_lens[b] + i. A token that sees no key gets out = 0.
 * With every block selected and full counts this is fp8kv_prefill_attn_fp8.
 * Errors: as fp8kv_prefill_attn_fp8; E_NULL for block_valid.
 */
int fp8kv_sparse_prefill_attn_fp8(
    const void* q, int64_t q_stride_b, int64_t q_stride_tok, int64_t q_stride_head,
    int32_t q_dtype, const uint8_t* k_cache, const uint8_t* v_cache,
    int64_t cache_stride_slot, int64_t cache_stride_head,
    const float* k_scale, const float* v_scale,
    int64_t scale_stride_slot, int64_t scale_stride_head, int64_t num_slots,
    const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* block_valid, int64_t block_valid_stride,
    const int32_t* context_lens, const int32_t* q_lens,
    int32_t batch, int32_t max_q, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale, int32_t max_context,
    void* out, int64_t out_stride_b, int64_t out_stride_tok, int64_t out_stride_head,
    int32_t out_dtype, void* stream);

/*
 * Compressed index keys and the index scorer ("fix(qwen4-exp): register
 * the QSA FP8 scale planes for KV offload", ROCm/ATOM #2655, description:
 * the compressed-index bullet and the stacked decode scorer paragraph).
 * Keys have head_dim 128 and are stored in one of two formats.
 */
typedef enum fp8kv_key_format {
    FP8KV_KEYS_MXFP4 = 0,   /* packed E2M1 pairs + one E8M0 exponent per 32 dims */
    FP8KV_KEYS_E4M3 = 1,    /* E4M3 codes + one fp32 scale per key              */
    FP8KV_KEYS_BF16 = 2     /* unquantized bf16 keys (fp8kv_index_keys_build)   */
} fp8kv_key_format;

/*
 * fp8kv_index_keys_quantize -- encode num_keys bf16 keys.
 *
 * keys        (device) bf16, element (n, d) at n * key_stride + d, d < 128;
 *             pointer 16-byte aligned, key_stride a multiple of 8.
 * FP8KV_KEYS_E4M3: the KV row quantizer (codes and scale exactly those of
 *   fp8kv_kv_quant_scatter): codes (device) uint8, code (n, d) at
 *   n * code_stride + d; scales (device) fp32, scale n at n * scale_stride.
 *   Code rows start on 8-byte boundaries.
 * FP8KV_KEYS_MXFP4: for each group g < 4 of 32 dims, e is the smallest
 *   integer with max |x| <= 6 * 2^e (exact comparison, clamped to
 *   [-127, 127]; an all-zero group has e = 0), scales (device) uint8 at
 *   n * scale_stride + g holds the E8M0 code e + 127, and every element is
 *   the E2M1 value nearest to x / 2^e (ties to the even code, sign of x
 *   kept). codes (device) uint8 at n * code_stride + j, j < 64: element 2j
 *   in the low nibble, 2j + 1 in the high nibble. Code rows start on 4-byte
 *   boundaries.
 * num_keys may be 0 (nothing is launched).
 * Errors: E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_UNSUPPORTED, E_LAUNCH.
 */
int fp8kv_index_keys_quantize(
    const void* keys, int64_t key_stride, int64_t num_keys, int32_t head_dim,
    int32_t key_format, uint8_t* codes, int64_t code_stride,
    void* scales, int64_t scale_stride, void* stream);

/*
 * fp8kv_index_keys_build -- build compressed index keys from raw bf16 index
 * keys ([ATOM] description, compressed-index bullet: the raw index keys are
 * kept in BF16, averaged in groups before the normalization, and a group
 * may span two prefill chunks). For every request b < batch and compressed key
 * g in [g0, g1):
 *   m[d] = (r[4g][d] + r[4g+1][d] + r[4g+2][d] + r[4g+3][d]) / 4      (fp32)
 *   k[d] = bf16_rne(m[d] / ||m||_2)            (0 when m = 0)
 * then k is stored in key_format exactly as fp8kv_index_keys_quantize would
 * store the bf16 key k (FP8KV_KEYS_BF16: the 128 bf16 values themselves).
 * Groups follow positions, not chunks: after a chunk ends at raw position
 * L, call with g1 = L / 4, and build the straddling group in the next call
 * once its fourth raw key exists.
 * raw     (device) bf16, raw key t of request b at b*raw_stride_b +
 *         t*raw_stride_tok (elements); 16-byte aligned rows.
 * codes   (device) key g of request b at b*code_stride_b + g*code_stride_key
 *         (bytes): 64 (MXFP4), 128 (E4M3) or 256 (BF16) bytes; rows aligned
 *         to 4 / 8 / 16 bytes.
 * scales  (device) E4M3: fp32 at b*scale_stride_b + g*scale_stride_key;
 *         MXFP4: 4 E8M0 bytes from there; unused (may be NULL) for BF16.
 * The fp32 mean and norm are accurate to a few fp32 ulps, so k is the
 * correctly rounded bf16 of the exact normalized mean except within about
 * 2^-16 (relative) of a rounding midpoint.
 * Errors: E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_UNSUPPORTED, E_LAUNCH.
 */
int fp8kv_index_keys_build(
    const void* raw, int64_t raw_stride_b, int64_t raw_stride_tok, int32_t batch,
    int64_t g0, int64_t g1, int32_t head_dim, int32_t key_format,
    uint8_t* codes, int64_t code_stride_b, int64_t code_stride_key,
    void* scales, int64_t scale_stride_b, int64_t scale_stride_key, void* stream);

/*
 * fp8kv_index_score_mxfp4 -- the decode-sized index scorer, over MXFP4 or
 * E4M3 keys:
 *   out[b, r, n] = sum_{h < num_heads} w[b, r, h] * max(0, q[b, r, h, :] . k^[b, n, :])
 * for b < batch, r < rows, n < num_keys, with k^ the dequantized key
 * (MXFP4: E2M1 value * 2^e of its group; E4M3: code value * key scale),
 * accumulated in fp32 (the products of bf16 q and the exactly widened key
 * elements are exact; the sums are fp32 MFMA and lane sums). Rows and
 * index heads share the 16 MFMA rows (the page's stacked decode scorer):
 * with H heads padded up to a power of two HP, 16 / HP rows x HP heads fill
 * one tile (HP = 4: 4 rows x 4 heads), so few heads cost no idle MFMA rows.
 *
 * q           (device) FP8KV_DTYPE_BF16, element (b, r, h, d) at
 *             b*q_stride_b + r*q_stride_row + h*q_stride_head + d; pointer
 *             16-byte aligned, strides multiples of 8.
 * w           (device) fp32, (b, r, h) at b*w_stride_b + r*w_stride_row +
 *             h*w_stride_head (any stride may be 0: broadcast).
 * codes       (device) key n of request b at b*codes_stride_b +
 *             n*codes_stride_key (bytes), laid out as written by
 *             fp8kv_index_keys_quantize; pointer and strides multiples of 16.
 * scales      (device) MXFP4: uint8 exponent (b, n, g) at b*scales_stride_b
 *             + n*scales_stride_key + g; E4M3: fp32 scale (b, n) at
 *             b*scales_stride_b + n*scales_stride_key (elements).
 * num_heads   1..16; head_dim 128; rows >= 1; batch, num_keys >= 0.
 * key_chunk   keys per workgroup: 0 = chosen for the current device, else
 *             a positive multiple of 16.
 * out         (device) fp32, (b, r, n) at b*out_stride_b + r*out_stride_row + n.
 *             Rows must not overlap: out_stride_row >= num_keys when rows > 1
 *             (else E_STRIDE), and ((rows + 31) * out_stride_row + num_keys)
 *             * 4 < 2^31 (else E_SHAPE).
 * Errors: E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_UNSUPPORTED, E_LAUNCH.
 */
int fp8kv_index_score_mxfp4(
    const void* q, int64_t q_stride_b, int64_t q_stride_row,
    int64_t q_stride_head, int32_t q_dtype,
    const float* w, int64_t w_stride_b, int64_t w_stride_row, int64_t w_stride_head,
    int32_t key_format, const uint8_t* codes, int64_t codes_stride_b,
    int64_t codes_stride_key, const void* scales, int64_t scales_stride_b,
    int64_t scales_stride_key, int32_t batch, int32_t rows, int32_t num_heads,
    int32_t head_dim, int32_t num_keys, int32_t key_chunk,
    float* out, int64_t out_stride_b, int64_t out_stride_row, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8KV_H */
