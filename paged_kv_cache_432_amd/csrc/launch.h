// Kernel launchers of libpa.so, called by the C ABI layer (abi.cpp) after it
// has validated the arguments.  Each returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                               int32_t max_blocks_per_req, int32_t num_seqs,
                               const int32_t* token_seq, const int32_t* token_pos,
                               int64_t num_tokens, hipStream_t stream);

// One decode row per query row of a mixed batch: row_lens [num_rows] (the
// row's keys under the causal mask or all of the request's) and row_table
// [num_rows, row_stride] (the request's block-table row).
hipError_t launch_expand_rows(const int32_t* cu_query_lens, const int32_t* seq_lens, const int32_t* block_table,
                              int32_t max_blocks_per_req, int32_t num_seqs, int64_t num_rows, int32_t causal,
                              int32_t* row_lens, int32_t* row_table, int32_t row_stride, hipStream_t stream);

// Copy-on-write: block pairs (src, dst) of every layer's K and V caches.
hipError_t launch_copy_blocks(void* key_cache, void* value_cache, int64_t layer_stride_bytes, int32_t num_layers,
                              int64_t num_blocks, int64_t block_bytes, const int64_t* block_mapping,
                              int64_t num_pairs, hipStream_t stream);

// fp8 scatter: K/V rows of `dtype` (0 fp32, 1 bf16) divided by their scale,
// stored one byte per element as E4M3 (fmt 0) or E5M2 (fmt 1) codes.
// pa_slot_mapping and the fp8 scatter in one launch.
hipError_t launch_slot_and_cache_fp8(int64_t* slot_mapping, const int32_t* block_table, int32_t max_blocks_per_req,
                                     int32_t num_seqs, const int32_t* token_seq, const int32_t* token_pos,
                                     const void* key, int64_t key_stride_bytes, const void* value,
                                     int64_t value_stride_bytes, void* key_cache, void* value_cache,
                                     int64_t num_tokens, int64_t num_slots, int32_t row_elems, int dtype,
                                     int fmt, float k_scale, float v_scale, hipStream_t stream);
hipError_t launch_reshape_and_cache_fp8(const void* key, int64_t key_stride_bytes, const void* value,
                                        int64_t value_stride_bytes, void* key_cache, void* value_cache,
                                        const int64_t* slot_mapping, int64_t num_tokens, int64_t num_slots,
                                        int32_t row_elems, int dtype, int fmt, float k_scale, float v_scale,
                                        hipStream_t stream);

// RoPE + QKV split + scatter (rope_cache_kernel); sizes in elements.
struct RopeArgs {
    void* query_out;            // [num_tokens, num_heads, 128], rows q_out_stride apart
    int64_t q_out_stride;
    const void* qkv;            // [num_tokens, (num_heads + 2 num_kv_heads) * 128], rows qkv_stride apart
    int64_t qkv_stride;
    const int64_t* positions;   // [num_tokens]
    const float* cos_sin;       // [max_position, rotary_dim]
    int64_t max_position;
    int32_t rotary_dim;
    int32_t neox_style;
    void* key_cache;
    void* value_cache;
    const int64_t* slot_mapping;
    int64_t num_slots;          // num_blocks * 16
    int64_t num_tokens;
    int32_t num_heads;
    int32_t num_kv_heads;
};
hipError_t launch_rope_cache(const RopeArgs& a, int dtype, hipStream_t stream);

// Slots and the scatter in one launch (slot_and_cache_kernel).
hipError_t launch_slot_and_cache(int64_t* slot_mapping, const int32_t* block_table, int32_t max_blocks_per_req,
                                 int32_t num_seqs, const int32_t* token_seq, const int32_t* token_pos,
                                 const void* key, int64_t key_stride_bytes, const void* value,
                                 int64_t value_stride_bytes, void* key_cache, void* value_cache, int64_t num_tokens,
                                 int64_t num_slots, int32_t row_bytes, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, int64_t key_stride, const void* value,
                                    int64_t value_stride, void* key_cache, void* value_cache,
                                    const int64_t* slot_mapping, int64_t num_tokens,
                                    int64_t num_slots, int32_t row_bytes, hipStream_t stream);

// Floats per partial record of one (piece, query head): 128 unnormalised
// outputs, the running max (base 2), the running sum, two pad floats (records
// stay 16-byte aligned).
constexpr int kDecodeRecordFloats = 132;

constexpr int kDecodePartitions = 0;   // one wave per (sequence, KV head, fixed partition)
constexpr int kDecodeStream = 1;       // equal shares of the flattened (sequence, block) space

struct DecodeArgs {
    void* out;
    const void* query;
    int64_t q_stride;              // elements between query rows
    const void* key_cache;
    const void* value_cache;
    const int32_t* block_table;
    int32_t bt_stride;             // max_blocks_per_req
    int64_t num_blocks;            // pool size: block ids are clamped into [0, num_blocks)
    const int32_t* seq_lens;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    float scale_log2;              // softmax scale (times the K scale of an fp8 cache) * log2(e): base-2 exponentials
    float out_scale;               // fp8 cache: the V scale, multiplying outputs and partial accumulators
    int32_t mode;                  // kDecodePartitions or kDecodeStream
    // partitions
    int32_t partition_tokens;      // tokens per split (multiple of 16), >= max_seq_len if unsplit
    int32_t max_partitions;        // ceil(max_seq_len / partition_tokens), >= 1
    // stream
    int32_t waves_per_group;       // KV heads (one wave each) per workgroup; divides num_kv_heads
    int32_t num_wg;                // grid size: workgroups resident at once
    int32_t min_quantum;           // fewest blocks per workgroup
    int32_t* prefix;               // [num_seqs + 1] blocks-per-KV-head prefix (written, then read)
    int32_t merge_pair;            // nonzero: the split merge takes two query heads per wave
    // partial records (split sequences only)
    float* part;
    // Append mode (bf16 stream decode, internal dtype 3): sequence b's newest
    // token, at position seq_lens[b] - 1, enters the attention from row b of
    // new_key / new_value instead of from the cache, and the same launch writes
    // that row to its cache slot (and the slot to slot_out[b], if set).
    const char* new_key;           // [num_seqs] rows of num_kv_heads * 128 bf16
    const char* new_value;
    int64_t new_key_stride;        // bytes between rows
    int64_t new_value_stride;
    int64_t* slot_out;             // [num_seqs] or null
    // fp8 append (internal dtypes 5, 6): the same rows are stored as codes of
    // x / k_scale and x / v_scale into the fp8 caches before they are read
    float k_scale;
    float v_scale;
    // Mixed batches: when set, [num_seqs + 1] offsets of each sequence's query
    // rows; only sequences with exactly one query row are attended (their row
    // and output row are cu_q[b]), the others are left to the prefill kernel.
    const int32_t* cu_q;
};

struct PrefillArgs {
    void* out;                     // [num_q_tokens, num_heads, 128]
    const void* query;
    int64_t q_stride;              // elements between query rows
    const void* key_cache;
    const void* value_cache;
    const int32_t* block_table;
    int32_t bt_stride;
    int64_t num_blocks;
    const int32_t* cu_query_lens;  // [num_seqs + 1]
    const int32_t* seq_lens;       // [num_seqs]
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    float scale_log2;
    int32_t causal;
    // Work split: the (query tile, 64-key tile) units of a KV head, U of them
    // in (sequence, tile, key tile) order, are shared by slots_per_kvh
    // workgroups (at most kPrefillMaxSlots), consecutive units each, balanced
    // on units plus a fixed set-up cost per query tile; grid = slots_per_kvh *
    // num_kv_heads, KV head fastest.
    int32_t slots_per_kvh;
    int32_t min_share;             // fewest cost units per workgroup
    float* part;                   // [grid][2][256 rows][132] partial records (a workgroup's first and
                                   // last segment)
    int32_t* split_count;          // number of listed (tile, KV head) pairs (written by workgroup 0)
    int4* split_list;              // [(slots_per_kvh - 1) * num_kv_heads]: first slot, slots | (record of
                                   // the first slot) << 24, first row, (tokens << 8) | KV head
};

// dtype: 0 = fp32, 1 = bf16, 2 = E4M3 cache (bf16 query and output), 3 = bf16
// in append mode, 4 = E5M2 cache (bf16 query and output).  group =
// num_heads / num_kv_heads in {1,2,4,8}.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int group, hipStream_t stream);

// Workgroups of the stream-mode decode kernel one compute unit holds at once.
int decode_stream_blocks_per_cu(int dtype, int group, int waves_per_group, int num_seqs);

// Attention of every sequence with two or more query rows (bf16 only).
hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t stream);
// Waves per prefill workgroup (4 or 8), each owning 32 query rows.
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
constexpr int kPrefillWaves = PA_PREFILL_WAVES;
static_assert(kPrefillWaves == 4 || kPrefillWaves == 8, "prefill waves");
// Query rows (tokens x grouped heads) per prefill workgroup tile.
constexpr int kPrefillRows = 32 * kPrefillWaves;
// Most prefill workgroups per KV head (the share boundaries live in LDS).
constexpr int kPrefillMaxSlots = 1024;
// Prefill workgroups one compute unit holds at once (bf16, group size G).
int prefill_blocks_per_cu(int group, int num_seqs);

// Memory probes (bytes a multiple of 16, pointers 16-byte aligned).
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups,
                              hipStream_t stream);
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, int32_t workgroups,
                              hipStream_t stream);
// Matrix-core rate probe: workgroups x 4 waves x iters x 4 x 32768 flops.
hipError_t launch_mfma_probe(uint32_t* sink, int32_t workgroups, int32_t iters, hipStream_t stream);

}  // namespace pa
