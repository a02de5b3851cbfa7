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

hipError_t launch_reshape_and_cache(const void* key, int64_t key_stride, const void* value,
                                    int64_t value_stride, void* key_cache, void* value_cache,
                                    const int64_t* slot_mapping, int64_t num_tokens,
                                    int64_t num_slots, int32_t row_bytes, hipStream_t stream);

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
    float scale_log2;              // softmax scale * log2(e): exponentials are taken base 2
    int32_t partition_tokens;      // tokens per split (multiple of 16), >= max_seq_len if unsplit
    int32_t max_partitions;        // ceil(max_seq_len / partition_tokens), >= 1
    float* part_acc;               // [num_seqs, num_heads, max_partitions, 128] (split only)
    float* part_ml;                // [num_seqs, num_heads, max_partitions, 2]   (split only)
};

// dtype: 0 = fp32, 1 = bf16.  group = num_heads / num_kv_heads in {1,2,4,8}.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int group, hipStream_t stream);

}  // namespace pa
