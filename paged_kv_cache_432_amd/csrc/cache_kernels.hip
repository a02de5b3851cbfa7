// Slot computation and the KV scatter ("reshape_and_cache") for gfx950.
//
// Both follow section "Paged Attention" of "AI Infra入门干货总结：大模型是如何高效
// 推理的": a token's slot is its request's page-table entry for logical block
// pos / block_size, times block_size, plus pos % block_size; the scatter copies
// the token's [num_kv_heads, head_dim] K and V rows to cache[slot / block_size,
// slot % block_size].  Both are pure index / copy work: no rounding is involved
// and results are bit-exact.
#include "device_common.h"
#include "launch.h"

namespace pa {

__global__ void __launch_bounds__(256)
slot_mapping_kernel(int64_t* __restrict__ out, const int32_t* __restrict__ block_table,
                    int32_t bt_stride, int32_t num_seqs, const int32_t* __restrict__ token_seq,
                    const int32_t* __restrict__ token_pos, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int32_t s = token_seq[i];
    const int32_t p = token_pos[i];
    int64_t slot = -1;
    if (s >= 0 && s < num_seqs && p >= 0 && p / kBlock < bt_stride) {
        const int32_t physical = block_table[(int64_t)s * bt_stride + p / kBlock];
        if (physical >= 0) slot = (int64_t)physical * kBlock + p % kBlock;
    }
    out[i] = slot;
}

// One workgroup per token: the first half of the threads copy the K row, the
// second half the V row, 16 bytes per thread per step (2 KiB rows in bf16 for
// 8 KV heads x 128 dims, so one step each).
__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(const char* __restrict__ key, int64_t key_stride_bytes,
                         const char* __restrict__ value, int64_t value_stride_bytes,
                         char* __restrict__ key_cache, char* __restrict__ value_cache,
                         const int64_t* __restrict__ slot_mapping, int64_t num_slots,
                         int32_t row_bytes) {
    const int64_t token = blockIdx.x;
    const int64_t slot = slot_mapping[token];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t block = slot / kBlock;
    const int64_t offset = slot % kBlock;
    const int64_t dst = (block * kBlock + offset) * (int64_t)row_bytes;
    const int32_t chunks = row_bytes >> 4;
    const bool is_v = threadIdx.x >= 128;
    const char* src = is_v ? value + token * value_stride_bytes : key + token * key_stride_bytes;
    char* dcache = (is_v ? value_cache : key_cache) + dst;
    for (int32_t c = threadIdx.x & 127; c < chunks; c += 128) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + ((int64_t)c << 4));
        *reinterpret_cast<u32x4_t*>(dcache + ((int64_t)c << 4)) = v;
    }
}

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                               int32_t max_blocks_per_req, int32_t num_seqs,
                               const int32_t* token_seq, const int32_t* token_pos,
                               int64_t num_tokens, hipStream_t stream) {
    const int64_t grid = (num_tokens + 255) / 256;
    hipLaunchKernelGGL(slot_mapping_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       slot_mapping, block_table, max_blocks_per_req, num_seqs, token_seq,
                       token_pos, num_tokens);
    return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, int64_t key_stride, const void* value,
                                    int64_t value_stride, void* key_cache, void* value_cache,
                                    const int64_t* slot_mapping, int64_t num_tokens,
                                    int64_t num_slots, int32_t row_bytes, hipStream_t stream) {
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)num_tokens), dim3(256), 0, stream,
                       (const char*)key, key_stride, (const char*)value, value_stride,
                       (char*)key_cache, (char*)value_cache, slot_mapping, num_slots, row_bytes);
    return hipGetLastError();
}

}  // namespace pa
