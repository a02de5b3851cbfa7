// Slot computation and the KV scatter ("reshape_and_cache") for gfx950.
//
// Both follow section "Paged Attention" of "AI Infra入门干货总结：大模型是如何高效
// 推理的": a token's slot is its request's page-table entry for logical block
// pos / block_size, times block_size, plus pos % block_size; the scatter copies
// the token's [num_kv_heads, head_dim] K and V rows to cache[slot / block_size,
// slot % block_size].  Both are pure index / copy work: no rounding is involved
// and results are bit-exact.
#include <type_traits>

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

// ---- copy-on-write of shared blocks ------------------------------------------
// Block dst of every layer's K and V cache becomes a copy of block src, for
// each (src, dst) pair ("AI Infra入门干货总结：大模型是如何高效推理的", section
// "Paged Attention": the [num_layers, 2, num_blocks, ...] cache; copy-on-write
// of blocks shared by a prefix).  Workgroup (pair, 2 * layer + K/V) moves one
// block, 16 bytes per thread per step.  Pairs run concurrently: no dst may be
// the src or dst of another pair in the same call.
__global__ void __launch_bounds__(256)
copy_blocks_kernel(char* __restrict__ key_cache, char* __restrict__ value_cache, int64_t layer_stride_bytes,
                   int64_t num_blocks, int64_t block_bytes, const int64_t* __restrict__ block_mapping) {
    const int64_t pair = blockIdx.x;
    const int64_t src = block_mapping[2 * pair], dst = block_mapping[2 * pair + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
    const int layer = blockIdx.y >> 1;
    char* base = ((blockIdx.y & 1) ? value_cache : key_cache) + layer * layer_stride_bytes;
    const u32x4_t* from = reinterpret_cast<const u32x4_t*>(base + src * block_bytes);
    u32x4_t* to = reinterpret_cast<u32x4_t*>(base + dst * block_bytes);
    for (int64_t c = threadIdx.x; c < block_bytes / 16; c += blockDim.x) to[c] = from[c];
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, int64_t layer_stride_bytes, int32_t num_layers,
                              int64_t num_blocks, int64_t block_bytes, const int64_t* block_mapping,
                              int64_t num_pairs, hipStream_t stream) {
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, (unsigned)(2 * num_layers)), dim3(256), 0,
                       stream, (char*)key_cache, (char*)value_cache, layer_stride_bytes, num_blocks, block_bytes,
                       block_mapping);
    return hipGetLastError();
}

// ---- fp8 (E4M3 or E5M2) scatter -------------------------------------------
// As reshape_and_cache_kernel, but each element x of a K (V) row is stored as
// the E4M3 (E5 = false) or E5M2 (E5 = true) code of x / k_scale (v_scale), by
// fp8_codes (device_common.h, shared with the decode's fp8 append form).  One
// workgroup per token: threads 0-127 take the K row, 128-255 the V row, 16
// elements (16 output bytes) per step.

template <typename Chunk, bool E5>
__global__ void __launch_bounds__(256)
reshape_and_cache_fp8_kernel(const char* __restrict__ key, int64_t key_stride_bytes,
                             const char* __restrict__ value, int64_t value_stride_bytes,
                             uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
                             const int64_t* __restrict__ slot_mapping, int64_t num_slots, int32_t row_elems,
                             float k_scale, float v_scale) {
    const int64_t token = blockIdx.x;
    const int64_t slot = slot_mapping[token];
    if (slot < 0 || slot >= num_slots) return;
    const bool is_v = threadIdx.x >= 128;
    const char* src = is_v ? value + token * value_stride_bytes : key + token * key_stride_bytes;
    uint8_t* dst = (is_v ? value_cache : key_cache) + slot * (int64_t)row_elems;
    const float scale = is_v ? v_scale : k_scale;
    for (int32_t c = threadIdx.x & 127; c < row_elems / 16; c += 128) {
        Chunk x0, x1;
        load_chunk<false>(x0, src + (int64_t)c * 16 * Chunk::kBytes / 8);
        load_chunk<false>(x1, src + ((int64_t)c * 16 + 8) * Chunk::kBytes / 8);
        *reinterpret_cast<u32x4_t*>(dst + (int64_t)c * 16) = fp8_codes<Chunk, E5>(x0, x1, scale);
    }
}

// The slot lookup of pa_slot_mapping and the fp8 scatter above in one launch:
// token t's slot is computed from (token_seq[t], token_pos[t]) and the block
// table (-1 for a padding or unallocated token), written to slot_out[t], and
// the token's rows are quantised into it.  The first 16 elements a thread
// handles are loaded before the slot is known.
template <typename Chunk, bool E5>
__global__ void __launch_bounds__(256)
slot_and_cache_fp8_kernel(int64_t* __restrict__ slot_out, const int32_t* __restrict__ block_table, int32_t bt_stride,
                          int32_t num_seqs, const int32_t* __restrict__ token_seq,
                          const int32_t* __restrict__ token_pos, const char* __restrict__ key,
                          int64_t key_stride_bytes, const char* __restrict__ value, int64_t value_stride_bytes,
                          uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache, int64_t num_slots,
                          int32_t row_elems, float k_scale, float v_scale) {
    const int64_t token = blockIdx.x;
    const bool is_v = threadIdx.x >= 128;
    const int32_t c0 = threadIdx.x & 127;
    const int32_t chunks = row_elems / 16;
    const char* src = is_v ? value + token * value_stride_bytes : key + token * key_stride_bytes;
    Chunk x0, x1;
    if (c0 < chunks) {
        load_chunk<false>(x0, src + (int64_t)c0 * 16 * Chunk::kBytes / 8);
        load_chunk<false>(x1, src + ((int64_t)c0 * 16 + 8) * Chunk::kBytes / 8);
    }
    const int32_t sq = token_seq[token];
    const int32_t p = token_pos[token];
    int64_t slot = -1;
    if (sq >= 0 && sq < num_seqs && p >= 0 && p / kBlock < bt_stride) {
        const int32_t physical = block_table[(int64_t)sq * bt_stride + p / kBlock];
        if (physical >= 0) slot = (int64_t)physical * kBlock + p % kBlock;
    }
    if (threadIdx.x == 0) slot_out[token] = slot;
    if (slot < 0 || slot >= num_slots) return;
    uint8_t* dst = (is_v ? value_cache : key_cache) + slot * (int64_t)row_elems;
    const float scale = is_v ? v_scale : k_scale;
    if (c0 < chunks) *reinterpret_cast<u32x4_t*>(dst + (int64_t)c0 * 16) = fp8_codes<Chunk, E5>(x0, x1, scale);
    for (int32_t c = c0 + 128; c < chunks; c += 128) {      // rows longer than 2048 elements
        load_chunk<false>(x0, src + (int64_t)c * 16 * Chunk::kBytes / 8);
        load_chunk<false>(x1, src + ((int64_t)c * 16 + 8) * Chunk::kBytes / 8);
        *reinterpret_cast<u32x4_t*>(dst + (int64_t)c * 16) = fp8_codes<Chunk, E5>(x0, x1, scale);
    }
}

template <typename Chunk, bool E5>
void slot_and_cache_fp8_typed(int64_t* slot_mapping, const int32_t* block_table, int32_t max_blocks_per_req,
                              int32_t num_seqs, const int32_t* token_seq, const int32_t* token_pos, const void* key,
                              int64_t key_stride_bytes, const void* value, int64_t value_stride_bytes, void* key_cache,
                              void* value_cache, int64_t num_tokens, int64_t num_slots, int32_t row_elems,
                              float k_scale, float v_scale, hipStream_t stream) {
    hipLaunchKernelGGL((slot_and_cache_fp8_kernel<Chunk, E5>), dim3((unsigned)num_tokens), dim3(256), 0, stream,
                       slot_mapping, block_table, max_blocks_per_req, num_seqs, token_seq, token_pos,
                       (const char*)key, key_stride_bytes, (const char*)value, value_stride_bytes,
                       (uint8_t*)key_cache, (uint8_t*)value_cache, num_slots, row_elems, k_scale, v_scale);
}

template <typename Chunk, bool E5>
void reshape_and_cache_fp8_typed(const void* key, int64_t key_stride_bytes, const void* value,
                                 int64_t value_stride_bytes, void* key_cache, void* value_cache,
                                 const int64_t* slot_mapping, int64_t num_tokens, int64_t num_slots,
                                 int32_t row_elems, float k_scale, float v_scale, hipStream_t stream) {
    hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<Chunk, E5>), dim3((unsigned)num_tokens), dim3(256), 0, stream,
                       (const char*)key, key_stride_bytes, (const char*)value, value_stride_bytes,
                       (uint8_t*)key_cache, (uint8_t*)value_cache, slot_mapping, num_slots, row_elems, k_scale,
                       v_scale);
}

hipError_t launch_slot_and_cache_fp8(int64_t* slot_mapping, const int32_t* block_table, int32_t max_blocks_per_req,
                                     int32_t num_seqs, const int32_t* token_seq, const int32_t* token_pos,
                                     const void* key, int64_t key_stride_bytes, const void* value,
                                     int64_t value_stride_bytes, void* key_cache, void* value_cache,
                                     int64_t num_tokens, int64_t num_slots, int32_t row_elems, int dtype, int fmt,
                                     float k_scale, float v_scale, hipStream_t stream) {
    auto run = [&](auto chunk, auto e5) {
        slot_and_cache_fp8_typed<decltype(chunk), decltype(e5)::value>(
            slot_mapping, block_table, max_blocks_per_req, num_seqs, token_seq, token_pos, key, key_stride_bytes,
            value, value_stride_bytes, key_cache, value_cache, num_tokens, num_slots, row_elems, k_scale, v_scale,
            stream);
    };
    if (dtype == 1) {
        if (fmt == 1) run(ChunkBF16{}, std::true_type{}); else run(ChunkBF16{}, std::false_type{});
    } else {
        if (fmt == 1) run(ChunkF32{}, std::true_type{}); else run(ChunkF32{}, std::false_type{});
    }
    return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* key, int64_t key_stride_bytes, const void* value,
                                        int64_t value_stride_bytes, void* key_cache, void* value_cache,
                                        const int64_t* slot_mapping, int64_t num_tokens, int64_t num_slots,
                                        int32_t row_elems, int dtype, int fmt, float k_scale, float v_scale,
                                        hipStream_t stream) {
    auto run = [&](auto chunk, auto e5) {
        reshape_and_cache_fp8_typed<decltype(chunk), decltype(e5)::value>(
            key, key_stride_bytes, value, value_stride_bytes, key_cache, value_cache, slot_mapping, num_tokens,
            num_slots, row_elems, k_scale, v_scale, stream);
    };
    if (dtype == 1) {
        if (fmt == 1) run(ChunkBF16{}, std::true_type{}); else run(ChunkBF16{}, std::false_type{});
    } else {
        if (fmt == 1) run(ChunkF32{}, std::true_type{}); else run(ChunkF32{}, std::false_type{});
    }
    return hipGetLastError();
}

// ---- RoPE + QKV split + scatter ---------------------------------------------
// The step just before attention ("AI Infra入门干货总结：大模型是如何高效推理的",
// section "Reshape & Cache" and its table; the RoPE summary near the article's
// opening): the fused projection row of a token is split into its Q, K and V
// column ranges, Q and K are turned pair by pair by the angles in row
// positions[t] of a [max_position, rotary_dim] cos/sin table, Q goes to
// query_out and K, V go straight into the paged cache at the token's slot.
// One pass over the row: every byte of it is read once and written once.
//
// Work item = 16 elements of one head: for a turned range, both members of
// eight pairs (halves paired: elements 8c.. and R/2 + 8c..; neighbours paired:
// elements 16c .. 16c + 15); past rotary_dim, 16 elements copied as they are.
// Each head has head_dim / 16 items; a token has (Hq + 2 Hkv) * 8 of them (Q
// and K heads turned or copied, V heads copied), spread over one workgroup.
template <typename Chunk, typename Elem>
__global__ void __launch_bounds__(256)
rope_cache_kernel(RopeArgs a) {
    constexpr int kItems = kHeadDim / 16;              // items per head
    const int64_t token = blockIdx.x;
    const int R = a.rotary_dim, half = R / 2, turned = R / 16;
    const int64_t p = min(max(a.positions[token], (int64_t)0), a.max_position - 1);
    const float* cs = a.cos_sin + p * R;
    const int64_t slot = a.slot_mapping[token];
    const bool cached = slot >= 0 && slot < a.num_slots;
    const int64_t cache_row = cached ? slot * (int64_t)a.num_kv_heads * kHeadDim : 0;
    const Elem* row = reinterpret_cast<const Elem*>(a.qkv) + token * a.qkv_stride;
    const int heads = a.num_heads + 2 * a.num_kv_heads;
    for (int it = threadIdx.x; it < heads * kItems; it += blockDim.x) {
        const int h = it / kItems, c = it % kItems;
        const bool is_q = h < a.num_heads, is_v = h >= a.num_heads + a.num_kv_heads;
        if (!is_q && !cached) continue;                // K and V of a padding token go nowhere
        Elem* dst;
        if (is_q) {
            dst = reinterpret_cast<Elem*>(a.query_out) + token * a.q_out_stride + (int64_t)h * kHeadDim;
        } else {
            const int kvh = h - a.num_heads - (is_v ? a.num_kv_heads : 0);
            dst = reinterpret_cast<Elem*>(is_v ? a.value_cache : a.key_cache) + cache_row + (int64_t)kvh * kHeadDim;
        }
        const Elem* src = row + (int64_t)h * kHeadDim;  // Q | K | V heads are consecutive in the row
        int oa, ob;                                     // element offsets of the item's two 8-element chunks
        if (is_v || c >= turned) {
            oa = is_v ? 16 * c : R + 16 * (c - turned);
            ob = oa + 8;
        } else if (a.neox_style) {
            oa = 8 * c;
            ob = half + 8 * c;
        } else {
            oa = 16 * c;
            ob = oa + 8;
        }
        Chunk ca, cb;
        load_chunk<false>(ca, src + oa);
        load_chunk<false>(cb, src + ob);
        if (!is_v && c < turned) {
            float x[8], y[8], co[8], si[8];
            to_f32(ca, x);
            to_f32(cb, y);
            const f32x4_t* cp = reinterpret_cast<const f32x4_t*>(cs + 8 * c);
            const f32x4_t* sp = reinterpret_cast<const f32x4_t*>(cs + half + 8 * c);
            const f32x4_t c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
            co[0] = c0.x; co[1] = c0.y; co[2] = c0.z; co[3] = c0.w;
            co[4] = c1.x; co[5] = c1.y; co[6] = c1.z; co[7] = c1.w;
            si[0] = s0.x; si[1] = s0.y; si[2] = s0.z; si[3] = s0.w;
            si[4] = s1.x; si[5] = s1.y; si[6] = s1.z; si[7] = s1.w;
            if (a.neox_style) {
                // pair j = (x[j], y[j]) with angle j of the chunk
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float u = x[j], v = y[j];
                    x[j] = fmaf(u, co[j], -v * si[j]);
                    y[j] = fmaf(v, co[j], u * si[j]);
                }
            } else {
                // pairs are neighbours: (x[0], x[1]) .. (x[6], x[7]) take angles
                // 0 .. 3 of the chunk, (y[0], y[1]) .. (y[6], y[7]) angles 4 .. 7
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float u = x[2 * j], v = x[2 * j + 1];
                    x[2 * j] = fmaf(u, co[j], -v * si[j]);
                    x[2 * j + 1] = fmaf(v, co[j], u * si[j]);
                    const float w = y[2 * j], z = y[2 * j + 1];
                    y[2 * j] = fmaf(w, co[4 + j], -z * si[4 + j]);
                    y[2 * j + 1] = fmaf(z, co[4 + j], w * si[4 + j]);
                }
            }
            store_chunk(dst + oa, x);
            store_chunk(dst + ob, y);
        } else {
            store_chunk_raw(dst + oa, ca);
            store_chunk_raw(dst + ob, cb);
        }
    }
}

hipError_t launch_rope_cache(const RopeArgs& a, int dtype, hipStream_t stream) {
    if (dtype == 1)
        hipLaunchKernelGGL((rope_cache_kernel<ChunkBF16, uint16_t>), dim3((unsigned)a.num_tokens), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((rope_cache_kernel<ChunkF32, float>), dim3((unsigned)a.num_tokens), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

// Slots and scatter in one launch: workgroup `token` loads its K and V row
// chunks first, then works out the slot exactly as slot_mapping_kernel does
// (the two loads' latencies overlap), thread 0 writes slot_mapping[token],
// and the rows go to cache[slot / 16, slot % 16] as in
// reshape_and_cache_kernel.  The row is at most 256 threads x 16 bytes per
// half (K on threads 0-127, V on 128-255), so each thread holds up to two
// chunks.
__global__ void __launch_bounds__(256)
slot_and_cache_kernel(int64_t* __restrict__ slot_out, const int32_t* __restrict__ block_table,
                      int32_t bt_stride, int32_t num_seqs, const int32_t* __restrict__ token_seq,
                      const int32_t* __restrict__ token_pos, const char* __restrict__ key,
                      int64_t key_stride_bytes, const char* __restrict__ value, int64_t value_stride_bytes,
                      char* __restrict__ key_cache, char* __restrict__ value_cache, int64_t num_slots,
                      int32_t row_bytes) {
    const int64_t token = blockIdx.x;
    const bool is_v = threadIdx.x >= 128;
    const int32_t t = threadIdx.x & 127;
    const int32_t chunks = row_bytes >> 4;
    const char* src = is_v ? value + token * value_stride_bytes : key + token * key_stride_bytes;
    u32x4_t c0 = u32x4_t{0u, 0u, 0u, 0u}, c1 = c0;
    if (t < chunks) c0 = *reinterpret_cast<const u32x4_t*>(src + ((int64_t)t << 4));
    if (t + 128 < chunks) c1 = *reinterpret_cast<const u32x4_t*>(src + ((int64_t)(t + 128) << 4));
    // token_seq null: token i is the newest token of sequence i, at position
    // token_pos[i] - 1 (token_pos then holds the sequence lengths)
    const int32_t sq = token_seq ? token_seq[token] : (int32_t)token;
    const int32_t p = token_seq ? token_pos[token] : token_pos[token] - 1;
    int64_t slot = -1;
    if (sq >= 0 && sq < num_seqs && p >= 0 && p / kBlock < bt_stride) {
        const int32_t physical = block_table[(int64_t)sq * bt_stride + p / kBlock];
        if (physical >= 0) slot = (int64_t)physical * kBlock + p % kBlock;
    }
    if (threadIdx.x == 0 && slot_out) slot_out[token] = slot;
    if (slot < 0 || slot >= num_slots) return;
    char* dst = (is_v ? value_cache : key_cache) + slot * (int64_t)row_bytes;
    if (t < chunks) *reinterpret_cast<u32x4_t*>(dst + ((int64_t)t << 4)) = c0;
    if (t + 128 < chunks) *reinterpret_cast<u32x4_t*>(dst + ((int64_t)(t + 128) << 4)) = c1;
    for (int32_t c = t + 256; c < chunks; c += 128)   // rows longer than 4 KiB
        *reinterpret_cast<u32x4_t*>(dst + ((int64_t)c << 4)) = *reinterpret_cast<const u32x4_t*>(src + ((int64_t)c << 4));
}

hipError_t launch_slot_and_cache(int64_t* slot_mapping, const int32_t* block_table, int32_t max_blocks_per_req,
                                 int32_t num_seqs, const int32_t* token_seq, const int32_t* token_pos,
                                 const void* key, int64_t key_stride_bytes, const void* value,
                                 int64_t value_stride_bytes, void* key_cache, void* value_cache, int64_t num_tokens,
                                 int64_t num_slots, int32_t row_bytes, hipStream_t stream) {
    hipLaunchKernelGGL(slot_and_cache_kernel, dim3((unsigned)num_tokens), dim3(256), 0, stream, slot_mapping,
                       block_table, max_blocks_per_req, num_seqs, token_seq, token_pos, (const char*)key,
                       key_stride_bytes, (const char*)value, value_stride_bytes, (char*)key_cache,
                       (char*)value_cache, num_slots, row_bytes);
    return hipGetLastError();
}

// Mixed-batch attention over an fp32 cache, as one decode row per query row
// (the causal mask of section "Attention (FlashAttention, Scaled Dot-Product
// Attention)" of the same article): row cu_q[b] + j of request b, with
// q = cu_q[b+1] - cu_q[b] rows and L = seq_lens[b] keys, attends keys
// 0 .. L - q + j when causal (all L otherwise), so its decode row has that
// many keys and a copy of the request's block-table row.  One workgroup per
// request; rows outside [0, num_rows) and table entries past the row's keys
// are left alone.
__global__ void __launch_bounds__(256)
expand_rows_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens,
                   const int32_t* __restrict__ block_table, int32_t bt_stride, int64_t num_rows, int32_t causal,
                   int32_t* __restrict__ row_lens, int32_t* __restrict__ row_table, int32_t row_stride) {
    const int b = blockIdx.x;
    const int64_t q0 = cu_q[b], q1 = cu_q[b + 1];
    const int64_t lo = max(q0, (int64_t)0), hi = min(q1, num_rows);
    const int64_t n = hi > lo ? hi - lo : 0;
    const int64_t q = q1 - q0;
    const int32_t L = max(min(seq_lens[b], min(bt_stride, row_stride) * kBlock), 0);
    const int32_t nb = (L + kBlock - 1) / kBlock;
    for (int64_t r = threadIdx.x; r < n; r += blockDim.x) {
        const int64_t j = lo + r - q0;                     // the row's index within the request
        row_lens[lo + r] = causal ? (int32_t)max(min((int64_t)L - q + j + 1, (int64_t)L), (int64_t)0) : L;
    }
    const int32_t* src = block_table + (int64_t)b * bt_stride;
    for (int64_t e = threadIdx.x; e < n * nb; e += blockDim.x) {
        const int64_t r = e / nb;
        const int32_t i = (int32_t)(e - r * nb);
        row_table[(lo + r) * row_stride + i] = src[i];
    }
}

hipError_t launch_expand_rows(const int32_t* cu_query_lens, const int32_t* seq_lens, const int32_t* block_table,
                              int32_t max_blocks_per_req, int32_t num_seqs, int64_t num_rows, int32_t causal,
                              int32_t* row_lens, int32_t* row_table, int32_t row_stride, hipStream_t stream) {
    hipLaunchKernelGGL(expand_rows_kernel, dim3((unsigned)num_seqs), dim3(256), 0, stream, cu_query_lens, seq_lens,
                       block_table, max_blocks_per_req, num_rows, causal, row_lens, row_table, row_stride);
    return hipGetLastError();
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
