// C ABI of libpa.so: argument checks, partition choice, workspace layout and
// dispatch to the gfx950 kernels.  Declarations and the contract are in
// include/pa.h.
#include "pa.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "host_status.h"
#include "launch.h"
#include "validate.h"

namespace {

thread_local char g_err[512] = "";

pa_status fail(pa_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

pa_status ok() {
    g_err[0] = '\0';
    return PA_OK;
}

pa_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

namespace pa {

pa_status report(pa_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

pa_status report_ok() { return ok(); }

}  // namespace pa

namespace {

int elem_bytes(pa_dtype d) { return d == PA_BF16 ? 2 : 4; }

// Sequences at most this many use the balanced stream mode when the caller
// leaves the split to the library (its workgroups keep a block-count prefix of
// every sequence in LDS).
constexpr int32_t kStreamMaxSeqs = 4096;
// Fewest blocks a stream workgroup takes, so that tiny batches are not cut
// into pieces smaller than the merge is worth.
constexpr int32_t kStreamMinQuantum = 8;

// Tokens per partition for the partitioned mode.  An explicit size is used as
// given; 0 (when the stream mode does not apply) picks the smallest of 256 /
// 512 / 1024 tokens that still gives every compute unit several waves; -1 (or
// a size at least max_seq_len) keeps every sequence in one partition.
int32_t choose_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                         int32_t requested) {
    const int32_t whole = max_seq_len > 0 ? ((max_seq_len + 15) / 16) * 16 : 16;
    if (requested < 0) return whole;
    if (requested > 0) return requested < whole ? requested : whole;
    const int64_t units = (int64_t)num_seqs * num_kv_heads;
    int32_t pt = 256;
    while (pt < 1024 && units * ((max_seq_len + pt - 1) / pt) > 16384) pt *= 2;
    return pt < whole ? pt : whole;
}

int32_t num_partitions(int32_t max_seq_len, int32_t pt) {
    return max_seq_len <= 0 ? 1 : (max_seq_len + pt - 1) / pt;
}

bool use_stream(int32_t num_seqs, int32_t partition_tokens) {
    return partition_tokens == 0 && num_seqs <= kStreamMaxSeqs;
}

// Stream-mode workgroups one compute unit of the current device holds at
// once, for `waves` KV heads (one wave each) per workgroup; cached.
int32_t stream_blocks_per_cu(int dtype, int32_t group, int32_t waves, int32_t num_seqs) {
    struct Entry { int dev, dtype, group, waves, lds_kib, n; };
    static std::mutex mu;
    static Entry cache[128];
    static int ncache = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const int lds_kib = (int)((((int64_t)num_seqs + 1) * 4 + 1023) / 1024);
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < ncache; ++i)
            if (cache[i].dev == dev && cache[i].dtype == dtype && cache[i].group == group &&
                cache[i].waves == waves && cache[i].lds_kib == lds_kib)
                return cache[i].n;
    }
    const int n = pa::decode_stream_blocks_per_cu(dtype, group, waves, lds_kib * 256 - 1);
    std::lock_guard<std::mutex> lock(mu);
    if (ncache < 128) cache[ncache++] = Entry{dev, dtype, group, waves, lds_kib, n};
    return n;
}

int32_t device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
}

// Stream-mode layout: the KV heads per workgroup (a divisor of num_kv_heads,
// at most 8) that keep the most waves resident per compute unit (ties go to
// the wider workgroup, whose waves read neighbouring rows of the same blocks),
// and the grid: every such workgroup the device holds at once.
struct StreamShape { int32_t waves, num_wg; };

StreamShape stream_shape(int dtype, int32_t group, int32_t num_kv_heads, int32_t num_seqs) {
    StreamShape best{1, 0};
    int32_t best_resident = 0;
    const int32_t cus = device_cus();
    if (cus <= 0) return best;
    for (int32_t w = 8; w >= 1; --w) {
        if (num_kv_heads % w) continue;
        const int32_t per_cu = stream_blocks_per_cu(dtype, group, w, num_seqs);
        if (per_cu * w > best_resident) {
            best_resident = per_cu * w;
            best = StreamShape{w, per_cu * cus};
        }
    }
    return best;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the partitioned mode: partial records of every split
// (sequence, head, partition).
size_t partition_ws_bytes(int32_t num_seqs, int32_t num_heads, int32_t nparts) {
    if (nparts <= 1) return 0;
    return (size_t)num_seqs * num_heads * nparts * pa::kDecodeRecordFloats * sizeof(float);
}

// Workspace of the stream mode: the block prefix, then two partial records per
// (workgroup, query head of its waves).
size_t stream_ws_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, StreamShape sh) {
    const int32_t waves = sh.waves, num_wg = sh.num_wg;
    const int32_t group = num_heads / num_kv_heads;
    return align256(((size_t)num_seqs + 1) * sizeof(int32_t)) +
           (size_t)num_wg * 2 * waves * group * pa::kDecodeRecordFloats * sizeof(float);
}


// Prefill grid: slots_per_kvh workgroups per KV head, filling the workgroups
// the device holds at once (at least one per KV head).  tiles bounds the
// query tiles from the host-side sizes.
struct PrefillShape { int64_t tiles; int32_t slots_per_kvh; };

constexpr int32_t kPrefillMinShare = 8;    // key tiles (512 keys)

PrefillShape prefill_shape(int32_t num_seqs, int64_t num_q_tokens, int32_t max_query_len, int32_t num_heads,
                           int32_t num_kv_heads) {
    const int32_t group = num_heads / num_kv_heads;
    const int64_t tq = pa::kPrefillRows / group;
    const int64_t half = num_q_tokens / 2;
    const int64_t by_tokens = (num_q_tokens + tq - 1) / tq + (num_seqs < half ? num_seqs : half);
    const int64_t by_seqs = (int64_t)num_seqs * ((max_query_len + tq - 1) / tq);
    PrefillShape p{};
    p.tiles = by_tokens < by_seqs ? by_tokens : by_seqs;
    int32_t per_cu = 0;
    {
        static std::mutex mu;
        static int cached_dev = -1, cached_group = 0, cached_kib = 0, cached_n = 0;
        int dev = 0;
        const int kib = (int)((((int64_t)num_seqs + 1) * 4 + 1023) / 1024);
        if (hipGetDevice(&dev) == hipSuccess) {
            std::lock_guard<std::mutex> lock(mu);
            if (dev != cached_dev || group != cached_group || kib != cached_kib) {
                cached_n = pa::prefill_blocks_per_cu(group, kib * 256 - 1);
                cached_dev = dev, cached_group = group, cached_kib = kib;
            }
            per_cu = cached_n;
        }
    }
    const int64_t slots = (int64_t)per_cu * device_cus();
    p.slots_per_kvh = slots > 0 ? (int32_t)std::min<int64_t>(std::max<int64_t>(1, slots / num_kv_heads),
                                                            pa::kPrefillMaxSlots)
                                : 0;
    return p;
}

// Prefill scratch: two partial records per workgroup, then the list of tiles
// to merge (a count, then one 16-byte entry per share boundary).
size_t prefill_records_bytes(const PrefillShape& p, int32_t num_kv_heads) {
    return (size_t)p.slots_per_kvh * num_kv_heads * 2 * pa::kPrefillRows * pa::kDecodeRecordFloats * sizeof(float);
}

size_t prefill_list_entries(const PrefillShape& p, int32_t num_kv_heads) {
    return (size_t)(p.slots_per_kvh - 1) * num_kv_heads + 1;
}

size_t prefill_part_bytes(const PrefillShape& p, int32_t num_kv_heads) {
    return prefill_records_bytes(p, num_kv_heads) + 16 + 16 * prefill_list_entries(p, num_kv_heads);
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(pa_status s) {
    switch (s) {
        case PA_OK: return "PA_OK";
        case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
        case PA_ERR_HIP: return "PA_ERR_HIP";
        default: break;
    }
    return "PA_ERR_UNKNOWN";
}

const char* pa_last_error_message(void) { return g_err; }

pa_status pa_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                          int32_t max_blocks_per_req, int32_t num_seqs,
                          const int32_t* token_seq, const int32_t* token_pos,
                          int64_t num_tokens, int32_t block_size, hipStream_t stream) {
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
    if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d (only 16)", block_size);
    if (num_tokens == 0) return ok();
    if (!slot_mapping || !token_seq || !token_pos) return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (num_seqs < 0 || max_blocks_per_req < 0) return fail(PA_ERR_INVALID_ARG, "negative table shape");
    if (num_seqs > 0 && max_blocks_per_req > 0 && !block_table)
        return fail(PA_ERR_INVALID_ARG, "null block_table");
    if (num_tokens > ((int64_t)1 << 31) * 256 - 1) return fail(PA_ERR_INVALID_ARG, "num_tokens too large");
    return hip_status(pa::launch_slot_mapping(slot_mapping, block_table, max_blocks_per_req, num_seqs,
                                              token_seq, token_pos, num_tokens, stream),
                      "slot_mapping launch");
}

pa_status pa_slot_mapping_and_cache(int64_t* slot_mapping, const int32_t* block_table, int32_t max_blocks_per_req,
                                    int32_t num_seqs, const int32_t* token_seq, const int32_t* token_pos,
                                    const void* key, int64_t key_token_stride, const void* value,
                                    int64_t value_token_stride, void* key_cache, void* value_cache,
                                    int64_t num_tokens, int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                    int32_t head_dim, pa_dtype dtype, hipStream_t stream) {
    if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
    if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d (only 16)", block_size);
    if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_seqs < 0 ||
        max_blocks_per_req < 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size");
    if (num_tokens == 0) return ok();
    if (!slot_mapping || !token_seq || !token_pos || !key || !value || !key_cache || !value_cache)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (num_seqs > 0 && max_blocks_per_req > 0 && !block_table) return fail(PA_ERR_INVALID_ARG, "null block_table");
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    const int64_t eb = elem_bytes(dtype);
    const int64_t row_bytes = row_elems * eb;
    if (row_bytes % 16 != 0 || row_bytes > (1 << 30))
        return fail(PA_ERR_UNSUPPORTED, "row of %lld bytes (must be a multiple of 16)", (long long)row_bytes);
    if (key_token_stride < row_elems || value_token_stride < row_elems)
        return fail(PA_ERR_INVALID_ARG, "token stride smaller than num_kv_heads * head_dim");
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
        (key_token_stride * eb) % 16 || (value_token_stride * eb) % 16)
        return fail(PA_ERR_INVALID_ARG, "rows must start on 16-byte boundaries");
    if (num_tokens > 0x7fffffff) return fail(PA_ERR_INVALID_ARG, "num_tokens too large");
    return hip_status(pa::launch_slot_and_cache(slot_mapping, block_table, max_blocks_per_req, num_seqs, token_seq,
                                                token_pos, key, key_token_stride * eb, value,
                                                value_token_stride * eb, key_cache, value_cache, num_tokens,
                                                num_blocks * 16, (int32_t)row_bytes, stream),
                      "slot_and_cache launch");
}

pa_status pa_reshape_and_cache(const void* key, int64_t key_token_stride, const void* value,
                               int64_t value_token_stride, void* key_cache, void* value_cache,
                               const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                               int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                               pa_dtype dtype, hipStream_t stream) {
    if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
    if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d (only 16)", block_size);
    if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size");
    if (num_tokens == 0) return ok();
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    const int64_t eb = elem_bytes(dtype);
    const int64_t row_bytes = row_elems * eb;
    if (row_bytes % 16 != 0 || row_bytes > (1 << 30))
        return fail(PA_ERR_UNSUPPORTED, "row of %lld bytes (must be a multiple of 16)", (long long)row_bytes);
    if (key_token_stride < row_elems || value_token_stride < row_elems)
        return fail(PA_ERR_INVALID_ARG, "token stride smaller than num_kv_heads * head_dim");
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
        (key_token_stride * eb) % 16 || (value_token_stride * eb) % 16)
        return fail(PA_ERR_INVALID_ARG, "rows must start on 16-byte boundaries");
    if (num_tokens > 0x7fffffff) return fail(PA_ERR_INVALID_ARG, "num_tokens too large");
    if (pa::debug_checks_enabled(stream)) {
        const pa_status dc = pa::debug_check_slots(slot_mapping, num_tokens, num_blocks, stream);
        if (dc != PA_OK) return dc;
    }
    return hip_status(pa::launch_reshape_and_cache(key, key_token_stride * eb, value,
                                                   value_token_stride * eb, key_cache, value_cache,
                                                   slot_mapping, num_tokens, num_blocks * 16,
                                                   (int32_t)row_bytes, stream),
                      "reshape_and_cache launch");
}

pa_status pa_copy_blocks(void* key_cache, void* value_cache, int64_t layer_stride_bytes, int32_t num_layers,
                         int64_t num_blocks, int64_t block_bytes, const int64_t* block_mapping, int64_t num_pairs,
                         hipStream_t stream) {
    if (num_layers < 0 || num_blocks < 0 || block_bytes <= 0 || num_pairs < 0 || layer_stride_bytes < 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size");
    if (num_pairs == 0 || num_layers == 0) return ok();
    if (!key_cache || !value_cache || !block_mapping) return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (block_bytes % 16 || !aligned16(key_cache) || !aligned16(value_cache) || layer_stride_bytes % 16)
        return fail(PA_ERR_INVALID_ARG, "blocks and layers must start on 16-byte boundaries");
    if (num_layers > 1 && layer_stride_bytes < num_blocks * block_bytes)
        return fail(PA_ERR_INVALID_ARG, "layer stride shorter than a layer's blocks");
    if (num_pairs > 0x7fffffff || num_layers > 32767) return fail(PA_ERR_INVALID_ARG, "grid too large");
    return hip_status(pa::launch_copy_blocks(key_cache, value_cache, layer_stride_bytes, num_layers, num_blocks,
                                             block_bytes, block_mapping, num_pairs, stream),
                      "copy_blocks launch");
}

pa_status pa_reshape_and_cache_fp8_ex(const void* key, int64_t key_token_stride, const void* value,
                                      int64_t value_token_stride, void* key_cache, void* value_cache,
                                      const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                                      int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                      pa_fp8_format format, float k_scale, float v_scale, hipStream_t stream) {
    if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "source dtype %d", (int)dtype);
    if (format != PA_FP8_E4M3 && format != PA_FP8_E5M2) return fail(PA_ERR_UNSUPPORTED, "fp8 format %d", (int)format);
    if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d (only 16)", block_size);
    if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size");
    if (!(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
        return fail(PA_ERR_INVALID_ARG, "scales must be finite and positive");
    if (num_tokens == 0) return ok();
    if (!key || !value || !key_cache || !value_cache || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "null pointer");
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    const int64_t eb = elem_bytes(dtype);
    if (row_elems % 16 != 0 || row_elems > (1 << 28))
        return fail(PA_ERR_UNSUPPORTED, "row of %lld elements (must be a multiple of 16)", (long long)row_elems);
    if (key_token_stride < row_elems || value_token_stride < row_elems)
        return fail(PA_ERR_INVALID_ARG, "token stride smaller than num_kv_heads * head_dim");
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
        (key_token_stride * eb) % 16 || (value_token_stride * eb) % 16)
        return fail(PA_ERR_INVALID_ARG, "rows must start on 16-byte boundaries");
    if (num_tokens > 0x7fffffff) return fail(PA_ERR_INVALID_ARG, "num_tokens too large");
    if (pa::debug_checks_enabled(stream)) {
        const pa_status dc = pa::debug_check_slots(slot_mapping, num_tokens, num_blocks, stream);
        if (dc != PA_OK) return dc;
    }
    return hip_status(pa::launch_reshape_and_cache_fp8(key, key_token_stride * eb, value, value_token_stride * eb,
                                                       key_cache, value_cache, slot_mapping, num_tokens,
                                                       num_blocks * 16, (int32_t)row_elems,
                                                       dtype == PA_BF16 ? 1 : 0, format == PA_FP8_E5M2 ? 1 : 0,
                                                       k_scale, v_scale, stream),
                      "reshape_and_cache_fp8 launch");
}

pa_status pa_reshape_and_cache_fp8(const void* key, int64_t key_token_stride, const void* value,
                                   int64_t value_token_stride, void* key_cache, void* value_cache,
                                   const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                                   int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                   float k_scale, float v_scale, hipStream_t stream) {
    return pa_reshape_and_cache_fp8_ex(key, key_token_stride, value, value_token_stride, key_cache, value_cache,
                                       slot_mapping, num_tokens, num_blocks, block_size, num_kv_heads, head_dim,
                                       dtype, PA_FP8_E4M3, k_scale, v_scale, stream);
}

pa_status pa_slot_mapping_and_cache_fp8_ex(int64_t* slot_mapping, const int32_t* block_table,
                                           int32_t max_blocks_per_req, int32_t num_seqs, const int32_t* token_seq,
                                           const int32_t* token_pos, const void* key, int64_t key_token_stride,
                                           const void* value, int64_t value_token_stride, void* key_cache,
                                           void* value_cache, int64_t num_tokens, int64_t num_blocks,
                                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                           pa_fp8_format format, float k_scale, float v_scale, hipStream_t stream) {
    if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "source dtype %d", (int)dtype);
    if (format != PA_FP8_E4M3 && format != PA_FP8_E5M2) return fail(PA_ERR_UNSUPPORTED, "fp8 format %d", (int)format);
    if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d (only 16)", block_size);
    if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_seqs < 0 ||
        max_blocks_per_req < 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size");
    if (!(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
        return fail(PA_ERR_INVALID_ARG, "scales must be finite and positive");
    if (num_tokens == 0) return ok();
    if (!slot_mapping || !token_seq || !token_pos || !key || !value || !key_cache || !value_cache)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (num_seqs > 0 && max_blocks_per_req > 0 && !block_table) return fail(PA_ERR_INVALID_ARG, "null block_table");
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    const int64_t eb = elem_bytes(dtype);
    if (row_elems % 16 != 0 || row_elems > (1 << 28))
        return fail(PA_ERR_UNSUPPORTED, "row of %lld elements (must be a multiple of 16)", (long long)row_elems);
    if (key_token_stride < row_elems || value_token_stride < row_elems)
        return fail(PA_ERR_INVALID_ARG, "token stride smaller than num_kv_heads * head_dim");
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
        (key_token_stride * eb) % 16 || (value_token_stride * eb) % 16)
        return fail(PA_ERR_INVALID_ARG, "rows must start on 16-byte boundaries");
    if (num_tokens > 0x7fffffff) return fail(PA_ERR_INVALID_ARG, "num_tokens too large");
    return hip_status(pa::launch_slot_and_cache_fp8(slot_mapping, block_table, max_blocks_per_req, num_seqs, token_seq,
                                                    token_pos, key, key_token_stride * eb, value,
                                                    value_token_stride * eb, key_cache, value_cache, num_tokens,
                                                    num_blocks * 16, (int32_t)row_elems, dtype == PA_BF16 ? 1 : 0,
                                                    format == PA_FP8_E5M2 ? 1 : 0, k_scale, v_scale, stream),
                      "slot_and_cache_fp8 launch");
}

pa_status pa_slot_mapping_and_cache_fp8(int64_t* slot_mapping, const int32_t* block_table,
                                        int32_t max_blocks_per_req, int32_t num_seqs, const int32_t* token_seq,
                                        const int32_t* token_pos, const void* key, int64_t key_token_stride,
                                        const void* value, int64_t value_token_stride, void* key_cache,
                                        void* value_cache, int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                                        int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype, float k_scale,
                                        float v_scale, hipStream_t stream) {
    return pa_slot_mapping_and_cache_fp8_ex(slot_mapping, block_table, max_blocks_per_req, num_seqs, token_seq,
                                            token_pos, key, key_token_stride, value, value_token_stride, key_cache,
                                            value_cache, num_tokens, num_blocks, block_size, num_kv_heads, head_dim,
                                            dtype, PA_FP8_E4M3, k_scale, v_scale, stream);
}

pa_status pa_rope_reshape_and_cache(void* query_out, int64_t q_out_token_stride, const void* qkv,
                                    int64_t qkv_token_stride, const int64_t* positions, const float* cos_sin_cache,
                                    int64_t max_position, int32_t rotary_dim, int32_t neox_style, void* key_cache,
                                    void* value_cache, const int64_t* slot_mapping, int64_t num_tokens,
                                    int64_t num_blocks, int32_t block_size, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, pa_dtype dtype, hipStream_t stream) {
    if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
    if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d (only 16)", block_size);
    if (head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d (only 128)", head_dim);
    if (rotary_dim < 16 || rotary_dim > head_dim || rotary_dim % 16)
        return fail(PA_ERR_UNSUPPORTED, "rotary_dim %d (a multiple of 16 in [16, head_dim])", rotary_dim);
    if (num_tokens < 0 || num_blocks < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_position <= 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size");
    if (num_tokens == 0) return ok();
    if (!query_out || !qkv || !positions || !cos_sin_cache || !key_cache || !value_cache || !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (num_tokens > 0x7fffffff) return fail(PA_ERR_INVALID_ARG, "num_tokens too large");
    if ((int64_t)num_heads + 2 * (int64_t)num_kv_heads > (1 << 20))
        return fail(PA_ERR_UNSUPPORTED, "too many heads");
    const int64_t eb = elem_bytes(dtype);
    const int64_t width = ((int64_t)num_heads + 2 * (int64_t)num_kv_heads) * head_dim;
    if (qkv_token_stride < width)
        return fail(PA_ERR_INVALID_ARG, "qkv token stride %lld below (num_heads + 2 num_kv_heads) * head_dim",
                    (long long)qkv_token_stride);
    if (q_out_token_stride < (int64_t)num_heads * head_dim)
        return fail(PA_ERR_INVALID_ARG, "query_out token stride below num_heads * head_dim");
    if (!aligned16(query_out) || !aligned16(qkv) || !aligned16(key_cache) || !aligned16(value_cache) ||
        !aligned16(cos_sin_cache) || (qkv_token_stride * eb) % 16 || (q_out_token_stride * eb) % 16)
        return fail(PA_ERR_INVALID_ARG, "rows must start on 16-byte boundaries");
    if (query_out == qkv && q_out_token_stride != qkv_token_stride)
        return fail(PA_ERR_INVALID_ARG, "in place, query_out must use the qkv row stride");
    pa::RopeArgs a{};
    a.query_out = query_out;
    a.q_out_stride = q_out_token_stride;
    a.qkv = qkv;
    a.qkv_stride = qkv_token_stride;
    a.positions = positions;
    a.cos_sin = cos_sin_cache;
    a.max_position = max_position;
    a.rotary_dim = rotary_dim;
    a.neox_style = neox_style ? 1 : 0;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.slot_mapping = slot_mapping;
    a.num_slots = num_blocks * 16;
    a.num_tokens = num_tokens;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    return hip_status(pa::launch_rope_cache(a, dtype == PA_BF16 ? 1 : 0, stream), "rope_reshape_and_cache launch");
}

int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                                   int32_t partition_tokens) {
    if (use_stream(num_seqs, partition_tokens)) return 0;
    return choose_partition(num_seqs, num_kv_heads, max_seq_len, partition_tokens);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t partition_tokens) {
    if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_heads % num_kv_heads)
        return 0;
    if (use_stream(num_seqs, partition_tokens)) {
        const int32_t group = num_heads / num_kv_heads;
        size_t bytes = 0;
        for (int dtype = 0; dtype < 7; ++dtype) {          // the largest of the layouts (fp32, bf16, E4M3 cache,
                                                           // append, E5M2 cache, the fp8 append forms)
            const size_t n = stream_ws_bytes(num_seqs, num_heads, num_kv_heads,
                                             stream_shape(dtype, group, num_kv_heads, num_seqs));
            bytes = n > bytes ? n : bytes;
        }
        return bytes;
    }
    const int32_t pt = choose_partition(num_seqs, num_kv_heads, max_seq_len, partition_tokens);
    size_t bytes = partition_ws_bytes(num_seqs, num_heads, num_partitions(max_seq_len, pt));
    if (partition_tokens == 0) {
        // pa_decode_fp8 and pa_decode_append_fp8 read a larger batch in
        // groups of kStreamMaxSeqs sequences, one stream-mode launch each, on
        // this one workspace
        const int32_t group = num_heads / num_kv_heads;
        for (int dtype : {2, 4, 5, 6}) {
            const size_t n = stream_ws_bytes(kStreamMaxSeqs, num_heads, num_kv_heads,
                                             stream_shape(dtype, group, num_kv_heads, kStreamMaxSeqs));
            bytes = n > bytes ? n : bytes;
        }
    }
    return bytes;
}

}  // extern "C"

namespace {

// A decode launch whose arguments have passed every check: what
// plan_decode fills in and launch_planned enqueues.
struct DecodePlan {
    pa::DecodeArgs a;
    int dt;
    int group;
};

// Checks shared by pa_decode and pa_chunked_prefill (grid, workspace size and
// alignment) and the kernel arguments, without launching anything (cu_q !=
// nullptr: only the single-row sequences of a mixed batch).
pa_status plan_decode(DecodePlan& plan, void* out, const void* query, int64_t q_token_stride, const void* key_cache,
                        const void* value_cache, const int32_t* block_table, int32_t max_blocks_per_req,
                        const int32_t* seq_lens, const int32_t* cu_q, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int64_t num_blocks, float scale, int32_t max_seq_len,
                        int32_t partition_tokens, void* workspace, size_t workspace_bytes, int dt, float k_scale,
                        float v_scale, const void* new_key = nullptr, int64_t new_key_stride_bytes = 0,
                        const void* new_value = nullptr, int64_t new_value_stride_bytes = 0,
                        int64_t* slot_out = nullptr) {
    // dt: 0 fp32, 1 bf16, 2 E4M3 / 4 E5M2 cache (bf16 query and output, stream mode only),
    // 3 bf16 in append mode (stream mode only; the new_* rows and slot_out), 5 E4M3 / 6 E5M2
    // cache in append mode (the same, and the rows stored as codes before they are read)
    const int32_t group = num_heads / num_kv_heads;
    plan.dt = dt;
    plan.group = group;
    pa::DecodeArgs& a = plan.a;
    a = pa::DecodeArgs{};
    a.out = out;
    a.query = query;
    a.q_stride = q_token_stride;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_table = block_table;
    a.bt_stride = max_blocks_per_req;
    a.num_blocks = num_blocks;
    a.seq_lens = seq_lens;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.scale_log2 = (float)((double)scale * (double)k_scale * 1.4426950408889634);
    a.out_scale = v_scale;
    a.cu_q = cu_q;
    a.new_key = static_cast<const char*>(new_key);
    a.new_value = static_cast<const char*>(new_value);
    a.new_key_stride = new_key_stride_bytes;
    a.new_value_stride = new_value_stride_bytes;
    a.slot_out = slot_out;
    a.k_scale = k_scale;
    a.v_scale = v_scale;

    size_t need = 0;
    if (use_stream(num_seqs, partition_tokens)) {
        const StreamShape sh = stream_shape(dt, group, num_kv_heads, num_seqs);
        if (sh.num_wg <= 0) return fail(PA_ERR_HIP, "cannot size the decode grid for the current device");
        need = stream_ws_bytes(num_seqs, num_heads, num_kv_heads, sh);
        a.mode = pa::kDecodeStream;
        a.waves_per_group = sh.waves;
        a.num_wg = sh.num_wg;
        a.min_quantum = kStreamMinQuantum;
        // The merge runs one wave per (sequence, query head), 8 resident per
        // SIMD.  Beyond one round of them (32 per compute unit), a wave takes
        // two heads of a KV head (group >= 2), one per half.
        a.merge_pair = group >= 2 && (int64_t)num_seqs * num_heads > 32LL * device_cus();
        if (workspace) {
            a.prefix = reinterpret_cast<int32_t*>(workspace);
            a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                              align256(((size_t)num_seqs + 1) * sizeof(int32_t)));
        }
    } else {
        const int32_t pt = choose_partition(num_seqs, num_kv_heads, max_seq_len, partition_tokens);
        const int32_t nparts = num_partitions(max_seq_len, pt);
        need = partition_ws_bytes(num_seqs, num_heads, nparts);
        const int64_t items = (int64_t)num_seqs * nparts * num_kv_heads;
        if ((items + 3) / 4 > 0x7fffffff) return fail(PA_ERR_INVALID_ARG, "grid too large");
        a.mode = pa::kDecodePartitions;
        a.partition_tokens = pt;
        a.max_partitions = nparts;
        a.part = reinterpret_cast<float*>(workspace);
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace ? workspace_bytes : 0,
                    need);
    if (need > 0 && !aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    return PA_OK;
}

pa_status launch_planned(const DecodePlan& plan, hipStream_t stream) {
    return hip_status(pa::launch_decode(plan.a, plan.dt, plan.group, stream), "decode launch");
}

// plan_decode, then its launch.
pa_status decode_common(void* out, const void* query, int64_t q_token_stride, const void* key_cache,
                        const void* value_cache, const int32_t* block_table, int32_t max_blocks_per_req,
                        const int32_t* seq_lens, const int32_t* cu_q, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int64_t num_blocks, float scale, int32_t max_seq_len,
                        int32_t partition_tokens, void* workspace, size_t workspace_bytes, int dt, float k_scale,
                        float v_scale, hipStream_t stream, const void* new_key = nullptr,
                        int64_t new_key_stride_bytes = 0, const void* new_value = nullptr,
                        int64_t new_value_stride_bytes = 0, int64_t* slot_out = nullptr) {
    DecodePlan plan;
    const pa_status st = plan_decode(plan, out, query, q_token_stride, key_cache, value_cache, block_table,
                                     max_blocks_per_req, seq_lens, cu_q, num_seqs, num_heads, num_kv_heads,
                                     num_blocks, scale, max_seq_len, partition_tokens, workspace, workspace_bytes,
                                     dt, k_scale, v_scale, new_key, new_key_stride_bytes, new_value,
                                     new_value_stride_bytes, slot_out);
    if (st != PA_OK) return st;
    return launch_planned(plan, stream);
}

// Shape checks shared by the attention entry points.
pa_status check_heads(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d (only 16)", block_size);
    if (head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d (only 128)", head_dim);
    if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads)
        return fail(PA_ERR_INVALID_ARG, "num_heads %d not a multiple of num_kv_heads %d", num_heads,
                    num_kv_heads);
    const int32_t group = num_heads / num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return fail(PA_ERR_UNSUPPORTED, "group size %d (supported: 1, 2, 4, 8)", group);
    return PA_OK;
}

// Workspace of the fp32 mixed batch: one decode row per query row, its key
// count and block-table row (stride: the blocks of max_seq_len), then the
// decode's own workspace.
struct F32Rows {
    int32_t row_stride;
    size_t table_off, table_bytes;
};
F32Rows f32_rows(int64_t rows, int32_t max_seq_len) {
    F32Rows f;
    f.row_stride = (int32_t)std::max<int64_t>(((int64_t)max_seq_len + 15) / 16, 1);
    f.table_off = align256((size_t)rows * sizeof(int32_t));
    f.table_bytes = align256((size_t)rows * (size_t)f.row_stride * sizeof(int32_t));
    return f;
}

// pa_decode_fp8_ex, and with append pa_decode_append_fp8 (the newest rows
// stored as codes by the decode launch itself).
pa_status decode_fp8_common(void* out, const void* query, int64_t q_token_stride, const void* key,
                            int64_t key_token_stride, const void* value, int64_t value_token_stride,
                            const void* key_cache, const void* value_cache, int64_t* slot_mapping,
                            const int32_t* block_table, int32_t max_blocks_per_req, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int64_t num_blocks, float scale, pa_fp8_format format,
                            float k_scale, float v_scale, int32_t max_seq_len, void* workspace,
                            size_t workspace_bytes, bool append, hipStream_t stream) {
    if (format != PA_FP8_E4M3 && format != PA_FP8_E5M2) return fail(PA_ERR_UNSUPPORTED, "fp8 format %d", (int)format);
    const pa_status hs = check_heads(num_heads, num_kv_heads, head_dim, block_size);
    if (hs != PA_OK) return hs;
    if (num_seqs < 0 || num_blocks < 0 || max_seq_len < 0 || max_blocks_per_req < 0)
        return fail(PA_ERR_INVALID_ARG, "negative size");
    if (!(isfinite(scale) && scale > 0.f)) return fail(PA_ERR_INVALID_ARG, "scale must be finite and positive");
    if (!(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
        return fail(PA_ERR_INVALID_ARG, "scales must be finite and positive");
    if ((int64_t)max_seq_len > (int64_t)max_blocks_per_req * 16)
        return fail(PA_ERR_INVALID_ARG, "max_seq_len %d exceeds max_blocks_per_req * 16", max_seq_len);
    if (num_seqs == 0) return ok();
    if (num_blocks == 0 && max_seq_len > 0) return fail(PA_ERR_INVALID_ARG, "empty cache pool");
    if (!out || !query || !seq_lens || !key_cache || !value_cache || (max_seq_len > 0 && !block_table) ||
        (append && (!key || !value)))
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (q_token_stride < (int64_t)num_heads * head_dim)
        return fail(PA_ERR_INVALID_ARG, "q_token_stride smaller than num_heads * head_dim");
    if (!aligned16(query) || (q_token_stride * 2) % 16 || !aligned16(out) || !aligned16(key_cache) ||
        !aligned16(value_cache))
        return fail(PA_ERR_INVALID_ARG, "query/out/cache rows must start on 16-byte boundaries");
    if (append) {
        const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
        if (key_token_stride < row_elems || value_token_stride < row_elems)
            return fail(PA_ERR_INVALID_ARG, "key/value token stride smaller than num_kv_heads * head_dim");
        if (!aligned16(key) || !aligned16(value) || (key_token_stride * 2) % 16 || (value_token_stride * 2) % 16)
            return fail(PA_ERR_INVALID_ARG, "key/value rows must start on 16-byte boundaries");
    }
    if (pa::debug_checks_enabled(stream)) {
        // (append: the newest token is read from the cache, so it needs its block)
        const pa_status dc = pa::debug_check_tables(block_table, max_blocks_per_req, seq_lens, num_seqs, num_blocks,
                                                    max_seq_len, stream);
        if (dc != PA_OK) return dc;
    }
    // An fp8 cache is read in the stream mode only, which takes at most
    // kStreamMaxSeqs sequences: a larger batch runs as consecutive launches
    // over groups of that many, each reusing the workspace after the one
    // before it on the stream.  Every group is planned before the first
    // launch.
    const int dt = append ? (format == PA_FP8_E5M2 ? 6 : 5) : (format == PA_FP8_E5M2 ? 4 : 2);
    std::vector<DecodePlan> plans((size_t)((num_seqs + kStreamMaxSeqs - 1) / kStreamMaxSeqs));
    for (size_t g = 0; g < plans.size(); ++g) {
        const int32_t c0 = (int32_t)g * kStreamMaxSeqs;
        const int32_t n = std::min(kStreamMaxSeqs, num_seqs - c0);
        const pa_status st = plan_decode(
            plans[g], static_cast<char*>(out) + (int64_t)c0 * num_heads * head_dim * 2,
            static_cast<const char*>(query) + (int64_t)c0 * q_token_stride * 2, q_token_stride, key_cache,
            value_cache, block_table ? block_table + (int64_t)c0 * max_blocks_per_req : nullptr, max_blocks_per_req,
            seq_lens + c0, nullptr, n, num_heads, num_kv_heads, num_blocks, scale, max_seq_len, 0, workspace,
            workspace_bytes, dt, k_scale, v_scale,
            append ? static_cast<const char*>(key) + (int64_t)c0 * key_token_stride * 2 : nullptr,
            key_token_stride * 2,
            append ? static_cast<const char*>(value) + (int64_t)c0 * value_token_stride * 2 : nullptr,
            value_token_stride * 2, append && slot_mapping ? slot_mapping + c0 : nullptr);
        if (st != PA_OK) return st;
    }
    for (const DecodePlan& plan : plans) {
        const pa_status st = launch_planned(plan, stream);
        if (st != PA_OK) return st;
    }
    return ok();
}

}  // namespace

extern "C" {

pa_status pa_decode_fp8_ex(void* out, const void* query, int64_t q_token_stride, const void* key_cache,
                           const void* value_cache, const int32_t* block_table, int32_t max_blocks_per_req,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                           pa_fp8_format format, float k_scale, float v_scale, int32_t max_seq_len, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    return decode_fp8_common(out, query, q_token_stride, nullptr, 0, nullptr, 0, key_cache, value_cache, nullptr,
                             block_table, max_blocks_per_req, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, scale, format, k_scale, v_scale, max_seq_len, workspace,
                             workspace_bytes, false, stream);
}

pa_status pa_decode_append_fp8(void* out, const void* query, int64_t q_token_stride, const void* key,
                               int64_t key_token_stride, const void* value, int64_t value_token_stride,
                               void* key_cache, void* value_cache, int64_t* slot_mapping, const int32_t* block_table,
                               int32_t max_blocks_per_req, const int32_t* seq_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, float scale, pa_fp8_format format, float k_scale, float v_scale,
                               int32_t max_seq_len, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_fp8_common(out, query, q_token_stride, key, key_token_stride, value, value_token_stride, key_cache,
                             value_cache, slot_mapping, block_table, max_blocks_per_req, seq_lens, num_seqs,
                             num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, format, k_scale,
                             v_scale, max_seq_len, workspace, workspace_bytes, true, stream);
}

pa_status pa_decode_fp8(void* out, const void* query, int64_t q_token_stride, const void* key_cache,
                        const void* value_cache, const int32_t* block_table, int32_t max_blocks_per_req,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale, float k_scale,
                        float v_scale, int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    return pa_decode_fp8_ex(out, query, q_token_stride, key_cache, value_cache, block_table, max_blocks_per_req,
                            seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                            PA_FP8_E4M3, k_scale, v_scale, max_seq_len, workspace, workspace_bytes, stream);
}

pa_status pa_decode(void* out, const void* query, int64_t q_token_stride, const void* key_cache,
                    const void* value_cache, const int32_t* block_table, int32_t max_blocks_per_req,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                    int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                    size_t workspace_bytes, pa_dtype dtype, hipStream_t stream) {
    if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
    const pa_status hs = check_heads(num_heads, num_kv_heads, head_dim, block_size);
    if (hs != PA_OK) return hs;
    if (num_seqs < 0 || num_blocks < 0 || max_seq_len < 0 || max_blocks_per_req < 0)
        return fail(PA_ERR_INVALID_ARG, "negative size");
    if (partition_tokens < -1 || (partition_tokens > 0 && partition_tokens % 16))
        return fail(PA_ERR_INVALID_ARG, "partition_tokens %d (0, -1 or a positive multiple of 16)",
                    partition_tokens);
    if (!(isfinite(scale) && scale > 0.f)) return fail(PA_ERR_INVALID_ARG, "scale must be finite and positive");
    if ((int64_t)max_seq_len > (int64_t)max_blocks_per_req * 16)
        return fail(PA_ERR_INVALID_ARG, "max_seq_len %d exceeds max_blocks_per_req * 16", max_seq_len);
    if (num_seqs == 0) return ok();
    if (num_blocks == 0 && max_seq_len > 0) return fail(PA_ERR_INVALID_ARG, "empty cache pool");
    if (!out || !query || !seq_lens || !key_cache || !value_cache || (max_seq_len > 0 && !block_table))
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    const int64_t eb = elem_bytes(dtype);
    if (q_token_stride < (int64_t)num_heads * head_dim)
        return fail(PA_ERR_INVALID_ARG, "q_token_stride smaller than num_heads * head_dim");
    if (!aligned16(query) || (q_token_stride * eb) % 16 || !aligned16(out) || !aligned16(key_cache) ||
        !aligned16(value_cache))
        return fail(PA_ERR_INVALID_ARG, "query/out/cache rows must start on 16-byte boundaries");
    if (pa::debug_checks_enabled(stream)) {
        const pa_status dc = pa::debug_check_tables(block_table, max_blocks_per_req, seq_lens, num_seqs, num_blocks,
                                                    max_seq_len, stream);
        if (dc != PA_OK) return dc;
    }
    return decode_common(out, query, q_token_stride, key_cache, value_cache, block_table, max_blocks_per_req,
                         seq_lens, nullptr, num_seqs, num_heads, num_kv_heads, num_blocks, scale, max_seq_len,
                         partition_tokens, workspace, workspace_bytes, dtype == PA_BF16 ? 1 : 0, 1.f, 1.f, stream);
}

pa_status pa_decode_append(void* out, const void* query, int64_t q_token_stride, const void* key,
                           int64_t key_token_stride, const void* value, int64_t value_token_stride, void* key_cache,
                           void* value_cache, int64_t* slot_mapping, const int32_t* block_table,
                           int32_t max_blocks_per_req, const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           float scale, int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                           pa_dtype dtype, hipStream_t stream) {
    if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
    const pa_status hs = check_heads(num_heads, num_kv_heads, head_dim, block_size);
    if (hs != PA_OK) return hs;
    if (num_seqs < 0 || num_blocks < 0 || max_seq_len < 0 || max_blocks_per_req < 0)
        return fail(PA_ERR_INVALID_ARG, "negative size");
    if (!(isfinite(scale) && scale > 0.f)) return fail(PA_ERR_INVALID_ARG, "scale must be finite and positive");
    if ((int64_t)max_seq_len > (int64_t)max_blocks_per_req * 16)
        return fail(PA_ERR_INVALID_ARG, "max_seq_len %d exceeds max_blocks_per_req * 16", max_seq_len);
    if (num_seqs == 0) return ok();
    if (num_blocks == 0 && max_seq_len > 0) return fail(PA_ERR_INVALID_ARG, "empty cache pool");
    if (!out || !query || !seq_lens || !key || !value || !key_cache || !value_cache ||
        (max_seq_len > 0 && !block_table))
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    const int64_t eb = elem_bytes(dtype);
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    if (q_token_stride < (int64_t)num_heads * head_dim)
        return fail(PA_ERR_INVALID_ARG, "q_token_stride smaller than num_heads * head_dim");
    if (key_token_stride < row_elems || value_token_stride < row_elems)
        return fail(PA_ERR_INVALID_ARG, "key/value token stride smaller than num_kv_heads * head_dim");
    if (!aligned16(query) || (q_token_stride * eb) % 16 || !aligned16(out) || !aligned16(key_cache) ||
        !aligned16(value_cache) || !aligned16(key) || !aligned16(value) || (key_token_stride * eb) % 16 ||
        (value_token_stride * eb) % 16)
        return fail(PA_ERR_INVALID_ARG, "query/out/key/value/cache rows must start on 16-byte boundaries");
    if (pa::debug_checks_enabled(stream)) {
        const pa_status dc = pa::debug_check_tables(block_table, max_blocks_per_req, seq_lens, num_seqs, num_blocks,
                                                    max_seq_len, stream, true);
        if (dc != PA_OK) return dc;
    }
    if (dtype == PA_BF16 && use_stream(num_seqs, 0))
        return decode_common(out, query, q_token_stride, key_cache, value_cache, block_table, max_blocks_per_req,
                             seq_lens, nullptr, num_seqs, num_heads, num_kv_heads, num_blocks, scale, max_seq_len, 0,
                             workspace, workspace_bytes, 3, 1.f, 1.f, stream, key, key_token_stride * eb, value,
                             value_token_stride * eb, slot_mapping);
    // fp32, or more sequences than the stream mode takes: the newest rows are
    // scattered first (token b of sequence b at position seq_lens[b] - 1), then
    // the plain decode reads them from the cache.  The decode is planned (grid,
    // workspace) before the scatter is enqueued, so a failed check writes
    // nothing.
    DecodePlan plan;
    pa_status st = plan_decode(plan, out, query, q_token_stride, key_cache, value_cache, block_table,
                               max_blocks_per_req, seq_lens, nullptr, num_seqs, num_heads, num_kv_heads, num_blocks,
                               scale, max_seq_len, 0, workspace, workspace_bytes, dtype == PA_BF16 ? 1 : 0, 1.f, 1.f);
    if (st != PA_OK) return st;
    st = hip_status(
        pa::launch_slot_and_cache(slot_mapping, block_table, max_blocks_per_req, num_seqs, nullptr, seq_lens, key,
                                  key_token_stride * eb, value, value_token_stride * eb, key_cache, value_cache,
                                  num_seqs, num_blocks * 16, (int32_t)(row_elems * eb), stream),
        "slot_and_cache launch");
    if (st != PA_OK) return st;
    return launch_planned(plan, stream);
}

size_t pa_chunked_prefill_workspace_bytes(int32_t num_seqs, int64_t num_q_tokens, int32_t max_query_len,
                                          int32_t max_seq_len, int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim) {
    return pa_chunked_prefill_workspace_bytes_ex(num_seqs, num_q_tokens, max_query_len, max_seq_len, num_heads,
                                                 num_kv_heads, head_dim, PA_BF16);
}

size_t pa_chunked_prefill_workspace_bytes_ex(int32_t num_seqs, int64_t num_q_tokens, int32_t max_query_len,
                                             int32_t max_seq_len, int32_t num_heads, int32_t num_kv_heads,
                                             int32_t head_dim, pa_dtype dtype) {
    if (num_seqs <= 0 || num_q_tokens <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads)
        return 0;
    if (dtype == PA_F32) {
        if (num_q_tokens > 0x7fffffff || max_seq_len < 0) return 0;
        const F32Rows fr = f32_rows(num_q_tokens, max_seq_len);
        return fr.table_off + fr.table_bytes +
               align256(pa_decode_workspace_bytes((int32_t)num_q_tokens, num_heads, num_kv_heads, head_dim,
                                                  max_seq_len, 0));
    }
    const size_t dec = align256(pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len, 0));
    if (max_query_len < 2) return dec;
    const PrefillShape ps = prefill_shape(num_seqs, num_q_tokens, max_query_len, num_heads, num_kv_heads);
    return dec + prefill_part_bytes(ps, num_kv_heads);
}

pa_status pa_chunked_prefill(void* out, const void* query, int64_t q_token_stride, const void* key_cache,
                             const void* value_cache, const int32_t* block_table, int32_t max_blocks_per_req,
                             const int32_t* cu_query_lens, const int32_t* seq_lens, int32_t num_seqs,
                             int64_t num_q_tokens, int32_t max_query_len, int32_t max_seq_len,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int64_t num_blocks, float scale, int32_t causal, void* workspace,
                             size_t workspace_bytes, pa_dtype dtype, hipStream_t stream) {
    if (dtype != PA_BF16 && dtype != PA_F32) return fail(PA_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
    const pa_status hs = check_heads(num_heads, num_kv_heads, head_dim, block_size);
    if (hs != PA_OK) return hs;
    if (num_seqs < 0 || num_q_tokens < 0 || num_blocks < 0 || max_seq_len < 0 || max_query_len < 0 ||
        max_blocks_per_req < 0)
        return fail(PA_ERR_INVALID_ARG, "negative size");
    if (causal != 0 && causal != 1) return fail(PA_ERR_INVALID_ARG, "causal %d (0 or 1)", causal);
    if (num_kv_heads > 255) return fail(PA_ERR_UNSUPPORTED, "num_kv_heads %d (at most 255)", num_kv_heads);
    if (!(isfinite(scale) && scale > 0.f)) return fail(PA_ERR_INVALID_ARG, "scale must be finite and positive");
    if ((int64_t)max_seq_len > (int64_t)max_blocks_per_req * 16)
        return fail(PA_ERR_INVALID_ARG, "max_seq_len %d exceeds max_blocks_per_req * 16", max_seq_len);
    if (num_seqs == 0 || num_q_tokens == 0) return ok();
    if (num_q_tokens > 0x7fffffff) return fail(PA_ERR_INVALID_ARG, "num_q_tokens too large");
    if (num_blocks == 0 && max_seq_len > 0) return fail(PA_ERR_INVALID_ARG, "empty cache pool");
    if (!out || !query || !seq_lens || !cu_query_lens || !key_cache || !value_cache ||
        (max_seq_len > 0 && !block_table))
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (q_token_stride < (int64_t)num_heads * head_dim)
        return fail(PA_ERR_INVALID_ARG, "q_token_stride smaller than num_heads * head_dim");
    if (!aligned16(query) || (q_token_stride * elem_bytes(dtype)) % 16 || !aligned16(out) || !aligned16(key_cache) ||
        !aligned16(value_cache))
        return fail(PA_ERR_INVALID_ARG, "query/out/cache rows must start on 16-byte boundaries");

    if (pa::debug_checks_enabled(stream)) {
        pa_status dc = pa::debug_check_query_lens(cu_query_lens, seq_lens, num_seqs, num_q_tokens, max_query_len, stream);
        if (dc == PA_OK)
            dc = pa::debug_check_tables(block_table, max_blocks_per_req, seq_lens, num_seqs, num_blocks, max_seq_len,
                                        stream);
        if (dc != PA_OK) return dc;
    }

    if (dtype == PA_F32) {
        // fp32: every query row as a decode row of its own -- its key count
        // under the mask and its request's table row, expanded into the
        // workspace -- read by the fp32 decode.  Planned before either launch.
        const F32Rows fr = f32_rows(num_q_tokens, max_seq_len);
        if (!workspace || workspace_bytes < fr.table_off + fr.table_bytes)
            return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace ? workspace_bytes : 0,
                        pa_chunked_prefill_workspace_bytes_ex(num_seqs, num_q_tokens, max_query_len, max_seq_len,
                                                              num_heads, num_kv_heads, head_dim, dtype));
        if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
        char* w = static_cast<char*>(workspace);
        int32_t* row_lens = reinterpret_cast<int32_t*>(w);
        int32_t* row_table = reinterpret_cast<int32_t*>(w + fr.table_off);
        const size_t dec_off = fr.table_off + fr.table_bytes;
        DecodePlan plan;
        const pa_status st = plan_decode(plan, out, query, q_token_stride, key_cache, value_cache, row_table,
                                         fr.row_stride, row_lens, nullptr, (int32_t)num_q_tokens, num_heads,
                                         num_kv_heads, num_blocks, scale, max_seq_len, 0, w + dec_off,
                                         workspace_bytes - dec_off, 0, 1.f, 1.f);
        if (st != PA_OK) return st;
        const pa_status ex = hip_status(pa::launch_expand_rows(cu_query_lens, seq_lens, block_table, max_blocks_per_req,
                                                               num_seqs, num_q_tokens, causal, row_lens, row_table,
                                                               fr.row_stride, stream),
                                        "expand_rows launch");
        if (ex != PA_OK) return ex;
        return launch_planned(plan, stream);
    }

    // workspace: the decode part's, then the prefill partial records and merge list
    const size_t dec_bytes =
        align256(pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len, 0));
    PrefillShape ps{};
    size_t need = dec_bytes;
    if (max_query_len >= 2) {
        ps = prefill_shape(num_seqs, num_q_tokens, max_query_len, num_heads, num_kv_heads);
        if (ps.slots_per_kvh <= 0) return fail(PA_ERR_HIP, "cannot size the prefill grid for the current device");
        // units per KV head stay below 2^30: at most tiles x (key tiles + 1)
        if (ps.tiles * ((int64_t)max_seq_len / 64 + 2) >= (int64_t)1 << 30)
            return fail(PA_ERR_INVALID_ARG, "too many query tiles x key tiles");
        need += prefill_part_bytes(ps, num_kv_heads);
    }
    if (!workspace || workspace_bytes < need)
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace ? workspace_bytes : 0, need);
    if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "workspace not 16-byte aligned");

    // single-row sequences: the decode kernel, reading its rows through cu_query_lens
    pa_status st = decode_common(out, query, q_token_stride, key_cache, value_cache, block_table,
                                 max_blocks_per_req, seq_lens, cu_query_lens, num_seqs, num_heads, num_kv_heads,
                                 num_blocks, scale, max_seq_len, 0, workspace, dec_bytes, dtype == PA_BF16 ? 1 : 0,
                                 1.f, 1.f, stream);
    if (st != PA_OK) return st;
    if (max_query_len < 2) return ok();

    // requests of two or more rows: the MFMA prefill kernel, each resident
    // workgroup taking an equal share of a KV head's (query tile, key tile)
    // units, then the merge of the tiles cut by a share boundary
    const int32_t group = num_heads / num_kv_heads;
    pa::PrefillArgs p{};
    p.out = out;
    p.query = query;
    p.q_stride = q_token_stride;
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.block_table = block_table;
    p.bt_stride = max_blocks_per_req;
    p.num_blocks = num_blocks;
    p.cu_query_lens = cu_query_lens;
    p.seq_lens = seq_lens;
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);
    p.causal = causal;
    p.slots_per_kvh = ps.slots_per_kvh;
    p.min_share = kPrefillMinShare;
    p.part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + dec_bytes);
    char* list = reinterpret_cast<char*>(workspace) + dec_bytes + prefill_records_bytes(ps, num_kv_heads);
    p.split_count = reinterpret_cast<int32_t*>(list);
    p.split_list = reinterpret_cast<int4*>(list + 16);
    return hip_status(pa::launch_prefill(p, group, stream), "prefill launch");
}

pa_status pa_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups,
                               hipStream_t stream) {
    if (bytes < 0 || bytes % 16 || workgroups < 0) return fail(PA_ERR_INVALID_ARG, "bytes %lld", (long long)bytes);
    if (bytes == 0) return ok();
    if (!src || !sink || !aligned16(src)) return fail(PA_ERR_INVALID_ARG, "null or misaligned pointer");
    return hip_status(pa::launch_stream_read(src, bytes, sink, workgroups, stream), "stream_read launch");
}

pa_status pa_probe_copy(void* dst, const void* src, int64_t bytes, int32_t workgroups, hipStream_t stream) {
    if (bytes < 0 || bytes % 16 || workgroups < 0) return fail(PA_ERR_INVALID_ARG, "bytes %lld", (long long)bytes);
    if (bytes == 0) return ok();
    if (!src || !dst || !aligned16(src) || !aligned16(dst))
        return fail(PA_ERR_INVALID_ARG, "null or misaligned pointer");
    return hip_status(pa::launch_stream_copy(dst, src, bytes, workgroups, stream), "stream_copy launch");
}

pa_status pa_probe_mfma(uint32_t* sink, int32_t workgroups, int32_t iters, hipStream_t stream) {
    if (workgroups <= 0 || iters < 0) return fail(PA_ERR_INVALID_ARG, "workgroups %d iters %d", workgroups, iters);
    if (!sink) return fail(PA_ERR_INVALID_ARG, "null sink");
    return hip_status(pa::launch_mfma_probe(sink, workgroups, iters, stream), "mfma probe launch");
}

}  // extern "C"
