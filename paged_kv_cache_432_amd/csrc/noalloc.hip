// Allocation-free form of pa_decode_append: the decode's workspace (the block
// prefix and the partial records of split sequences) lives in a file-scope
// device array of the library instead of a caller buffer, so the call
// allocates nothing and takes no workspace argument.  Declared in
// include/pa.h.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "host_status.h"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;

// One copy per device, at its own address; held until the process ends.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (the array's name in host code is only a stand-in for the symbol).
pa_status scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return pa::report(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return pa::report(PA_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return pa::report(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                              hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_append_noalloc(void* out, const void* query, int64_t q_token_stride, const void* key,
                                   int64_t key_token_stride, const void* value, int64_t value_token_stride,
                                   void* key_cache, void* value_cache, int64_t* slot_mapping,
                                   const int32_t* block_table, int32_t max_blocks_per_req, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int64_t num_blocks, float scale, int32_t max_seq_len,
                                   pa_dtype dtype, hipStream_t stream) {
    void* ws = nullptr;
    const pa_status s = scratch_of_current_device(&ws);
    if (s != PA_OK) return s;
    // pa_decode_append runs every check (the workspace size included) before
    // its first launch; the scratch array stands in for the workspace.
    const pa_status st = pa_decode_append(out, query, q_token_stride, key, key_token_stride, value,
                                          value_token_stride, key_cache, value_cache, slot_mapping, block_table,
                                          max_blocks_per_req, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                          block_size, num_blocks, scale, max_seq_len, ws, kScratchBytes, dtype,
                                          stream);
    if (st == PA_ERR_WORKSPACE)
        return pa::report(PA_ERR_WORKSPACE,
                          "pa_decode_append_noalloc: the call needs more scratch than the %zu bytes the library "
                          "holds per device (use pa_decode_append with a workspace of "
                          "pa_decode_workspace_bytes(...) bytes)",
                          kScratchBytes);
    return st;
}

}  // extern "C"
