// Host-side checks of the device-array contract of include/pa.h: the contents
// of block tables, lengths, query offsets and slot mappings, which the launch
// path cannot check without a host synchronisation.  The pa_validate_* calls
// take host copies; with PA_DEBUG=1 in the environment the attention and
// scatter entry points copy their arrays to the host (synchronising the
// stream) and run the same checks before launching anything.
#include <hip/hip_runtime.h>
#include <stdlib.h>
#include <string.h>

#include <unordered_set>
#include <vector>

#include "host_status.h"
#include "pa.h"
#include "validate.h"

namespace {

bool overflow_blocks(int32_t len, int32_t block_size, int32_t max_blocks) {
    return ((int64_t)len + block_size - 1) / block_size > max_blocks;
}

}  // namespace

extern "C" {

pa_status pa_validate_block_tables(const int32_t* block_table, int32_t max_blocks_per_req, const int32_t* seq_lens,
                                   int32_t num_seqs, int64_t num_blocks, int32_t block_size, int32_t max_seq_len) {
    if (num_seqs < 0 || max_blocks_per_req < 0 || num_blocks < 0 || block_size <= 0 || max_seq_len < 0)
        return pa::report(PA_ERR_INVALID_ARG, "negative size");
    if (num_seqs == 0) return pa::report_ok();
    if (!seq_lens || (max_blocks_per_req > 0 && !block_table)) return pa::report(PA_ERR_INVALID_ARG, "null pointer");
    if ((int64_t)max_seq_len > (int64_t)max_blocks_per_req * block_size)
        return pa::report(PA_ERR_INVALID_ARG, "max_seq_len %d exceeds max_blocks_per_req * block_size", max_seq_len);
    for (int32_t b = 0; b < num_seqs; ++b) {
        const int32_t L = seq_lens[b];
        if (L < 0 || L > max_seq_len)
            return pa::report(PA_ERR_INVALID_ARG, "seq_lens[%d] = %d outside [0, max_seq_len = %d]", b, L, max_seq_len);
        if (overflow_blocks(L, block_size, max_blocks_per_req))
            return pa::report(PA_ERR_INVALID_ARG, "seq_lens[%d] = %d needs more than %d blocks", b, L,
                              max_blocks_per_req);
        const int32_t nblk = (int32_t)(((int64_t)L + block_size - 1) / block_size);
        const int32_t* row = block_table + (int64_t)b * max_blocks_per_req;
        for (int32_t i = 0; i < nblk; ++i)
            if (row[i] < 0 || (int64_t)row[i] >= num_blocks)
                return pa::report(PA_ERR_INVALID_ARG, "block_table[%d][%d] = %d outside the pool of %lld blocks", b, i,
                                  row[i], (long long)num_blocks);
    }
    return pa::report_ok();
}

pa_status pa_validate_slot_mapping(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                                   int32_t block_size) {
    if (num_tokens < 0 || num_blocks < 0 || block_size <= 0) return pa::report(PA_ERR_INVALID_ARG, "negative size");
    if (num_tokens == 0) return pa::report_ok();
    if (!slot_mapping) return pa::report(PA_ERR_INVALID_ARG, "null pointer");
    std::unordered_set<int64_t> seen;
    seen.reserve((size_t)num_tokens * 2);
    const int64_t pool = num_blocks * block_size;
    for (int64_t i = 0; i < num_tokens; ++i) {
        const int64_t s = slot_mapping[i];
        if (s < 0 || s >= pool) continue;               // skipped by the scatter
        if (!seen.insert(s).second)
            return pa::report(PA_ERR_INVALID_ARG, "slot_mapping[%lld] = %lld is written by an earlier token too",
                              (long long)i, (long long)s);
    }
    return pa::report_ok();
}

pa_status pa_validate_query_lens(const int32_t* cu_query_lens, const int32_t* seq_lens, int32_t num_seqs,
                                 int64_t num_q_tokens, int32_t max_query_len) {
    if (num_seqs < 0 || num_q_tokens < 0 || max_query_len < 0) return pa::report(PA_ERR_INVALID_ARG, "negative size");
    if (!cu_query_lens || (num_seqs > 0 && !seq_lens)) return pa::report(PA_ERR_INVALID_ARG, "null pointer");
    if (cu_query_lens[0] != 0) return pa::report(PA_ERR_INVALID_ARG, "cu_query_lens[0] = %d, not 0", cu_query_lens[0]);
    for (int32_t b = 0; b < num_seqs; ++b) {
        const int32_t q = cu_query_lens[b + 1] - cu_query_lens[b];
        if (q < 0) return pa::report(PA_ERR_INVALID_ARG, "cu_query_lens decreases at %d", b + 1);
        if (q > max_query_len)
            return pa::report(PA_ERR_INVALID_ARG, "request %d has %d query rows, more than max_query_len %d", b, q,
                              max_query_len);
        if (q > seq_lens[b])
            return pa::report(PA_ERR_INVALID_ARG, "request %d has %d query rows but seq_lens %d", b, q, seq_lens[b]);
    }
    if ((int64_t)cu_query_lens[num_seqs] != num_q_tokens)
        return pa::report(PA_ERR_INVALID_ARG, "cu_query_lens[%d] = %d, not num_q_tokens %lld", num_seqs,
                          cu_query_lens[num_seqs], (long long)num_q_tokens);
    return pa::report_ok();
}

}  // extern "C"

namespace pa {

bool debug_checks_enabled(hipStream_t stream) {
    const char* v = getenv("PA_DEBUG");
    if (!v || !*v || strcmp(v, "0") == 0) return false;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess || st != hipStreamCaptureStatusNone)
        return false;                                   // no host copies while a graph is being recorded
    return true;
}

namespace {

template <typename T>
pa_status to_host(std::vector<T>& dst, const T* src, int64_t n, hipStream_t stream) {
    dst.resize((size_t)(n > 0 ? n : 0));
    if (n <= 0) return PA_OK;
    hipError_t e = hipMemcpyAsync(dst.data(), src, (size_t)n * sizeof(T), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return report(PA_ERR_HIP, "PA_DEBUG copy to host: %s", hipGetErrorString(e));
    return PA_OK;
}

}  // namespace

pa_status debug_check_tables(const int32_t* block_table, int32_t max_blocks_per_req, const int32_t* seq_lens,
                             int32_t num_seqs, int64_t num_blocks, int32_t max_seq_len, hipStream_t stream,
                             bool append) {
    std::vector<int32_t> bt, sl;
    pa_status s = to_host(sl, seq_lens, num_seqs, stream);
    if (s == PA_OK) s = to_host(bt, block_table, (int64_t)num_seqs * max_blocks_per_req, stream);
    if (s != PA_OK) return s;
    if (append) {
        for (int32_t b = 0; b < num_seqs; ++b) {
            if (sl[b] < 0 || sl[b] > max_seq_len)
                return report(PA_ERR_INVALID_ARG, "seq_lens[%d] = %d outside [0, max_seq_len = %d]", b, sl[b],
                              max_seq_len);
            sl[b] = sl[b] > 0 ? sl[b] - 1 : 0;          // the newest token needs no block
        }
    }
    return pa_validate_block_tables(bt.data(), max_blocks_per_req, sl.data(), num_seqs, num_blocks, 16, max_seq_len);
}

pa_status debug_check_query_lens(const int32_t* cu_query_lens, const int32_t* seq_lens, int32_t num_seqs,
                                 int64_t num_q_tokens, int32_t max_query_len, hipStream_t stream) {
    std::vector<int32_t> cu, sl;
    pa_status s = to_host(cu, cu_query_lens, (int64_t)num_seqs + 1, stream);
    if (s == PA_OK) s = to_host(sl, seq_lens, num_seqs, stream);
    if (s != PA_OK) return s;
    return pa_validate_query_lens(cu.data(), sl.data(), num_seqs, num_q_tokens, max_query_len);
}

pa_status debug_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks, hipStream_t stream) {
    std::vector<int64_t> sm;
    const pa_status s = to_host(sm, slot_mapping, num_tokens, stream);
    if (s != PA_OK) return s;
    return pa_validate_slot_mapping(sm.data(), num_tokens, num_blocks, 16);
}

}  // namespace pa
