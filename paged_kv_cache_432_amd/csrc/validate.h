// PA_DEBUG=1 checks of the device-array contract on host copies (validate.cpp),
// called by the entry points before they launch anything.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// PA_DEBUG is set (and not "0") and `stream` is not recording a graph.
bool debug_checks_enabled(hipStream_t stream);

// Block tables and lengths (pa_validate_block_tables on host copies).  With
// `append`, the newest token of each sequence (position seq_lens[b] - 1) may
// lack a block: only the blocks of the tokens before it are checked.
pa_status debug_check_tables(const int32_t* block_table, int32_t max_blocks_per_req, const int32_t* seq_lens,
                             int32_t num_seqs, int64_t num_blocks, int32_t max_seq_len, hipStream_t stream,
                             bool append = false);
pa_status debug_check_query_lens(const int32_t* cu_query_lens, const int32_t* seq_lens, int32_t num_seqs,
                                 int64_t num_q_tokens, int32_t max_query_len, hipStream_t stream);
pa_status debug_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks, hipStream_t stream);

}  // namespace pa
