/*
 * pa.h -- C ABI of libpa.so: paged KV-cache attention for AMD Instinct MI355X
 * (gfx950).
 *
 * The operations and the tensor layouts follow the Tencent engineering article
 * "AI Infra入门干货总结：大模型是如何高效推理的":
 *   - section "Paged Attention": the per-layer caches
 *     key_cache / value_cache [num_blocks, block_size, num_kv_heads, head_dim],
 *     block_table [max_num_reqs, max_num_blocks_per_req] of physical block ids,
 *     slot_mapping [num_tokens] of int64 slots, slot = block * block_size + offset,
 *     and the default block_size of 16;
 *   - section "Reshape & Cache": new K and V rows are column slices of the fused
 *     QKV output, reshaped to [num_tokens, num_kv_heads, head_dim] and scattered
 *     into the cache by slot_mapping before attention reads them;
 *   - section "Attention (FlashAttention, Scaled Dot-Product Attention)":
 *     softmax(Q K^T / sqrt(d_k) + M) V with kv_head = q_head / (num_heads /
 *     num_kv_heads), Q [query_lens, num_heads, head_dim], K/V gathered through
 *     block_table, seq_lens counting every KV token including this step's, the
 *     online softmax that fuses the steps into one kernel, and Flash-Decoding's
 *     split of the KV axis merged with log-sum-exp (its closing summary).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates device memory and keeps no pointer after a call returns;
 *     buffers must stay alive until the work enqueued on `stream` completes.
 *   - All work is enqueued on `stream` (0 = the default stream) without host
 *     synchronisation.  Calls are ordered by the stream: a scatter must be
 *     enqueued before the attention call that reads the tokens it writes.
 *   - Host-side argument checks run before any launch; a failed check launches
 *     nothing and returns a status; pa_last_error_message() gives the detail.
 *   - The contents of device arrays are the caller's contract and are not
 *     checked (that would need a host sync): block ids in [0, num_blocks) for
 *     every block a sequence uses, seq_lens[b] <= max_seq_len <=
 *     max_blocks_per_req * block_size, distinct non-negative slots in one
 *     scatter.  Kernels still never touch memory outside the arrays they are
 *     given for out-of-range positions, request indices or slots; they skip
 *     such tokens instead.
 *   - Supported now: block_size 16, head_dim 128, num_heads / num_kv_heads in
 *     {1, 2, 4, 8}, dtype PA_F32 or PA_BF16 (Q, K, V, caches and outputs all of
 *     that dtype; arithmetic in fp32).  Other values return PA_ERR_UNSUPPORTED.
 *   - The softmax scale of every attention call (pa_decode, pa_decode_append,
 *     pa_decode_fp8, pa_chunked_prefill) must be finite and > 0 (the pages'
 *     1 / sqrt(d_k)); anything else returns PA_ERR_INVALID_ARG.  The kernels
 *     take the running maximum of the raw scores as the softmax reference,
 *     which is the maximum of the scaled scores only for a positive scale.
 *   - Functions are thread-safe; the only global state is a per-thread error
 *     message.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, inconsistent shapes, misaligned rows */
    PA_ERR_UNSUPPORTED = 2,   /* a shape or dtype this build does not implement */
    PA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the query function's size */
    PA_ERR_HIP = 4,           /* a kernel launch failed (hipGetLastError) */
    PA_STATUS_RESERVED_MIN_ = -0x7fffffff - 1,   /* range widened to every int, as for pa_dtype */
    PA_STATUS_RESERVED_MAX_ = 0x7fffffff
} pa_status;

/* The two reserved values widen the enumeration's range to every int, so that
 * a caller's out-of-range value is a valid pa_dtype that the checks reject
 * (PA_ERR_UNSUPPORTED) rather than undefined behaviour in the C++ library. */
typedef enum {
    PA_F32 = 0,
    PA_BF16 = 1,
    PA_DTYPE_RESERVED_MIN_ = -0x7fffffff - 1,
    PA_DTYPE_RESERVED_MAX_ = 0x7fffffff
} pa_dtype;

int32_t pa_abi_version(void);
const char *pa_status_string(pa_status status);
/* Detail of the calling thread's last non-OK status (empty string if none). */
const char *pa_last_error_message(void);

/*
 * pa_slot_mapping -- the page-table lookup of section "Paged Attention":
 *   slot_mapping[i] = block_table[token_seq[i], token_pos[i] / block_size] * block_size
 *                     + token_pos[i] % block_size
 * for every token i (worked example on the page: row [5, 8, 12], position 25
 * -> slot 137).
 *
 * slot_mapping  out, int64 [num_tokens]
 * block_table   int32 [num_seqs, max_blocks_per_req], row-major
 * token_seq     int32 [num_tokens]: request index of each token
 * token_pos     int32 [num_tokens]: logical position of each token in its request
 * A token whose request index or position is negative or out of range, or whose
 * table entry is negative, gets slot -1 (the scatter skips it).
 * num_tokens == 0 is a no-op.
 */
pa_status pa_slot_mapping(int64_t *slot_mapping, const int32_t *block_table,
                          int32_t max_blocks_per_req, int32_t num_seqs,
                          const int32_t *token_seq, const int32_t *token_pos,
                          int64_t num_tokens, int32_t block_size, hipStream_t stream);

/*
 * pa_slot_mapping followed by pa_reshape_and_cache, fused into one launch:
 * the slots of the tokens are computed as pa_slot_mapping does and written to
 * slot_mapping (for the scatters of the other layers of the step), and each
 * token's K and V rows are scattered to them as pa_reshape_and_cache does.
 * Arguments as in those two calls; the results are identical to calling them
 * in turn.
 */
pa_status pa_slot_mapping_and_cache(int64_t *slot_mapping, const int32_t *block_table,
                                    int32_t max_blocks_per_req, int32_t num_seqs,
                                    const int32_t *token_seq, const int32_t *token_pos,
                                    const void *key, int64_t key_token_stride,
                                    const void *value, int64_t value_token_stride,
                                    void *key_cache, void *value_cache,
                                    int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                                    int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                    hipStream_t stream);

/*
 * pa_reshape_and_cache -- the scatter of section "Paged Attention" /
 * "Reshape & Cache": for each token i with s = slot_mapping[i] >= 0, copy
 *   key[i, :, :]   -> key_cache[s / block_size, s % block_size, :, :]
 *   value[i, :, :] -> value_cache[s / block_size, s % block_size, :, :]
 * bit for bit.  Slots < 0 (padding) and slots >= num_blocks * block_size are
 * skipped.
 *
 * key, value      [num_tokens, num_kv_heads, head_dim]; token rows are
 *                 key_token_stride / value_token_stride ELEMENTS apart (e.g. the
 *                 K and V column slices of a [num_tokens, 6144] fused QKV
 *                 output); heads and dims are contiguous.  Row starts must be
 *                 16-byte aligned.
 * key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim], contiguous
 */
pa_status pa_reshape_and_cache(const void *key, int64_t key_token_stride,
                               const void *value, int64_t value_token_stride,
                               void *key_cache, void *value_cache,
                               const int64_t *slot_mapping, int64_t num_tokens,
                               int64_t num_blocks, int32_t block_size,
                               int32_t num_kv_heads, int32_t head_dim,
                               pa_dtype dtype, hipStream_t stream);

/*
 * Host-side block manager and step scheduler (the input side of the path; no
 * GPU work, no device memory).  "AI Infra入门干货总结：大模型是如何高效推理的",
 * sections "连续批处理 (Continuous Batching)" and "Paged Attention", and its
 * appendix 4 on preemption; the inference field notes' prefix-caching entry.
 *
 * A request holds its tokens (prompt, then outputs) and the number it has
 * computed; each pa_kvm_schedule call schedules, for every running request in
 * arrival order and then for waiting requests first come first served, the
 * tokens it has not computed yet, within max_num_batched_tokens per step,
 * max_num_seqs running requests and max_model_len tokens per request, and
 * allocates the 16-token blocks they need.  When a running request cannot get
 * its blocks, the newest running request is preempted: all its blocks are
 * freed, its computed count is reset to 0 and it goes to the front of the
 * waiting queue (recomputation).  A waiting request that cannot get its
 * blocks waits; no waiting request is admitted in a step that preempted.
 * With prefix caching, full computed blocks are registered under a hash of
 * their tokens and of the blocks before them; a new request starts from the
 * longest run of its full prompt blocks found there (never covering its last
 * prompt token), sharing those blocks.  pa_kvm_fork makes a request that
 * shares all blocks of a running one; the first step that writes into a
 * shared block gives the writer a fresh block and lists the (old, new) pair
 * in copy_pairs, for pa_copy_blocks before the step's scatter.
 *
 * Use per step: pa_kvm_schedule -> (copy_pairs via pa_copy_blocks,
 * slot_mapping via pa_reshape_and_cache, then attention over block_table,
 * seq_lens, cu_query_lens) -> pa_kvm_commit with one next token per scheduled
 * request (or -1): a request whose computed count reaches its token count
 * appends it.  The step's arrays belong to the manager and stay valid until
 * the next pa_kvm_schedule.  A manager is not thread-safe.
 */
typedef struct pa_kvm pa_kvm;

typedef struct {
    int32_t num_seqs;              /* scheduled requests: the step's batch rows */
    int64_t num_tokens;            /* scheduled tokens, flattened */
    int32_t max_blocks_per_req;    /* block_table row length: the most blocks a scheduled request holds */
    const int64_t *request_ids;    /* [num_seqs] */
    const int32_t *query_lens;     /* [num_seqs] tokens computed this step */
    const int32_t *cu_query_lens;  /* [num_seqs + 1] */
    const int32_t *seq_lens;       /* [num_seqs] tokens attended: computed + this step's */
    const int32_t *block_table;    /* [num_seqs, max_blocks_per_req], -1 past the request's blocks */
    const int32_t *token_ids;      /* [num_tokens] input tokens of the step, row by row */
    const int32_t *positions;      /* [num_tokens] their positions */
    const int64_t *slot_mapping;   /* [num_tokens] their slots */
    const int64_t *copy_pairs;     /* [num_copies, 2] (src, dst) blocks to copy before the scatter */
    int32_t num_copies;
    const int64_t *preempted;      /* [num_preempted] requests preempted this step */
    int32_t num_preempted;
} pa_kvm_step;

pa_kvm *pa_kvm_create(int32_t num_blocks, int32_t max_num_seqs, int32_t max_num_batched_tokens,
                      int32_t max_model_len, int32_t enable_prefix_caching);
void pa_kvm_destroy(pa_kvm *m);
pa_status pa_kvm_add_request(pa_kvm *m, int64_t request_id, const int32_t *prompt, int32_t prompt_len);
pa_status pa_kvm_fork(pa_kvm *m, int64_t parent_id, int64_t child_id);
pa_status pa_kvm_finish(pa_kvm *m, int64_t request_id);
pa_status pa_kvm_schedule(pa_kvm *m, pa_kvm_step *step);
pa_status pa_kvm_commit(pa_kvm *m, const int32_t *next_tokens, int32_t num_seqs);
int32_t pa_kvm_num_free_blocks(const pa_kvm *m);
int32_t pa_kvm_num_cached_blocks(const pa_kvm *m);
int32_t pa_kvm_block_ref(const pa_kvm *m, int32_t block);
pa_status pa_kvm_request_info(const pa_kvm *m, int64_t request_id, int32_t *num_computed,
                              int32_t *num_tokens, int32_t *running, int32_t *blocks,
                              int32_t blocks_cap, int32_t *num_blocks);

/*
 * Copy-on-write of shared blocks.  Sequences that share a prefix point their
 * block tables at the same physical blocks (prefix caching); before one of
 * them writes into a shared block, the caller gives it a fresh block and this
 * call copies the contents ("AI Infra入门干货总结：大模型是如何高效推理的", section
 * "Paged Attention": the [num_layers, 2, num_blocks, block_size, num_kv_heads,
 * head_dim] cache; the inference field notes' chapter on batching and memory
 * management names copy-on-write and prefix caching).
 *
 * For each pair p of block_mapping (int64 [num_pairs][2] = (src, dst), device
 * memory): block dst of every layer's K and V cache becomes a byte copy of
 * block src.  Layer l's K cache starts layer_stride_bytes * l after
 * key_cache, its V cache as far after value_cache (for the pages' unified
 * tensor kv: key_cache = kv[0, 0], value_cache = kv[0, 1], layer_stride_bytes
 * = 2 * num_blocks * block_bytes).  block_bytes = block_size * num_kv_heads *
 * head_dim * element size (any dtype, fp8 included), a multiple of 16.
 * Pairs with an id outside [0, num_blocks) are skipped.  Pairs run
 * concurrently: no dst may appear as the src or dst of another pair in the
 * same call.  One launch; num_pairs = 0 is a no-op.
 */
pa_status pa_copy_blocks(void *key_cache, void *value_cache, int64_t layer_stride_bytes,
                         int32_t num_layers, int64_t num_blocks, int64_t block_bytes,
                         const int64_t *block_mapping, int64_t num_pairs, hipStream_t stream);

/*
 * fp8 KV cache: the scatter.  ("AI Infra入门干货总结：大模型是如何高效推理的" and the
 * inference field notes gathered with it name quantising the KV cache as the
 * way to move fewer bytes per decoded token, e4m3 and e5m2 both in use; the
 * format is its published definition, OCP 8-bit floating point E4M3: bias 7,
 * 3 mantissa bits, subnormals m * 2^-9, S.1111.111 NaN, largest 448.)
 *
 * As pa_reshape_and_cache, but the caches hold one byte per element: element
 * x of a token's K row is stored as E4M3(x / k_scale), V as E4M3(x / v_scale),
 * where the division is float32 (correctly rounded), magnitudes beyond 448
 * saturate to 448, NaN stays NaN, and the code is the nearest one, ties to the
 * even mantissa.  A stored code c then stands for value(c) * scale.
 *
 * key, value      [num_tokens, num_kv_heads, head_dim] in `dtype` (PA_BF16 or
 *                 PA_F32), token rows *_token_stride ELEMENTS apart, 16-byte
 *                 aligned.
 * key_cache, value_cache  uint8 [num_blocks, block_size, num_kv_heads, head_dim].
 * k_scale, v_scale  finite, > 0: one scale per cache (per layer), chosen by
 *                 the caller (e.g. the largest |x| expected over 448).
 * num_kv_heads * head_dim must be a multiple of 16.  Slots < 0 or past the
 * pool are skipped.  num_tokens = 0 is a no-op.
 */
pa_status pa_reshape_and_cache_fp8(const void *key, int64_t key_token_stride,
                                   const void *value, int64_t value_token_stride,
                                   void *key_cache, void *value_cache,
                                   const int64_t *slot_mapping, int64_t num_tokens,
                                   int64_t num_blocks, int32_t block_size,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   pa_dtype dtype, float k_scale, float v_scale,
                                   hipStream_t stream);

/*
 * pa_slot_mapping followed by pa_reshape_and_cache_fp8, fused into one launch
 * (as pa_slot_mapping_and_cache is for bf16/fp32 caches): the tokens' slots
 * are computed as pa_slot_mapping does and written to slot_mapping, and each
 * token's K and V rows are quantised into them as pa_reshape_and_cache_fp8
 * does.  Arguments as in those two calls; the results are identical to
 * calling them in turn.
 */
pa_status pa_slot_mapping_and_cache_fp8(int64_t *slot_mapping, const int32_t *block_table,
                                        int32_t max_blocks_per_req, int32_t num_seqs,
                                        const int32_t *token_seq, const int32_t *token_pos,
                                        const void *key, int64_t key_token_stride,
                                        const void *value, int64_t value_token_stride,
                                        void *key_cache, void *value_cache,
                                        int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                                        int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                        float k_scale, float v_scale, hipStream_t stream);

/*
 * fp8 KV cache: decode attention over caches written by
 * pa_reshape_and_cache_fp8.  Same operation and arguments as pa_decode with
 * query and out in bf16, each cached K element standing for value(code) *
 * k_scale and each V element for value(code) * v_scale.  The codes are widened
 * to bf16 exactly; k_scale is folded into the softmax scale and v_scale into
 * the output, so the arithmetic is that of the bf16 path.  It always uses the
 * balanced stream mode (no partition_tokens), which takes up to 4096
 * sequences per launch: a larger batch runs as consecutive launches over
 * groups of 4096 sequences on the same workspace, all checked before the
 * first.  Workspace: pa_decode_workspace_bytes(num_seqs, num_heads,
 * num_kv_heads, head_dim, max_seq_len, 0) bytes, 16-byte aligned.
 */
pa_status pa_decode_fp8(void *out, const void *query, int64_t q_token_stride,
                        const void *key_cache, const void *value_cache,
                        const int32_t *block_table, int32_t max_blocks_per_req,
                        const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int64_t num_blocks, float scale, float k_scale, float v_scale,
                        int32_t max_seq_len, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * The other 8-bit format of the pages' fp8 KV cache.  The three calls above
 * store and read E4M3 codes; each has an _ex form that takes the format:
 *   PA_FP8_E4M3  as above;
 *   PA_FP8_E5M2  OCP E5M2: bias 15, 2 mantissa bits, subnormals m * 2^-16,
 *                infinity at S.11111.00 and NaN at S.11111.{01,10,11}, largest
 *                finite 57344.  The scatter stores E5M2(x / scale) with the
 *                same rules as E4M3 (float32 division, nearest code, ties to
 *                the even mantissa, NaN kept), magnitudes beyond 57344
 *                (infinity included) saturating to 57344, so that stored codes
 *                are finite; the decode widens the codes exactly (every finite
 *                E5M2 value is a bf16 and an fp16 value) and then computes as
 *                pa_decode_fp8 does.
 * A cache must be read in the format it was written in.  Other format values
 * return PA_ERR_UNSUPPORTED.
 */
typedef enum {
    PA_FP8_E4M3 = 0,
    PA_FP8_E5M2 = 1,
    PA_FP8_FORMAT_RESERVED_MIN_ = -0x7fffffff - 1,   /* range widened to every int, as for pa_dtype */
    PA_FP8_FORMAT_RESERVED_MAX_ = 0x7fffffff
} pa_fp8_format;

pa_status pa_reshape_and_cache_fp8_ex(const void *key, int64_t key_token_stride,
                                      const void *value, int64_t value_token_stride,
                                      void *key_cache, void *value_cache,
                                      const int64_t *slot_mapping, int64_t num_tokens,
                                      int64_t num_blocks, int32_t block_size,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      pa_dtype dtype, pa_fp8_format format,
                                      float k_scale, float v_scale, hipStream_t stream);
pa_status pa_slot_mapping_and_cache_fp8_ex(int64_t *slot_mapping, const int32_t *block_table,
                                           int32_t max_blocks_per_req, int32_t num_seqs,
                                           const int32_t *token_seq, const int32_t *token_pos,
                                           const void *key, int64_t key_token_stride,
                                           const void *value, int64_t value_token_stride,
                                           void *key_cache, void *value_cache,
                                           int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                                           int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                           pa_fp8_format format, float k_scale, float v_scale,
                                           hipStream_t stream);
pa_status pa_decode_fp8_ex(void *out, const void *query, int64_t q_token_stride,
                           const void *key_cache, const void *value_cache,
                           const int32_t *block_table, int32_t max_blocks_per_req,
                           const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, float scale, pa_fp8_format format,
                           float k_scale, float v_scale, int32_t max_seq_len,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_append_fp8 -- the decode step over an fp8 cache in one call, as
 * pa_decode_append is for bf16 (the article's sections "Paged Attention" and
 * "Reshape & Cache": this step's K/V rows are written to their slots, then
 * attention reads the cache).  Row b of key / value (bf16, [num_seqs,
 * num_kv_heads, head_dim], the newest token of sequence b, at position
 * seq_lens[b] - 1) is stored as fp8 codes in its slot and attended to with the
 * rest of the sequence.  The results are those of
 *   pa_slot_mapping_and_cache_fp8_ex(slot_mapping, block_table, ...,
 *       token_seq = b, token_pos = seq_lens[b] - 1, key, value, ..., PA_BF16,
 *       format, k_scale, v_scale)
 * followed by pa_decode_fp8_ex(...): slot_mapping, the caches and out bit for
 * bit.  The decode launch stores the codes itself: the workgroup that reads a
 * sequence's last block stores the newest token into it first (no other
 * workgroup reads that block).  Arguments as for
 * pa_decode_append (key_token_stride / value_token_stride in elements; rows
 * 16-byte aligned; slot_mapping may be NULL) and pa_decode_fp8_ex (format,
 * scales, the stream mode in groups of 4096 sequences, the workspace of
 * pa_decode_workspace_bytes(..., 0)).  Every check runs before the first
 * launch: a call that returns an error has written nothing.
 */
pa_status pa_decode_append_fp8(void *out, const void *query, int64_t q_token_stride,
                               const void *key, int64_t key_token_stride,
                               const void *value, int64_t value_token_stride,
                               void *key_cache, void *value_cache, int64_t *slot_mapping,
                               const int32_t *block_table, int32_t max_blocks_per_req,
                               const int32_t *seq_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, float scale,
                               pa_fp8_format format, float k_scale, float v_scale,
                               int32_t max_seq_len, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * The step just before attention, fused into one pass ("AI Infra入门干货总结：
 * 大模型是如何高效推理的", section "Reshape & Cache" and its table, and the RoPE
 * summary near its opening): split each token's fused QKV projection row into
 * its Q | K | V column ranges, turn Q and K by the token's position (RoPE),
 * write Q to query_out and scatter K and V into the paged cache exactly as
 * pa_reshape_and_cache does.
 *
 * The turn: with R = rotary_dim and row = cos_sin_cache[positions[t], :]
 * (cos of the R/2 angles in columns 0 .. R/2-1, their sin in R/2 .. R-1), pair
 * i < R/2 of a head, (x[a], x[b]), becomes (x[a] cos_i - x[b] sin_i,
 * x[b] cos_i + x[a] sin_i), where (a, b) = (i, i + R/2) when neox_style != 0
 * (halves paired) and (2i, 2i + 1) otherwise (neighbours paired).  Dimensions
 * R .. head_dim-1 are copied unchanged.  Arithmetic is fp32 (bf16 inputs are
 * exact in fp32), each output rounded once to the storage dtype (nearest
 * even).  V is copied bit for bit.
 *
 * query_out       [num_tokens, num_heads, head_dim], rows q_out_token_stride
 *                 ELEMENTS apart.  May be qkv itself (same stride): Q is then
 *                 turned in place.  No other overlap with any input is allowed.
 * qkv             [num_tokens, (num_heads + 2 num_kv_heads) * head_dim], rows
 *                 qkv_token_stride ELEMENTS apart (>= that width).
 * positions       int64 [num_tokens]: the token's position in its sequence.  A
 *                 position outside [0, max_position) breaks the caller's
 *                 contract; it is clamped into the table so no read leaves it.
 * cos_sin_cache   float32 [max_position, rotary_dim], contiguous, built once by
 *                 the caller (e.g. theta_i = rope_theta^(-2i/R), row p =
 *                 cos(p theta_i) then sin(p theta_i)).
 * slot_mapping    int64 [num_tokens]; a slot < 0 (padding) or past the pool
 *                 skips that token's K/V scatter; its Q is still written.
 * key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim].
 * rotary_dim      a multiple of 16 in [16, head_dim]; head_dim must be 128,
 *                 block_size 16.
 * All row starts (qkv, query_out, caches, cos_sin_cache) 16-byte aligned.
 * num_tokens = 0 is a no-op.  One launch on `stream`, no allocation.
 */
pa_status pa_rope_reshape_and_cache(void *query_out, int64_t q_out_token_stride,
                                    const void *qkv, int64_t qkv_token_stride,
                                    const int64_t *positions, const float *cos_sin_cache,
                                    int64_t max_position, int32_t rotary_dim, int32_t neox_style,
                                    void *key_cache, void *value_cache,
                                    const int64_t *slot_mapping, int64_t num_tokens,
                                    int64_t num_blocks, int32_t block_size,
                                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                    pa_dtype dtype, hipStream_t stream);

/*
 * Workspace bytes pa_decode needs for these arguments (0 when no sequence is
 * split).  Same partition rule as pa_decode: partition_tokens > 0 is used as
 * given (a multiple of block_size), 0 picks a size from the shapes, -1 never
 * splits.  With partition_tokens 0 the size also covers pa_decode_append and
 * pa_decode_fp8(_ex) (past 4096 sequences: their groups of 4096).
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len,
                                 int32_t partition_tokens);

/* Partition size pa_decode will use for these arguments (tokens per split). */
int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                   int32_t max_seq_len, int32_t partition_tokens);

/*
 * pa_decode -- one query token per sequence (query_lens = 1) attending to all
 * seq_lens[b] tokens of its paged K/V:
 *   out[b, h, :] = sum_t softmax_t(scale * <q[b, h], k_t>) v_t,
 *   k_t, v_t = cache[block_table[b, t / 16], t % 16, h / (num_heads / num_kv_heads), :]
 * computed in one pass with the online softmax (running max and sum, rescaled
 * by exp(m_old - m_new)).  A sequence longer than the partition size is split
 * into partitions whose partial (max, sum, unnormalised output) are merged with
 * log-sum-exp weights in a second kernel.  seq_lens[b] == 0 gives zeros.
 *
 * out          [num_seqs, num_heads, head_dim], contiguous, dtype
 * query        [num_seqs, num_heads, head_dim]; token rows q_token_stride
 *              ELEMENTS apart, heads and dims contiguous, rows 16-byte aligned
 * key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim]
 * block_table  int32 [num_seqs, max_blocks_per_req]
 * seq_lens     int32 [num_seqs], this step's token included
 * max_seq_len  host-side upper bound of seq_lens (sizes the grid)
 * workspace    device scratch of at least pa_decode_workspace_bytes(...) bytes
 *              (may be NULL when that is 0); its contents need no
 *              initialisation and are overwritten.
 */
pa_status pa_decode(void *out, const void *query, int64_t q_token_stride,
                    const void *key_cache, const void *value_cache,
                    const int32_t *block_table, int32_t max_blocks_per_req,
                    const int32_t *seq_lens, int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int64_t num_blocks, float scale,
                    int32_t max_seq_len, int32_t partition_tokens,
                    void *workspace, size_t workspace_bytes,
                    pa_dtype dtype, hipStream_t stream);

/*
 * pa_decode_append -- one decode step of sections "Paged Attention" and
 * "Reshape & Cache" in one call: each sequence's newest token (position
 * seq_lens[b] - 1) is written into the paged cache and then attended to
 * with the rest of the sequence.  The results are those of
 *   pa_slot_mapping_and_cache(slot_mapping, block_table, ..., token_seq = b,
 *                             token_pos = seq_lens[b] - 1, key, value, ...)
 * followed by pa_decode(..., partition_tokens = 0, ...): slot_mapping and the
 * caches bit for bit, out within the rounding of pa_decode (the newest token's
 * term is added in another order).  On bf16 with at most 4096 sequences it is
 * one decode launch (plus the split merge): attention reads the newest token
 * from its input row, and the same launch writes that row to its cache slot,
 * which no workgroup of the launch reads.  Otherwise (fp32, more sequences)
 * the scatter and pa_decode run one after the other.
 *
 * key, value    [num_seqs, num_kv_heads, head_dim]: row b is the newest token
 *               of sequence b; rows key_token_stride / value_token_stride
 *               ELEMENTS apart, 16-byte aligned.  Rows of sequences with
 *               seq_lens[b] <= 0 are not read.
 * slot_mapping  out, int64 [num_seqs] (may be NULL): the newest token's slot,
 *               or -1 where the request has no block for it (then nothing is
 *               written for that token), for the scatters of the other layers.
 * key_cache, value_cache  written at those slots only.
 * Other arguments as for pa_decode; the workspace is
 * pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
 * max_seq_len, 0) bytes.  seq_lens[b] counts the newest token.  Every check
 * (the workspace's size and alignment included) runs before the first launch
 * on both routes: a call that returns an error has written neither the caches
 * nor slot_mapping.
 */
pa_status pa_decode_append(void *out, const void *query, int64_t q_token_stride,
                           const void *key, int64_t key_token_stride,
                           const void *value, int64_t value_token_stride,
                           void *key_cache, void *value_cache, int64_t *slot_mapping,
                           const int32_t *block_table, int32_t max_blocks_per_req,
                           const int32_t *seq_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, float scale,
                           int32_t max_seq_len, void *workspace, size_t workspace_bytes,
                           pa_dtype dtype, hipStream_t stream);

/*
 * pa_decode_append_noalloc -- pa_decode_append for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same operation, arguments and results
 * as pa_decode_append, without the workspace: the decode's scratch (block
 * prefix and partial records) is a file-scope device array of the library,
 * PA_NOALLOC_SCRATCH_BYTES (32 MiB) per device, 256-byte aligned, which each
 * device the library runs on holds from its first call until the process
 * ends.  The call allocates nothing (no hipMalloc or allocating library
 * routine).  A call that needs more scratch than that (pa_decode_workspace_bytes
 * above it: many sequences with explicit partitions, or a very wide stream
 * grid) returns PA_ERR_WORKSPACE and launches nothing.  The scratch needs no
 * initialisation (every byte read is first written by the same call); every
 * call on one device shares that device's array, so calls that overlap on one
 * device (on different streams, or from different threads without ordering)
 * race and give undefined results.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pa_status pa_decode_append_noalloc(void *out, const void *query, int64_t q_token_stride,
                                   const void *key, int64_t key_token_stride,
                                   const void *value, int64_t value_token_stride,
                                   void *key_cache, void *value_cache, int64_t *slot_mapping,
                                   const int32_t *block_table, int32_t max_blocks_per_req,
                                   const int32_t *seq_lens, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int64_t num_blocks, float scale,
                                   int32_t max_seq_len, pa_dtype dtype, hipStream_t stream);

/*
 * pa_chunked_prefill -- attention of a mixed batch in one call: chunks of
 * query_len >= 2 rows (chunked prefill) next to single-row decodes, all
 * reading K/V from the paged cache after this step's rows were scattered
 * (the article's section "Attention (FlashAttention, Scaled Dot-Product
 * Attention)": a varlen call over the flattened batch, cu_seqlens isolating
 * requests, the causal mask M, and v1's rule that prefill too reads the paged
 * cache).  For request b with q_b = cu_query_lens[b+1] - cu_query_lens[b]
 * rows and L_b = seq_lens[b] tokens, query row j (flattened row
 * cu_query_lens[b] + j) sits at position L_b - q_b + j and attends keys
 * 0 .. L_b - q_b + j when causal (all L_b keys otherwise; a row that sees no
 * key outputs zeros):
 *   out[row, h, :] = sum_t softmax_t(scale * <q[row, h], k_t>) v_t,
 *   kv_head = h / (num_heads / num_kv_heads).
 * Requests with q_b == 1 run through the decode kernel (as pa_decode with
 * automatic splitting); requests with q_b >= 2 run on the matrix cores
 * (Q.K^T in bf16 MFMA, P.V in fp16 MFMA with V exact in fp16, fp32
 * accumulation; a workgroup that meets |V| >= 2^16 redoes its work with the
 * probabilities carried as a bf16 hi/lo pair), their (query tile, key tile)
 * work shared by the resident workgroups in equal parts of a cost that also
 * charges each query tile a fixed set-up, and tiles cut by a share
 * boundary merged with log-sum-exp weights; q_b == 0 requests produce
 * nothing.  Over an fp32 cache every query row runs as a decode row of its
 * own: a first kernel writes, into the workspace, each row's key count under
 * the mask (L_b - q_b + j + 1, or L_b) and a copy of its request's
 * block-table row, and the fp32 decode (as pa_decode) reads them, each row
 * re-reading its keys (a path for accuracy, not for speed).
 *
 * out          [num_q_tokens, num_heads, head_dim] of dtype, contiguous
 * query        [num_q_tokens, num_heads, head_dim] of dtype; rows q_token_stride
 *              ELEMENTS apart (heads/dims contiguous, rows 16-byte aligned)
 * key_cache, value_cache, block_table, block_size, num_blocks: as pa_decode
 * cu_query_lens int32 [num_seqs + 1], cu_query_lens[0] == 0,
 *              cu_query_lens[num_seqs] == num_q_tokens, non-decreasing
 * seq_lens     int32 [num_seqs]: tokens in the cache for the request, this
 *              step's rows included (seq_lens[b] >= q_b)
 * max_query_len, max_seq_len: host-side upper bounds of q_b and seq_lens
 * causal       1 (the chunked-prefill case) or 0
 * workspace    >= pa_chunked_prefill_workspace_bytes_ex(..., dtype) bytes of
 *              device scratch (no initialisation needed; 16-byte aligned);
 *              required even when no request is split
 * dtype        PA_BF16 or PA_F32 (caches, query and out alike)
 *
 * pa_chunked_prefill_workspace_bytes is the PA_BF16 size; 0 for an invalid
 * shape.
 */
size_t pa_chunked_prefill_workspace_bytes(int32_t num_seqs, int64_t num_q_tokens, int32_t max_query_len,
                                          int32_t max_seq_len, int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim);
size_t pa_chunked_prefill_workspace_bytes_ex(int32_t num_seqs, int64_t num_q_tokens, int32_t max_query_len,
                                             int32_t max_seq_len, int32_t num_heads, int32_t num_kv_heads,
                                             int32_t head_dim, pa_dtype dtype);
pa_status pa_chunked_prefill(void *out, const void *query, int64_t q_token_stride,
                             const void *key_cache, const void *value_cache,
                             const int32_t *block_table, int32_t max_blocks_per_req,
                             const int32_t *cu_query_lens, const int32_t *seq_lens,
                             int32_t num_seqs, int64_t num_q_tokens, int32_t max_query_len,
                             int32_t max_seq_len, int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                             int32_t causal, void *workspace, size_t workspace_bytes,
                             pa_dtype dtype, hipStream_t stream);

/*
 * Checks of the device-array contract (see the conventions at the top), on
 * HOST copies of the arrays: the launch path cannot check array contents
 * without a host synchronisation, so a harness or a debugging caller runs
 * these.  Each returns PA_OK, or PA_ERR_INVALID_ARG with the first offending
 * entry named in pa_last_error_message().
 *
 * pa_validate_block_tables: 0 <= seq_lens[b] <= max_seq_len <=
 *   max_blocks_per_req * block_size, and block_table[b][i] in [0, num_blocks)
 *   for every block a sequence uses (i < ceil(seq_lens[b] / block_size)).
 *   Several tables may name the same block (shared prefixes).
 * pa_validate_slot_mapping: no two tokens write the same slot (slots < 0 or
 *   past the pool are skipped by the scatters and ignored here).
 * pa_validate_query_lens: cu_query_lens[0] = 0, non-decreasing, ending at
 *   num_q_tokens; each request's rows at most max_query_len and at most its
 *   seq_lens.
 *
 * With PA_DEBUG=1 in the environment, pa_decode, pa_decode_append (and its
 * allocation-free form), pa_decode_fp8(_ex), pa_chunked_prefill,
 * pa_reshape_and_cache and pa_reshape_and_cache_fp8(_ex) copy their arrays to
 * the host (synchronising `stream`), run these checks and return their status
 * before launching anything.  pa_decode_append checks the blocks of each
 * sequence's tokens before its newest one (the newest token may have no block;
 * then it is not written).  Skipped while `stream` records a graph.
 */
pa_status pa_validate_block_tables(const int32_t *block_table, int32_t max_blocks_per_req,
                                   const int32_t *seq_lens, int32_t num_seqs, int64_t num_blocks,
                                   int32_t block_size, int32_t max_seq_len);
pa_status pa_validate_slot_mapping(const int64_t *slot_mapping, int64_t num_tokens,
                                   int64_t num_blocks, int32_t block_size);
pa_status pa_validate_query_lens(const int32_t *cu_query_lens, const int32_t *seq_lens,
                                 int32_t num_seqs, int64_t num_q_tokens, int32_t max_query_len);

/*
 * Memory probes.  They are not part of the attention path: they give its
 * HBM-bound roofline a measured denominator on the same GPU (decode reads the
 * whole KV cache and is bound by memory, per the article's section "Attention
 * (FlashAttention, Scaled Dot-Product Attention)"), and a transfer of known
 * size for scaling hardware traffic counters.
 *
 * pa_probe_stream_read reads `bytes` from `src` once (16-byte loads over a
 * grid-stride loop) and writes nothing in practice (`sink`, one uint32, is
 * written only if the XOR of all words equals a fixed 32-bit constant).
 * pa_probe_copy copies `bytes` from `src` to `dst` (non-overlapping).
 * bytes: a multiple of 16; pointers 16-byte aligned; workgroups: grid size in
 * 256-thread workgroups, 0 = automatic.  bytes == 0 is a no-op.
 */
pa_status pa_probe_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t workgroups,
                               hipStream_t stream);
pa_status pa_probe_copy(void *dst, const void *src, int64_t bytes, int32_t workgroups,
                        hipStream_t stream);

/*
 * Matrix-core probe.  Not part of the attention path: it gives the MFMA-bound
 * roofline of the chunked prefill (a dense contraction over the query rows,
 * the article's section "Attention (FlashAttention, Scaled Dot-Product
 * Attention)") the rate the matrix cores sustain on the same GPU, next to the
 * nominal peak.  `workgroups` workgroups of 4 waves each run `iters` rounds of
 * 4 independent v_mfma_f32_32x32x16_bf16 products: workgroups * 4 * iters * 4
 * * 32768 flops.  `sink` (one uint32) is written only if the accumulators sum
 * to a fixed value, which does not happen.  workgroups > 0, iters >= 0;
 * PA_ERR_INVALID_ARG otherwise.
 */
pa_status pa_probe_mfma(uint32_t *sink, int32_t workgroups, int32_t iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
