/*
 * CPU oracle for paged KV-cache attention.  TEST INFRASTRUCTURE ONLY: the
 * tests, the smoke check and the benchmark's CPU-baseline leg call it; the
 * product path never does.  It shares no code, header or helper with the HIP
 * library.
 *
 * It is the plain definition, written for a reader to check by eye:
 *   - slot of a token: the page table lookup and the block/offset split of
 *     "AI Infra入门干货总结：大模型是如何高效推理的", section "Paged Attention"
 *     (slot_idx = block_idx * block_size + block_offset, worked example
 *     block_table [5, 8, 12], position 25 -> slot 137);
 *   - scatter: copy each new token's K and V rows into the slot its
 *     slot_mapping entry names (same section, reshape_and_cache);
 *   - attention: softmax(Q K^T / sqrt(d_k) + M) V per query head, with the
 *     grouped-query map kv_head = q_head / (num_heads / num_kv_heads), the K/V
 *     rows gathered token by token through block_table, and M the causal mask
 *     (same article, section "Attention (FlashAttention, Scaled Dot-Product
 *     Attention)", its formula and its step table).
 *
 * The softmax is the naive two-pass one (max, then exp / sum) in fp64.  There is
 * no online softmax, no tiling and no split here: those are the GPU's
 * reformulations and are checked against this.
 *
 * Inputs are the exact storage the GPU reads: dtype 0 = float32, dtype 1 =
 * bf16 bit patterns (uint16).  Both are widened to double before any
 * arithmetic.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_E4M3 2
#define ORACLE_E5M2 3

/* Number of threads the attention loop uses (OpenMP), for reporting. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

double oracle_e4m3_value(uint8_t code);
double oracle_e5m2_value(uint8_t code);

/* Threads the attention loop may use from now on (OpenMP); for timing. */
void oracle_set_threads(int32_t n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static double widen(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    if (dtype == ORACLE_E4M3)
        return oracle_e4m3_value(((const uint8_t *)base)[idx]);
    if (dtype == ORACLE_E5M2)
        return oracle_e5m2_value(((const uint8_t *)base)[idx]);
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;   /* bf16 is the top half of a float32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Slot of logical position `pos` of the request whose block_table row is
 * `bt_row`: the logical block pos / block_size is looked up in the page table,
 * then slot = physical_block * block_size + pos % block_size. */
int64_t oracle_slot(const int32_t *bt_row, int64_t pos, int32_t block_size)
{
    int64_t logical_block = pos / block_size;
    int64_t physical_block = bt_row[logical_block];
    int64_t block_offset = pos % block_size;
    return physical_block * block_size + block_offset;
}

/* slot_mapping for a list of (request, position) tokens.  A negative position
 * or request marks a padding token (slot -1, skipped by the scatter); a table
 * entry < 0 (no block allocated) also yields -1. */
void oracle_slot_mapping(const int32_t *block_table, int64_t bt_row_stride,
                         const int32_t *token_seq, const int32_t *token_pos, int64_t num_tokens,
                         int32_t block_size, int64_t *slot_mapping)
{
    for (int64_t i = 0; i < num_tokens; i++) {
        if (token_seq[i] < 0 || token_pos[i] < 0) {
            slot_mapping[i] = -1;
            continue;
        }
        const int32_t *row = block_table + (int64_t)token_seq[i] * bt_row_stride;
        if (row[token_pos[i] / block_size] < 0) {
            slot_mapping[i] = -1;
            continue;
        }
        slot_mapping[i] = oracle_slot(row, token_pos[i], block_size);
    }
}

/* reshape_and_cache: for every token with slot s >= 0, split s back into
 * (block, offset) and copy the token's [num_kv_heads, head_dim] K row and V row
 * into cache[block, offset, :, :].  Bit copy; nothing else in the cache
 * changes.  Token rows are `key_stride` / `value_stride` elements apart. */
void oracle_reshape_and_cache(const void *key, int64_t key_stride,
                              const void *value, int64_t value_stride,
                              void *key_cache, void *value_cache,
                              const int64_t *slot_mapping, int64_t num_tokens,
                              int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                              int32_t elem_bytes)
{
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    for (int64_t i = 0; i < num_tokens; i++) {
        int64_t s = slot_mapping[i];
        if (s < 0)
            continue;
        int64_t block = s / block_size;
        int64_t offset = s % block_size;
        int64_t dst = (block * block_size + offset) * row_elems;   /* [num_blocks, block_size, Hkv, D] */
        memcpy((char *)key_cache + dst * elem_bytes,
               (const char *)key + i * key_stride * elem_bytes, (size_t)(row_elems * elem_bytes));
        memcpy((char *)value_cache + dst * elem_bytes,
               (const char *)value + i * value_stride * elem_bytes, (size_t)(row_elems * elem_bytes));
    }
}

/* Attention over the paged cache, one function for decode and chunked prefill.
 *
 * Request b has query_len_b = cu_query_lens[b+1] - cu_query_lens[b] query rows
 * (flattened at rows cu_query_lens[b] ..) and seq_lens[b] KV tokens, this
 * step's tokens included.  Query row j sits at absolute position
 * seq_lens[b] - query_len_b + j; with `causal` it sees keys 0 .. that position,
 * otherwise all seq_lens[b] keys.  A row that sees no key outputs zeros.
 *
 * out:   double [num_q_tokens, num_heads, head_dim]
 * query: [num_q_tokens, num_heads, head_dim], rows q_stride elements apart,
 *        storage dtype `dtype`
 * key_cache, value_cache: [num_blocks, block_size, num_kv_heads, head_dim],
 *        storage dtype `kv_dtype`; an element stands for its stored value
 *        times k_scale (keys) or v_scale (values), the scales being 1 except
 *        for an fp8 cache
 * probs (optional): the softmax row of every (query row, head), at
 *        probs[(row * num_heads + h) * probs_stride + t]
 */
void oracle_attention(double *out, const void *query, int64_t q_stride,
                      const void *key_cache, const void *value_cache,
                      const int32_t *block_table, int64_t bt_row_stride,
                      const int32_t *cu_query_lens, const int32_t *seq_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, double scale, int32_t causal, int32_t dtype,
                      int32_t kv_dtype, double k_scale, double v_scale,
                      double *probs, int64_t probs_stride)
{
    const int32_t group = num_heads / num_kv_heads;
    const int64_t num_q_tokens = cu_query_lens[num_seqs];
    const int64_t n_rows = num_q_tokens * num_heads;

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t row_head = 0; row_head < n_rows; row_head++) {
        const int64_t row = row_head / num_heads;
        const int32_t h = (int32_t)(row_head % num_heads);

        int32_t b = 0;                                   /* request owning this query row */
        while (cu_query_lens[b + 1] <= row)
            b++;
        const int64_t qlen = cu_query_lens[b + 1] - cu_query_lens[b];
        const int64_t j = row - cu_query_lens[b];
        const int64_t L = seq_lens[b];
        const int64_t pos_q = L - qlen + j;
        const int64_t n = causal ? pos_q + 1 : L;        /* keys 0 .. n-1 are visible */
        const int32_t kvh = h / group;                   /* grouped-query head map */
        const int32_t *bt_row = block_table + (int64_t)b * bt_row_stride;

        double *o = out + row_head * head_dim;
        for (int32_t d = 0; d < head_dim; d++)
            o[d] = 0.0;
        if (n <= 0)
            continue;

        double *s = (double *)malloc(sizeof(double) * (size_t)n);
        const int64_t qbase = row * q_stride + (int64_t)h * head_dim;

        /* pass 1: scores s_t = scale * <q, k_t>, with k_t gathered through the
         * page table, and their maximum */
        double m = -INFINITY;
        for (int64_t t = 0; t < n; t++) {
            int64_t blk = bt_row[t / block_size];
            int64_t off = t % block_size;
            int64_t kbase = ((blk * block_size + off) * num_kv_heads + kvh) * (int64_t)head_dim;
            double dot = 0.0;
            for (int32_t d = 0; d < head_dim; d++)
                dot += widen(query, qbase + d, dtype) * (widen(key_cache, kbase + d, kv_dtype) * k_scale);
            s[t] = scale * dot;
            if (s[t] > m)
                m = s[t];
        }

        /* pass 2: p_t = exp(s_t - m), l = sum p_t, out = sum p_t v_t / l */
        double l = 0.0;
        for (int64_t t = 0; t < n; t++) {
            s[t] = exp(s[t] - m);
            l += s[t];
        }
        for (int64_t t = 0; t < n; t++) {
            int64_t blk = bt_row[t / block_size];
            int64_t off = t % block_size;
            int64_t vbase = ((blk * block_size + off) * num_kv_heads + kvh) * (int64_t)head_dim;
            double w = s[t] / l;
            for (int32_t d = 0; d < head_dim; d++)
                o[d] += w * (widen(value_cache, vbase + d, kv_dtype) * v_scale);
            if (probs)
                probs[row_head * probs_stride + t] = w;
        }
        free(s);
    }
}

/* ---------------------------------------------------------------------------
 * The step just before attention: split a fused QKV projection row, rotate Q
 * and K by their token's position (RoPE), and hand K and V to the scatter.
 * "AI Infra入门干货总结：大模型是如何高效推理的", section "Reshape & Cache" and its
 * table (Q is the first num_heads * head_dim columns of the projection, K the
 * next num_kv_heads * head_dim, V the last; RoPE is applied elementwise from a
 * cos/sin table of shape [max_position_embeddings, rotary_dim] looked up by
 * position), and the RoPE summary near its opening (each pair of dimensions is
 * a point in the complex plane, turned by the angle position * theta).
 * ------------------------------------------------------------------------- */

/* cos/sin table: row p holds cos(p * theta_i) in columns 0 .. R/2-1 and
 * sin(p * theta_i) in columns R/2 .. R-1, with theta_i = base^(-2i / R) (the
 * RoFormer frequency schedule; the pages give the base, 500000 for Llama-3-8B,
 * and the table's shape). */
void oracle_rope_table(double *table, int64_t max_position, int32_t rotary_dim, double base)
{
    const int32_t half = rotary_dim / 2;
    for (int64_t p = 0; p < max_position; p++) {
        for (int32_t i = 0; i < half; i++) {
            double theta = pow(base, -2.0 * i / rotary_dim);
            double angle = (double)p * theta;
            table[p * rotary_dim + i] = cos(angle);
            table[p * rotary_dim + half + i] = sin(angle);
        }
    }
}

/* Turn one head vector x (head_dim values, widened to double) by the angles of
 * one table row.  Pair i (i < R/2) is the point (x[a], x[b]) with
 * a = i, b = i + R/2 when neox_style (halves paired), or a = 2i, b = 2i + 1
 * otherwise (neighbours paired); it becomes
 *   (x[a] cos - x[b] sin,  x[b] cos + x[a] sin).
 * Dimensions from rotary_dim on are not turned. */
static void rotate_head(double *out, const double *x, const float *row, int32_t rotary_dim,
                        int32_t neox_style, int32_t head_dim)
{
    const int32_t half = rotary_dim / 2;
    for (int32_t d = 0; d < head_dim; d++)
        out[d] = x[d];
    for (int32_t i = 0; i < half; i++) {
        int32_t a = neox_style ? i : 2 * i;
        int32_t b = neox_style ? i + half : 2 * i + 1;
        double c = (double)row[i];
        double s = (double)row[half + i];
        out[a] = x[a] * c - x[b] * s;
        out[b] = x[b] * c + x[a] * s;
    }
}

/* For each token t of a fused projection qkv [num_tokens, (Hq + 2 Hkv) * D]
 * (rows qkv_stride elements apart, dtype 0 = float32, 1 = bf16 bits):
 *   q_out[t, h, :] = rotate(Q head h of row t, position[t])       (fp64)
 *   k_out[t, h, :] = rotate(K head h of row t, position[t])       (fp64)
 *   v_out[t, h, :] = V head h of row t                            (fp64, as stored)
 * cos_sin: float32 [max_position, rotary_dim], laid out as oracle_rope_table
 * writes it; positions must lie in [0, max_position). */
void oracle_rope_qkv(double *q_out, double *k_out, double *v_out, const void *qkv, int64_t qkv_stride,
                     const int64_t *positions, const float *cos_sin, int32_t rotary_dim,
                     int32_t neox_style, int64_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t dtype)
{
    double *x = (double *)malloc(sizeof(double) * head_dim);
    const int64_t k_col = (int64_t)num_heads * head_dim;
    const int64_t v_col = k_col + (int64_t)num_kv_heads * head_dim;
    for (int64_t t = 0; t < num_tokens; t++) {
        const float *row = cos_sin + positions[t] * rotary_dim;
        const int64_t base = t * qkv_stride;
        for (int32_t h = 0; h < num_heads; h++) {
            for (int32_t d = 0; d < head_dim; d++)
                x[d] = widen(qkv, base + (int64_t)h * head_dim + d, dtype);
            rotate_head(q_out + (t * num_heads + h) * head_dim, x, row, rotary_dim, neox_style, head_dim);
        }
        for (int32_t h = 0; h < num_kv_heads; h++) {
            for (int32_t d = 0; d < head_dim; d++)
                x[d] = widen(qkv, base + k_col + (int64_t)h * head_dim + d, dtype);
            rotate_head(k_out + (t * num_kv_heads + h) * head_dim, x, row, rotary_dim, neox_style, head_dim);
            for (int32_t d = 0; d < head_dim; d++)
                v_out[(t * num_kv_heads + h) * head_dim + d] =
                    widen(qkv, base + v_col + (int64_t)h * head_dim + d, dtype);
        }
    }
    free(x);
}

/* ---------------------------------------------------------------------------
 * fp8 KV cache.  The pages say only that halving the bits per KV entry nearly
 * halves decode time, and that e4m3 and e5m2 are both in use.  The format is
 * taken from its published definition (OCP 8-bit floating point, E4M3): sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m * 2^-9; S.1111.111 is NaN and there is no infinity, so the
 * largest finite value is 1.75 * 2^8 = 448.  A cached value is
 * code_value * scale, one float32 scale for K and one for V.
 * ------------------------------------------------------------------------- */

/* The real number a code stands for (NaN for the two NaN codes). */
double oracle_e4m3_value(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Encode y: the nearest of the 127 finite magnitudes 0x00 .. 0x7E, a tie going
 * to the code whose mantissa is even, and magnitudes beyond 448 (infinity
 * included) saturated to 448; NaN gives the NaN code.  The sign bit is y's. */
uint8_t oracle_e4m3_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0;
    if (isnan(y))
        return sign | 0x7F;
    double a = fabs((double)y);
    if (a >= 448.0)
        return sign | 0x7E;
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs(oracle_e4m3_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | (uint8_t)best;
}

/* The other 8-bit format the pages name, from the same specification: OCP
 * E5M2 -- sign, 5 exponent bits with bias 15, 2 mantissa bits; exponent field
 * 0 holds the subnormals m * 2^-16; exponent field 31 holds infinity (mantissa
 * 0) and NaN (mantissa 1 .. 3); the largest finite value is 1.75 * 2^15 =
 * 57344. */
double oracle_e5m2_value(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 2) & 31;
    int m = code & 3;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -16);
    else
        v = ldexp(1.0 + m / 4.0, e - 15);
    return sign ? -v : v;
}

/* Encode y as E5M2: the nearest of the finite magnitudes 0x00 .. 0x7B, a tie
 * going to the code whose mantissa is even, and magnitudes beyond 57344
 * (infinity included) saturated to 57344, as for E4M3, so that a stored code
 * is always finite; NaN gives the NaN code 0x7F.  The sign bit is y's. */
uint8_t oracle_e5m2_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0;
    if (isnan(y))
        return sign | 0x7F;
    double a = fabs((double)y);
    if (a >= 57344.0)
        return sign | 0x7B;
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7B; c++) {
        double d = fabs(oracle_e5m2_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | (uint8_t)best;
}

static uint8_t encode_fp8(float y, int32_t fmt)
{
    return fmt == 1 ? oracle_e5m2_encode(y) : oracle_e4m3_encode(y);
}

/* The fp8 scatter: like oracle_reshape_and_cache, but each element x of the
 * token's K (V) row is stored as the code of x / k_scale (v_scale), the
 * division done in float32, in the format fmt (0: E4M3, encoded by
 * oracle_e4m3_encode; 1: E5M2, by oracle_e5m2_encode).  key/value are float32
 * (dtype 0) or bf16 bits (dtype 1); the caches hold one byte per element. */
void oracle_reshape_and_cache_fp8(const void *key, int64_t key_stride, const void *value, int64_t value_stride,
                                  uint8_t *key_cache, uint8_t *value_cache, const int64_t *slot_mapping,
                                  int64_t num_tokens, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t dtype, float k_scale, float v_scale, int32_t fmt)
{
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    /* bf16 sources have 65536 bit patterns: the code of each (the same
     * encode(x / scale) as below) is worked out once per pair of scales, and
     * looked up.  Not thread-safe: the oracle's scatter runs on one thread. */
    static uint8_t kcode_memo[65536], vcode_memo[65536];
    static float memo_k = 0.f, memo_v = 0.f;
    static int32_t memo_fmt = -1;
    const uint8_t *kcode = NULL, *vcode = NULL;
    if (dtype == ORACLE_BF16) {
        if (memo_fmt != fmt || memo_k != k_scale || memo_v != v_scale) {
            for (int32_t u = 0; u < 65536; u++) {
                uint16_t bits = (uint16_t)u;
                float x = (float)widen(&bits, 0, ORACLE_BF16);
                kcode_memo[u] = encode_fp8(x / k_scale, fmt);
                vcode_memo[u] = encode_fp8(x / v_scale, fmt);
            }
            memo_k = k_scale, memo_v = v_scale, memo_fmt = fmt;
        }
        kcode = kcode_memo;
        vcode = vcode_memo;
    }
    for (int64_t i = 0; i < num_tokens; i++) {
        int64_t s = slot_mapping[i];
        if (s < 0)
            continue;
        int64_t dst = ((s / block_size) * block_size + s % block_size) * row_elems;
        for (int64_t e = 0; e < row_elems; e++) {
            if (kcode) {
                key_cache[dst + e] = kcode[((const uint16_t *)key)[i * key_stride + e]];
                value_cache[dst + e] = vcode[((const uint16_t *)value)[i * value_stride + e]];
                continue;
            }
            float k = (float)widen(key, i * key_stride + e, dtype);
            float v = (float)widen(value, i * value_stride + e, dtype);
            key_cache[dst + e] = encode_fp8(k / k_scale, fmt);
            value_cache[dst + e] = encode_fp8(v / v_scale, fmt);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Copy-on-write of shared blocks.  Sequences that share a prefix point their
 * block tables at the same physical blocks (prefix caching); before one of
 * them writes into a shared block it gets a private copy ("AI Infra入门干货总结：
 * 大模型是如何高效推理的", section "Paged Attention": the cache is
 * [num_layers, 2, num_blocks, block_size, num_kv_heads, head_dim]; the
 * inference field notes' chapter on batching and memory management names
 * copy-on-write and prefix caching).
 *
 * For each pair (src, dst) of block_mapping [num_pairs][2], in order, with
 * both in [0, num_blocks): block dst of every layer's K and V cache becomes a
 * byte copy of block src.  Layer l's K cache starts layer_stride_bytes * l
 * after key_cache, its V cache as far after value_cache; a block is
 * block_bytes long.  Pairs with an id outside the pool are skipped.
 * ------------------------------------------------------------------------- */
void oracle_copy_blocks(void *key_cache, void *value_cache, int64_t layer_stride_bytes, int32_t num_layers,
                        int64_t num_blocks, int64_t block_bytes, const int64_t *block_mapping, int64_t num_pairs)
{
    for (int64_t p = 0; p < num_pairs; p++) {
        int64_t src = block_mapping[2 * p], dst = block_mapping[2 * p + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)
            continue;
        for (int32_t l = 0; l < num_layers; l++) {
            char *k = (char *)key_cache + l * layer_stride_bytes;
            char *v = (char *)value_cache + l * layer_stride_bytes;
            memmove(k + dst * block_bytes, k + src * block_bytes, (size_t)block_bytes);
            memmove(v + dst * block_bytes, v + src * block_bytes, (size_t)block_bytes);
        }
    }
}
