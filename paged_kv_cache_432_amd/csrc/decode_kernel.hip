// Paged decode attention for gfx950: one query token per sequence against its
// paged K/V, with the online softmax, and long contexts split into pieces whose
// partial results are merged with log-sum-exp weights.
//
// What is computed follows "AI Infra入门干货总结：大模型是如何高效推理的":
//   section "Attention (FlashAttention, Scaled Dot-Product Attention)" -- scores
//   scale * <q, k_t>, softmax, weighted sum of v_t; kv_head = q_head / G with
//   G = num_heads / num_kv_heads; K/V rows found through block_table; the
//   running max / running sum, with earlier partial results rescaled when the
//   max grows, so that the scores never leave the chip;
//   its closing summary -- Flash-Decoding splits the KV axis to occupy more
//   compute units and merges the pieces with log-sum-exp.
//
// One wavefront attends one KV head of one sequence over a contiguous range of
// its 16-token blocks.  For bf16 the products run on the matrix cores
// (attend_mfma(): per block, S^T = K Q^T and O^T += V^T P^T as 16x16 MFMA tiles
// whose lane layouts let P and V pass from the loads to the products without
// any exchange; see there).  The vector path (attend() below, used for fp32):
//   * The G query heads of the KV head share every K/V row the wave loads, so
//     each cache byte is read once per call.
//   * A 16-token block of one KV head is 16 rows of 256 B (bf16), Hkv*256 B
//     apart.  Two lane layouts read it with 16-byte loads:
//       K layout: lane = 4*t + c holds token t, dims {32j + 8c .. +8 : j<4}; a
//         quad of lanes covers one row, so <q_h, k_t> needs a 2-step quad
//         reduction only;
//       V layout: lane = 16*g + d holds dims 8d .. 8d+7 of tokens 4g .. 4g+3;
//         every load instruction covers 4 whole rows, and each lane's running
//         output is G x 8 fp32 values that need no exchange until the end.
//     The probabilities move from the K layout to the V layout through 16*G
//     floats of LDS per wave.
//   * The running max is shared by the whole wave per head; a wave-uniform
//     branch skips the max reduction and the rescale unless some score of the
//     block exceeds it.  Exponentials are base 2 with log2(e) folded into the
//     scale.
//   * Block ids are loaded 64 at a time (one per lane) and broadcast with
//     v_readlane.  K/V are read with buffer loads whose resource is the block:
//     two blocks are in flight (the next one's loads are issued as soon as a
//     block is consumed), and a load past the range gets an empty resource (no
//     memory access, zeros), so that every load in the loop is unconditional
//     and the compiler's wait counts stay exact.
//
// Two ways of cutting the work into wavefronts:
//   * partitions (partition_tokens > 0 or -1): one wave per (sequence, KV
//     head, partition of a fixed number of tokens);
//   * balanced stream (the automatic choice): the grid is exactly as many
//     workgroups as the GPU holds at once; the (sequence, block) space is
//     flattened and every workgroup takes an equal contiguous share of it, one
//     wave per KV head of a group.  A sequence cut between workgroups leaves
//     a partial result in each, merged afterwards; a workgroup holds at most
//     two such pieces (its first and its last).  A matrix-core wave keeps its
//     first piece's record in LDS and writes both records when its share is
//     done, so that no record write lands in the middle of the read stream.
//   * append mode (pa_decode_append): each sequence's newest token is one more
//     unit after its cached blocks, read from its input row; the merge launch
//     copies it to its cache slot.  Over an fp8 cache (pa_decode_append_fp8)
//     the workgroup that reads a sequence's last block first stores the newest
//     token's codes into it, and the walk is the plain one.
//   * the split merge takes one wave per (sequence, query head), or, past one
//     round of resident waves, two heads of a KV head per wave.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kWavesPerGroup = 4;        // partitioned mode: waves per workgroup
constexpr int kRec = kDecodeRecordFloats; // partial record: 128 acc, max, sum, pad
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format (gfx9)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

template <bool NT>
__device__ __forceinline__ void buffer_chunk(ChunkBF16& c, rsrc_t r, uint32_t off) {
    c.w = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, NT ? 2 : 0));
}
template <bool NT>
__device__ __forceinline__ void buffer_chunk(ChunkF32& c, rsrc_t r, uint32_t off) {
    c.a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, NT ? 2 : 0));
    c.b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off + 16, 0, NT ? 2 : 0));
}

#ifndef PA_DECODE_QUERY_IN_LDS_FROM
#define PA_DECODE_QUERY_IN_LDS_FROM 8
#endif
#ifndef PA_DECODE_PIPELINE_DEPTH
#define PA_DECODE_PIPELINE_DEPTH 2
#endif
// Query rows live in LDS at G = 8, where registers would hold 8 x 16 bf16 of
// them per lane (16 copies of each, one per token lane) and leave one wave per
// SIMD.  At G = 4 they stay in registers: LDS reads on every block cost more
// than the third wave per SIMD they would free (measured on the Llama-3-8B
// decode shapes).  fp32 rows, twice the registers, move to LDS from G = 4.
template <typename Elem, int G>
constexpr bool kQueryInLds = G >= (sizeof(Elem) == 4 ? 4 : PA_DECODE_QUERY_IN_LDS_FROM);

// Blocks each wave keeps in flight.  Three also fit two waves per SIMD (252
// VGPRs at G = 4) but measured the same as two on the Llama-3-8B and G = 8
// decode shapes, so two it is (239 VGPRs).  An fp32 block holds twice the
// registers: at G = 8 two of them spill, so those waves keep one.
template <typename Elem, int G>
constexpr int kPipelineDepth = sizeof(Elem) == 4 && G >= 8 ? 1 : PA_DECODE_PIPELINE_DEPTH;

// Per-wave state of one (sequence, KV head) range: the G query rows (in
// registers, in the K layout, or -- QL -- in the wave's LDS slot, read back
// per block: lanes of one dim chunk read the same address, a broadcast), the
// running max / sum of each head (lane c keeps heads c and c+4), and the
// unnormalised output in the V layout.
template <typename Chunk, typename Elem, int G, bool QL>
struct WaveState {
    static constexpr int NSEL = (G + 3) / 4;
    Chunk q[QL ? 1 : G][4];
    Elem* qs;                      // QL: this wave's [G][128] query rows in LDS
    float m[NSEL], l[NSEL];
    float acc[G][8];
};

template <typename Chunk, typename Elem, int G, bool QL>
__device__ __forceinline__ void load_query(const DecodeArgs& a, int64_t row, int kvh, int lane,
                                           WaveState<Chunk, Elem, G, QL>& st) {
    const int c = lane & 3;
    const Elem* qp = reinterpret_cast<const Elem*>(a.query) + row * a.q_stride + (int64_t)kvh * G * kHeadDim;
    if constexpr (QL) {
        // G*16 chunks of 8 elements, spread over the lanes, copied to LDS
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i0 = 0; i0 < G * 16; i0 += kWave) {
            const int i = i0 + lane;
            if (i < G * 16) {
                Chunk x;
                load_chunk<false>(x, qp + i * 8);
                store_chunk_raw(st.qs + i * 8, x);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) load_chunk<false>(st.q[h][j], qp + h * kHeadDim + j * 32 + c * 8);
    }
#pragma unroll
    for (int r = 0; r < WaveState<Chunk, Elem, G, QL>::NSEL; ++r) { st.m[r] = -INFINITY; st.l[r] = 0.f; }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.f;
}

// Online-softmax attention of one wave over blocks [0, nblk) of the table row
// `bt` (its first entry is the range's first block); `tok_first` is the token
// position of that block and `tok_end` the sequence length (tokens at or past
// it are masked out).
template <typename Chunk, typename Elem, int G, bool QL, bool NT, int NBUF>
__device__ __forceinline__ void attend(const DecodeArgs& a, int kvh, const int32_t* __restrict__ bt,
                                       int nblk, int tok_first, int tok_end, float* pl, int lane,
                                       WaveState<Chunk, Elem, G, QL>& st) {
    constexpr int NSEL = WaveState<Chunk, Elem, G, QL>::NSEL;
    constexpr int EPC = 8;
    const int Hkv = a.num_kv_heads;
    const uint32_t eb = sizeof(Elem);
    const uint32_t tok_bytes = (uint32_t)Hkv * kHeadDim * eb;       // between tokens of a block
    const uint32_t blk_bytes = tok_bytes * kBlock;
    const int t = lane >> 2, c = lane & 3;                          // K layout
    const int g = lane >> 4, dch = lane & 15;                       // V layout
    const uint32_t koff = t * tok_bytes + (uint32_t)kvh * kHeadDim * eb + c * EPC * eb;
    const uint32_t voff = 4 * g * tok_bytes + (uint32_t)kvh * kHeadDim * eb + dch * EPC * eb;
    const char* kc = reinterpret_cast<const char*>(a.key_cache);
    const char* vc = reinterpret_cast<const char*>(a.value_cache);

    for (int cb = 0; cb < nblk; cb += kWave) {
        const int nb = min(kWave, nblk - cb);
        const int bid = lane < nb ? bt[cb + lane] : 0;

        auto issue = [&](Chunk (&kb)[4], Chunk (&vb)[4], int i) {
            // Past the range: an empty resource, so the loads touch no memory.
            // An id outside the pool (a caller error) is clamped into it: wrong
            // values, but no access outside the cache.
            const int64_t phys = min(max((int64_t)__builtin_amdgcn_readlane(bid, min(i, nb - 1)), (int64_t)0),
                                     a.num_blocks - 1);
            const int nrec = i < nb ? (int)blk_bytes : 0;
            const int64_t off = phys * (int64_t)blk_bytes;
            const rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + off), (short)0, nrec, kRsrcWord3);
            const rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + off), (short)0, nrec, kRsrcWord3);
#pragma unroll
            for (int j = 0; j < 4; ++j) buffer_chunk<NT>(kb[j], rk, koff + j * 32 * eb);
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) buffer_chunk<NT>(vb[i4], rv, voff + i4 * tok_bytes);
        };

        auto process = [&](const Chunk (&kb)[4], const Chunk (&vb)[4], int i) {
            const int tok0 = tok_first + (cb + i) * kBlock;
            const bool tail = tok0 + kBlock > tok_end;

            // scores of token t for every head of the group (quad reduction)
            float s[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float x = 0.f;
                if constexpr (QL) {
                    Chunk qh[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) load_chunk<false>(qh[j], st.qs + h * kHeadDim + j * 32 + c * 8);
#pragma unroll
                    for (int j = 0; j < 4; ++j) x = dot_chunk(qh[j], kb[j], x);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) x = dot_chunk(st.q[h][j], kb[j], x);
                }
                x += dpp<kQuadSwap1>(x);
                x += dpp<kQuadSwap2>(x);
                s[h] = x;
            }
            // lane c keeps head c (and c + 4 when G = 8)
            float ss[NSEL];
#pragma unroll
            for (int r = 0; r < NSEL; ++r) {
                float v = -INFINITY;
#pragma unroll
                for (int h = 0; h < G; ++h)
                    if (h == c + 4 * r) v = s[h];
                v *= a.scale_log2;
                if (tail && tok0 + t >= tok_end) v = -INFINITY;
                ss[r] = v;
            }

            bool grow = false;
#pragma unroll
            for (int r = 0; r < NSEL; ++r) grow |= ss[r] > st.m[r];
            if (__builtin_amdgcn_ballot_w64(grow)) {
                float alpha[NSEL];
#pragma unroll
                for (int r = 0; r < NSEL; ++r) {
                    float bm = ss[r];
                    bm = fmaxf(bm, dpp<kRowRor4>(bm));
                    bm = fmaxf(bm, dpp<kRowRor8>(bm));
                    bm = fmaxf(bm, shfl_xor_f(bm, 16));
                    bm = fmaxf(bm, shfl_xor_f(bm, 32));
                    const float mn = fmaxf(st.m[r], bm);
                    alpha[r] = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(st.m[r] - mn);
                    st.l[r] *= alpha[r];
                    st.m[r] = mn;
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float ah = readlane_f(alpha[h / 4], h % 4);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) st.acc[h][e] *= ah;
                }
            }

#pragma unroll
            for (int r = 0; r < NSEL; ++r) {
                if (c + 4 * r < G) {
                    const float p = __builtin_amdgcn_exp2f(ss[r] - st.m[r]);
                    st.l[r] += p;
                    pl[t * G + c + 4 * r] = p;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int row = 4 * g + i4;
                float pr[G];
#pragma unroll
                for (int h = 0; h < G; ++h) pr[h] = pl[row * G + h];
                float vf[EPC];
                to_f32(vb[i4], vf);
                if (tail && tok0 + row >= tok_end) {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) vf[e] = 0.f;       // stale or poisoned slot: select out
                }
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < EPC; ++e) st.acc[h][e] = fmaf(pr[h], vf[e], st.acc[h][e]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };

        // NBUF blocks in flight: block i + NBUF is issued as soon as block i is
        // consumed.
        Chunk kbuf[NBUF][4], vbuf[NBUF][4];
#pragma unroll
        for (int b = 0; b < NBUF; ++b) issue(kbuf[b], vbuf[b], b);
        for (int i = 0; i < nb; i += NBUF) {
#pragma unroll
            for (int b = 0; b < NBUF; ++b) {
                if (b == 0 || i + b < nb) process(kbuf[b], vbuf[b], i + b);
                issue(kbuf[b], vbuf[b], i + b + NBUF);
            }
        }
    }
}

// Finish a range: sum the per-lane pieces, then either normalise and store the
// G output rows at `out` (out[h * 128 + d]), or store the unnormalised rows
// with their (max, sum) as partial records at `rec` (record h at rec + h * kRec).
template <typename Chunk, typename Elem, int G, bool QL>
__device__ __forceinline__ void finish(WaveState<Chunk, Elem, G, QL>& st, int lane, Elem* out, float* rec) {
    const int g = lane >> 4, dch = lane & 15;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            st.acc[h][e] += shfl_xor_f(st.acc[h][e], 16);
            st.acc[h][e] += shfl_xor_f(st.acc[h][e], 32);
        }
#pragma unroll
    for (int r = 0; r < WaveState<Chunk, Elem, G, QL>::NSEL; ++r) {
        st.l[r] += dpp<kRowRor4>(st.l[r]);
        st.l[r] += dpp<kRowRor8>(st.l[r]);
        st.l[r] += shfl_xor_f(st.l[r], 16);
        st.l[r] += shfl_xor_f(st.l[r], 32);
    }
    float lh[G], mh[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        lh[h] = readlane_f(st.l[h / 4], h % 4);
        mh[h] = readlane_f(st.m[h / 4], h % 4);
    }
    if (g != 0) return;
    if (out) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float inv = lh[h] > 0.f ? 1.f / lh[h] : 0.f;
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = st.acc[h][e] * inv;
            store_chunk(out + h * kHeadDim + dch * 8, f);
        }
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            store_chunk(rec + h * kRec + dch * 8, st.acc[h]);
            if (dch == h) *reinterpret_cast<float2*>(rec + h * kRec + kHeadDim) = make_float2(mh[h], lh[h]);
        }
    }
}

// ---- matrix-core wave (bf16) ------------------------------------------------
// The same attention of one wave over a block range, with the products on the
// matrix cores: per 16-token block, S^T = K Q^T on v_mfma_f32_16x16x32_bf16
// (16 tokens x 16 head columns, the G heads and zero padding) and
// O^T += V^T P^T on v_mfma_f32_16x16x16_bf16.  Lane l = 16g + i:
//   * K operand of product step ks: token i, dims 32ks + 8g .. +8, so that one
//     load instruction reads 64 contiguous bytes of each of the 16 rows; Q is
//     held in the same order;
//   * S^T accumulator: head i, tokens 4g .. 4g+3 -- exactly the B-operand
//     layout of P^T in the second product, so P stays in registers;
//   * V operand: the V layout of the vector path (dims 8i .. 8i+7 of tokens
//     4g .. 4g+3), read as output row i of dim tile dt meaning dim 8i + dt, so
//     each operand is one byte permute of two loaded words, no transpose;
//   * O^T accumulator: acc[dt][r] = O[head i][8 (4g + r) + dt].
// P enters the second product as two bf16 operands, hi = p truncated to bf16
// and lo = bf16(p - hi) (~16 bits of p).  The reference max is raised only when
// a block's maximum exceeds it by more than 2^8 (log2 units), so the rescale of
// the accumulators is rare; p stays below 256.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
constexpr float kMfmaSlack = 8.f;

// Matrix-core path for bf16 at G >= this group size (the vector path below it
// and for fp32).
#ifndef PA_DECODE_MFMA_FROM
#define PA_DECODE_MFMA_FROM 1
#endif
template <typename Elem, int G>
constexpr bool kMfmaWave = sizeof(Elem) == 2 && G >= PA_DECODE_MFMA_FROM;

// Blocks each matrix-core wave keeps in flight (its loop has far less vector
// work per block than the vector path's, so more of the wave's time is spent
// waiting on memory: three measured 4-7% faster than two).
#ifndef PA_DECODE_MFMA_DEPTH
#define PA_DECODE_MFMA_DEPTH 3
#endif
constexpr int kMfmaDepth = PA_DECODE_MFMA_DEPTH;
// K/V loads of the stream decode with the streaming (non-temporal) cache hint.
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif
constexpr bool kDecodeNT = PA_DECODE_NT != 0;
// Blocks in flight per wave over an fp8 cache: each holds half the bytes of a
// bf16 block, so twice as many keep the same bytes in flight.
#ifndef PA_DECODE_FP8_DEPTH
#define PA_DECODE_FP8_DEPTH 6
#endif
constexpr int kFp8Depth = PA_DECODE_FP8_DEPTH;

struct MfmaState {
    u32x4_t q[4];                  // B operand of S^T for product step ks: dims 32ks + 8g .. +8 (zero past G)
    float m, l;                    // head i: reference max (log2 units); this lane's part of the sum
    f32x4_t acc[8];
};

template <int G>
__device__ __forceinline__ void load_query_mfma(const DecodeArgs& a, int64_t row, int kvh, int lane, MfmaState& st) {
    const int i = lane & 15, g = lane >> 4;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.query) + row * a.q_stride +
                         (int64_t)(kvh * G + (i < G ? i : 0)) * kHeadDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        st.q[ks] = i < G ? *reinterpret_cast<const u32x4_t*>(qp + 32 * ks) : u32x4_t{0u, 0u, 0u, 0u};
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// One block's online softmax and O^T += V^T P^T for the matrix-core wave: s
// holds the lane's scores (head i, tokens 4g .. 4g+3, masked ones -inf), v its
// V chunks (tokens 4g .. 4g+3, dims 8i .. 8i+7).
// v[r]: eight 16-bit V values (dims 8i .. 8i+7 of token 4g + r).  F16: v is
// fp16 (exact for an fp8 cache), P is rounded once to fp16 and one
// 16x16x16 f16 product per dim tile takes it; the row sum adds the same
// rounded P.  Otherwise v is bf16 and P goes in as bf16 hi + lo, two products.
template <bool F16 = false>
__device__ __forceinline__ void softmax_pv_mfma(const DecodeArgs& a, MfmaState& st, f32x4_t s, const u32x4_t (&v)[4]) {
    float mx = maximum(maximum(s[0], s[1]), maximum(s[2], s[3]));
    mx = max_across_rows(mx);
    const float mblk = mx * a.scale_log2;
    const bool bump = mblk > st.m + kMfmaSlack;
    const float mn = bump ? mblk : st.m;
    const float msafe = mn == -INFINITY ? 0.f : mn;
    const float alpha = bump ? __builtin_amdgcn_exp2f(st.m - mn) : 1.f;
    if (__builtin_amdgcn_ballot_w64(bump && st.m != -INFINITY)) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.acc[dt] *= alpha;
    }
    st.m = mn;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], a.scale_log2, -msafe));
    if constexpr (F16) {
        const f16x2_t p01 = __builtin_convertvector(f32x2_t{p[0], p[1]}, f16x2_t);
        const f16x2_t p23 = __builtin_convertvector(f32x2_t{p[2], p[3]}, f16x2_t);
        const f16x2_t one = f16x2_t{(_Float16)1.f, (_Float16)1.f};
        st.l = __builtin_amdgcn_fdot2(p23, one, __builtin_amdgcn_fdot2(p01, one, st.l * alpha, false), false);
        const f16x4_t P = f16x4_t{p01.x, p01.y, p23.x, p23.y};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
            const int w = dt >> 1;
            const u32x2_t av = u32x2_t{__builtin_amdgcn_perm(v[1][w], v[0][w], sel),
                                       __builtin_amdgcn_perm(v[3][w], v[2][w], sel)};
            st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, av), P, st.acc[dt], 0, 0, 0);
        }
        return;
    }
    st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    uint32_t u[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) u[r] = __float_as_uint(p[r]);
    // hi = p truncated to bf16 (top 16 bits); lo = bf16(p - hi), p - hi exact in fp32
    const u32x2_t phi = u32x2_t{__builtin_amdgcn_perm(u[1], u[0], 0x07060302u),
                                __builtin_amdgcn_perm(u[3], u[2], 0x07060302u)};
    const u32x2_t plo = u32x2_t{pack_bf16x2(p[0] - __uint_as_float(u[0] & 0xffff0000u),
                                            p[1] - __uint_as_float(u[1] & 0xffff0000u)),
                                pack_bf16x2(p[2] - __uint_as_float(u[2] & 0xffff0000u),
                                            p[3] - __uint_as_float(u[3] & 0xffff0000u))};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        // element dt of the four token chunks: word dt / 2, low or high half
        const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
        const int w = dt >> 1;
        const u32x2_t av = u32x2_t{__builtin_amdgcn_perm(v[1][w], v[0][w], sel),
                                   __builtin_amdgcn_perm(v[3][w], v[2][w], sel)};
        const s16x4_t A = __builtin_bit_cast(s16x4_t, av);
        st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(s16x4_t, phi), st.acc[dt],
                                                               0, 0, 0);
        st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(s16x4_t, plo), st.acc[dt],
                                                               0, 0, 0);
    }
}

template <int G, bool NT, int NBUF>
__device__ __forceinline__ void attend_mfma(const DecodeArgs& a, int kvh, const int32_t* __restrict__ bt, int nblk,
                                            int tok_first, int tok_end, int lane, MfmaState& st) {
    const uint32_t tok_bytes = (uint32_t)a.num_kv_heads * kHeadDim * 2;
    const uint32_t blk_bytes = tok_bytes * kBlock;
    const int i = lane & 15, g = lane >> 4;
    const uint32_t koff = i * tok_bytes + (uint32_t)kvh * kHeadDim * 2 + g * 16;
    const uint32_t voff = 4 * g * tok_bytes + (uint32_t)kvh * kHeadDim * 2 + i * 16;
    const char* kc = reinterpret_cast<const char*>(a.key_cache);
    const char* vc = reinterpret_cast<const char*>(a.value_cache);

    for (int cb = 0; cb < nblk; cb += kWave) {
        const int nb = min(kWave, nblk - cb);
        const int bid = lane < nb ? bt[cb + lane] : 0;

        auto issue = [&](u32x4_t (&kb)[4], u32x4_t (&vb)[4], int j) {
            // The resource spans the block's valid tokens' rows: tokens past the
            // end (stale or poisoned slots) and blocks past the range read as
            // zeros without touching memory.  An id outside the pool is clamped
            // into it.
            const int64_t phys = min(max((int64_t)__builtin_amdgcn_readlane(bid, min(j, nb - 1)), (int64_t)0),
                                     a.num_blocks - 1);
            const int valid = j < nb ? min(max(tok_end - (tok_first + (cb + j) * kBlock), 0), kBlock) : 0;
            const int nrec = __builtin_amdgcn_readfirstlane(valid * (int)tok_bytes);
            const int64_t off = phys * (int64_t)blk_bytes;
            const rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + off), (short)0, nrec, kRsrcWord3);
            const rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + off), (short)0, nrec, kRsrcWord3);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kb[ks] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(koff + 64 * ks), 0,
                                                                                             NT ? 2 : 0));
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vb[r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rv, (int)(voff + r * tok_bytes), 0, NT ? 2 : 0));
        };

        auto process = [&](const u32x4_t (&kb)[4], const u32x4_t (&vb)[4], int j) {
            // tokens of the block this lane's scores cover: 4g .. 4g+3; those past
            // the end are masked (their K and V rows read as zeros)
            const int nval = tok_end - (tok_first + (cb + j) * kBlock) - 4 * g;
            f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb[ks]),
                                                            __builtin_bit_cast(bf16x8_t, st.q[ks]), s, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r] = r < nval ? s[r] : -INFINITY;
            softmax_pv_mfma(a, st, s, vb);
        };

        // Blocks are issued in the order they are consumed (the scheduling
        // barriers keep it), so that each wait covers only the block it needs.
        u32x4_t kbuf[NBUF][4], vbuf[NBUF][4];
#pragma unroll
        for (int b = 0; b < NBUF; ++b) {
            issue(kbuf[b], vbuf[b], b);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int j = 0; j < nb; j += NBUF) {
#pragma unroll
            for (int b = 0; b < NBUF; ++b) {
                if (b == 0 || j + b < nb) process(kbuf[b], vbuf[b], j + b);
                issue(kbuf[b], vbuf[b], j + b + NBUF);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// Finish a range of the matrix-core wave: as finish(), lanes of head i < G
// writing dims 32g + 8r .. +8 from acc[0..7][r].
// SC: every output and partial accumulator is multiplied by oscale (the V
// scale of an fp8 cache).
template <int G, bool SC = false>
__device__ __forceinline__ void finish_mfma(const MfmaState& st, int lane, uint16_t* out, float* rec,
                                            float oscale = 1.f) {
    const int i = lane & 15, g = lane >> 4;
    const float l = sum_across_rows(st.l);
    if (i >= G) return;
    if (out) {
        const float inv = (l > 0.f ? 1.f / l : 0.f) * (SC ? oscale : 1.f);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float f[8];
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) f[dt] = st.acc[dt][r] * inv;
            store_chunk(out + i * kHeadDim + 32 * g + 8 * r, f);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float f[8];
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) f[dt] = SC ? st.acc[dt][r] * oscale : st.acc[dt][r];
            store_chunk(rec + i * kRec + 32 * g + 8 * r, f);
        }
        if (g == 0) *reinterpret_cast<float2*>(rec + i * kRec + kHeadDim) = make_float2(st.m, l);
    }
}

// Query (and output) row of sequence b, or -1 when b is not a single-row
// sequence of a mixed batch (the prefill kernel attends those).
__device__ __forceinline__ int64_t decode_row(const DecodeArgs& a, int64_t b) {
    if (!a.cu_q) return b;
    const int32_t r = a.cu_q[b];
    return a.cu_q[b + 1] - r == 1 ? (int64_t)r : -1;
}

__device__ __forceinline__ int seq_len_of(const DecodeArgs& a, int64_t b) {
    // Lengths beyond the block table's row are cut to it, so that no table entry
    // outside the row is read even when seq_lens breaks the contract.
    return max(min(a.seq_lens[b], a.bt_stride * kBlock), 0);
}

// The matrix-core wave over its whole share of the stream mode: units
// u0 .. u1-1 (sequence, KV-head group, block), KV head grp * W + wi of each.
// The share is a run of segments, one per (sequence, group), and its blocks
// are loaded NBUF ahead straight across segment boundaries.  The workgroup
// (whose waves all walk the same units) first writes an LDS table of the
// share, up to kShareTable units at a time: per unit the physical block id,
// its valid token count, the group, the query row and the blocks left in the
// sequence.  The waves read it with LDS loads, whose wait count is apart from
// that of the K/V loads in flight, so no step of the walk waits for memory
// except on the data it is about to use.  Each segment's query is loaded when
// the previous segment starts.  At a boundary the wave finishes one segment
// (rows, or a partial record in the workgroup's slot 0 for its first segment
// and slot 1 for its last) and starts the next with its blocks in flight.
constexpr int kShareTable = 1024;
constexpr int kFirstBlock = 1 << 30;                  // table flag: block 0 of its sequence
// Table flag (append mode): the unit is the sequence's newest token, read from
// its input row (the unit's id field holds the row) as a one-token block.
constexpr int kAppendUnit = 0x80;

// fp8 append form: the newest token of each sequence (position seq_lens[b] -
// 1, input row b) is quantised into its slot by the workgroup whose share holds
// the sequence's last block, once that block's table window is built and before
// any of the window's blocks is read (no other workgroup reads that block).
// s_last[0] counts the window's last blocks (of a sequence and KV-head group),
// s_last[1..] are their table indices.  The table entry gives the block id, the
// block's token count (the newest token is the last of them) and the group; the
// slot rule is the page-table lookup's (-1, and nothing stored, without a
// block).  The owner of group 0's last block writes slot_out[b].  Tasks: (last
// block, head of the group, K or V, 16-element chunk of the 128), each a
// 32-byte load of the bf16 row, the scatter's encoder and a 16-byte store.
template <bool E5>
__device__ void store_newest_fp8(const DecodeArgs& a, const int4* s_tab, const int32_t* s_last, int W) {
    const int per = W * 2 * (kHeadDim / 16);
    const int tasks = s_last[0] * per;
    const int64_t num_slots = a.num_blocks * kBlock;
    const int64_t tok_bytes = (int64_t)a.num_kv_heads * kHeadDim;   // one byte per code
    for (int t = threadIdx.x; t < tasks; t += blockDim.x) {
        const int4 e = s_tab[s_last[1 + t / per]];
        int r = t % per;
        const int c = r % (kHeadDim / 16);
        r /= kHeadDim / 16;
        const bool is_v = (r & 1) != 0;
        const int hw = r >> 1;
        const int grp = e.y >> 8, valid = e.y & 0xff;
        const int64_t b = e.z;                         // the input row: the sequence (no mixed batch here)
        const int kvh = grp * W + hw;
        const char* src = (is_v ? a.new_value + b * a.new_value_stride : a.new_key + b * a.new_key_stride) +
                          ((int64_t)kvh * kHeadDim + 16 * c) * 2;
        ChunkBF16 x0, x1;
        load_chunk<false>(x0, src);
        load_chunk<false>(x1, src + 16);
        const int64_t slot = e.x >= 0 ? (int64_t)e.x * kBlock + valid - 1 : -1;
        if (grp == 0 && hw == 0 && !is_v && c == 0 && a.slot_out) a.slot_out[b] = slot;
        if (slot < 0 || slot >= num_slots) continue;
        uint8_t* dst = reinterpret_cast<uint8_t*>(const_cast<void*>(is_v ? a.value_cache : a.key_cache)) +
                       slot * tok_bytes + (int64_t)kvh * kHeadDim + 16 * c;
        *reinterpret_cast<u32x4_t*>(dst) = fp8_codes<ChunkBF16, E5>(x0, x1, is_v ? a.v_scale : a.k_scale);
    }
}

// One block's K and V rows of one KV head as a lane holds them in flight.
// bf16: K dims 32ks + 8g .. +8 of token i for product step ks; V dims 8i .. +8
// of tokens 4g .. 4g+3.  fp8 (one byte per element): K bytes 32g .. 32g+31 of
// token i (dims 32g + 8ks .. +8 feed step ks: the query is loaded in the same
// dim order, so the product is unchanged); V as bf16, 8 bytes per token.
template <bool F8> struct KvBuf;
template <> struct KvBuf<false> { u32x4_t k[4], v[4]; };
template <> struct KvBuf<true> { u32x4_t k[2]; u32x2_t v[4]; };

// Two fp8 codes (the low or high half of a word) -> two fp16 / two bf16, for
// E4M3 (E5 = false) or E5M2 (E5 = true) codes.
template <bool E5, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16(uint32_t w) {
    if constexpr (E5)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.f, HI));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, HI));
}
template <bool E5, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16(uint32_t w) {
    if constexpr (E5)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.f, HI));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HI));
}
// Eight fp8 values in two words -> eight fp16, exactly, byte e -> element e:
// every E4M3 value is an fp16 value (at most 448, at least 2^-9), and so is
// every finite E5M2 value (the same exponent range as fp16, fewer mantissa
// bits).
template <bool E5>
__device__ __forceinline__ u32x4_t fp8x8_to_f16(uint32_t w0, uint32_t w1) {
    return u32x4_t{fp8x2_to_f16<E5, false>(w0), fp8x2_to_f16<E5, true>(w0), fp8x2_to_f16<E5, false>(w1),
                   fp8x2_to_f16<E5, true>(w1)};
}
// Eight fp8 values in two words -> eight bf16, exactly (every E4M3 and every
// finite E5M2 value is a bf16 value), byte e -> element e.
template <bool E5>
__device__ __forceinline__ u32x4_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
    return u32x4_t{fp8x2_to_bf16<E5, false>(w0), fp8x2_to_bf16<E5, true>(w0), fp8x2_to_bf16<E5, false>(w1),
                   fp8x2_to_bf16<E5, true>(w1)};
}

// s_first: this wave's LDS area of 2 x G records.  The record of the wave's
// first segment, when that segment is cut, is kept there and written out with
// the last one when the share is done: during the share the only global writes
// are the rows of whole segments (records written in the middle of the read
// stream measured 4-10% slower decode calls).  The last segment's record, when
// cut, is staged in the second half, so that both leave as coalesced stores.
template <int G, bool NT, int NBUF, bool F8 = false, bool AP = false, bool E5 = false>
__device__ __forceinline__ void stream_share_mfma(const DecodeArgs& a, const int32_t* s_pref, int4* s_tab, int64_t u0,
                                                  int64_t u1, int W, int NG, int wi, int lane, float* s_first,
                                                  int32_t* s_last) {
    const int total = (int)(u1 - u0);                  // the same for every wave of the workgroup
    if (total <= 0) return;
    const int B = a.num_seqs;
    constexpr int kEb = F8 ? 1 : 2;                    // cache bytes per element
    // the newest token as a unit of its own, read from its input row (bf16
    // append); or (fp8 append) stored into the cache as codes after each table
    // window is built, before any of its blocks is read
    constexpr bool APR = AP && !F8;
    constexpr bool APS = AP && F8;
    const uint32_t tok_bytes = (uint32_t)a.num_kv_heads * kHeadDim * kEb;
    const uint32_t blk_bytes = tok_bytes * kBlock;
    const int i = lane & 15, g = lane >> 4;
    // the KV head's row start goes in the base
    const uint32_t koff = i * tok_bytes + g * (F8 ? 32 : 16);
    const uint32_t voff = 4 * g * tok_bytes + i * (F8 ? 8 : 16);
    const char* kc = reinterpret_cast<const char*>(a.key_cache);
    const char* vc = reinterpret_cast<const char*>(a.value_cache);

    int c0 = 0, c1 = 0;                                // the table holds blocks [c0, c1)
    // the table entry of block j in [c0, c1), the same address in every lane
    auto entry = [&](int j, int& id, int& valid, int& grp, bool& app) {
        const int2 e = *reinterpret_cast<const int2*>(&s_tab[j - c0]);
        id = __builtin_amdgcn_readfirstlane(e.x);
        const int vg = __builtin_amdgcn_readfirstlane(e.y);
        valid = vg & (APR ? kAppendUnit - 1 : 0xff);
        app = APR && (vg & kAppendUnit) != 0;
        grp = vg >> 8;
    };

    auto issue = [&](KvBuf<F8>& buf, int j) {
        int id = 0, valid = 0, grp = 0;
        bool app = false;
        if (j < c1) entry(j, id, valid, grp, app);
        const int64_t phys = min(max((int64_t)id, (int64_t)0), a.num_blocks - 1);   // an id outside the pool: clamped
        // the resource spans the block's valid rows: past-the-end slots and
        // blocks past the table read as zeros without touching memory
        int nrec = valid * (int)tok_bytes;
        const int64_t hoff = (int64_t)(grp * W + wi) * kHeadDim * kEb;
        const int64_t off = phys * (int64_t)blk_bytes + hoff;
        const char* kb = kc + off;
        const char* vb = vc + off;
        if constexpr (APR) {
            // the newest token: its input row is token 0 of a one-token block
            // (lanes of the other tokens read past the 256 bytes: zeros)
            kb = app ? a.new_key + id * a.new_key_stride + hoff : kb;
            vb = app ? a.new_value + id * a.new_value_stride + hoff : vb;
            nrec = app ? kHeadDim * kEb : nrec;
        }
        const rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, nrec, kRsrcWord3);
        const rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vb, (short)0, nrec, kRsrcWord3);
        if constexpr (F8) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
                buf.k[h] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(koff + 16 * h), 0, NT ? 2 : 0));
#pragma unroll
            for (int r = 0; r < 4; ++r)
                buf.v[r] = __builtin_bit_cast(
                    u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(voff + r * tok_bytes), 0, NT ? 2 : 0));
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                buf.k[ks] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(koff + 64 * ks), 0, NT ? 2 : 0));
#pragma unroll
            for (int r = 0; r < 4; ++r)
                buf.v[r] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(voff + r * tok_bytes), 0, NT ? 2 : 0));
        }
    };

    // the current segment, and the query of the segment starting at block qn_at
    MfmaState st;
    u32x4_t qn[4];
    int qn_at = -1;
    int seg_end = 0;                                   // first block past the current segment
    bool seg_whole = false, seg_first = true;
    uint16_t* seg_out = nullptr;
    // (query row, KV head, blocks left in the sequence, first block?) of block j
    auto segment_at = [&](int j, int64_t& row, int& kvh, int& rem, bool& first) {
        const int4 e = s_tab[j - c0];
        row = __builtin_amdgcn_readfirstlane(e.z);
        kvh = (__builtin_amdgcn_readfirstlane(e.y) >> 8) * W + wi;
        const int w = __builtin_amdgcn_readfirstlane(e.w);
        rem = w & (kFirstBlock - 1);
        first = (w & kFirstBlock) != 0;
    };
    auto query_of = [&](int j, u32x4_t (&q)[4]) {
        int64_t row;
        int kvh, rem;
        bool first;
        segment_at(j, row, kvh, rem, first);
        // dims of step ks: 32ks + 8g .. +8 (bf16 cache), 32g + 8ks .. +8 (fp8)
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.query) + row * a.q_stride +
                             (int64_t)(kvh * G + (i < G ? i : 0)) * kHeadDim + (F8 ? 32 : 8) * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            q[ks] = i < G ? *reinterpret_cast<const u32x4_t*>(qp + (F8 ? 8 : 32) * ks) : u32x4_t{0u, 0u, 0u, 0u};
    };
    auto prefetch_query = [&]() {                      // the next segment's query, if it is in the table
        if (seg_end < c1) {
            query_of(seg_end, qn);
            qn_at = seg_end;
        }
    };
    bool first_in_lds = false;
    auto finish_segment = [&]() {
        if (seg_first && !seg_whole) {                 // the first segment's record: to LDS
            finish_mfma<G, F8>(st, lane, nullptr, s_first, a.out_scale);
            first_in_lds = true;
            return;
        }
        float* rec = a.part + ((((int64_t)blockIdx.x * 2 + (seg_first ? 0 : 1)) * W + wi) * G) * kRec;
        finish_mfma<G, F8>(st, lane, seg_whole ? seg_out : nullptr, seg_whole ? nullptr : rec, a.out_scale);
    };
    auto start_segment = [&](int j) {                  // block j begins a segment
        int64_t row;
        int kvh, rem;
        bool first;
        segment_at(j, row, kvh, rem, first);
        if (qn_at == j) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) st.q[ks] = qn[ks];
        } else {
            // not prefetched (the share's first segment, or one past a table
            // refill): load it here and wait for it on this path alone
            query_of(j, st.q);
            __builtin_amdgcn_s_waitcnt(0);
        }
        st.m = -INFINITY;
        st.l = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        seg_end = min(total, j + rem);
        seg_whole = first && seg_end - j == rem;
        seg_first = j == 0;
        seg_out = reinterpret_cast<uint16_t*>(a.out) + (row * a.num_heads + (int64_t)kvh * G) * kHeadDim;
        qn_at = -1;
        prefetch_query();
    };

    auto process = [&](const KvBuf<F8>& buf, int j) {
        if (j == seg_end) {                            // wave-uniform
            if (j > 0) finish_segment();
            start_segment(j);
        }
        int id, valid, grp;
        bool app;
        entry(j, id, valid, grp, app);
        const int nval = valid - 4 * g;                // this lane's tokens 4g .. 4g+3 of the block
        u32x4_t kb[4], vb[4];
        if constexpr (F8) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4_t w = buf.k[h];
                kb[2 * h] = fp8x8_to_bf16<E5>(w.x, w.y);
                kb[2 * h + 1] = fp8x8_to_bf16<E5>(w.z, w.w);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const u32x2_t w = buf.v[r];
                vb[r] = fp8x8_to_f16<E5>(w.x, w.y);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                kb[k] = buf.k[k];
                vb[k] = buf.v[k];
            }
        }
        f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb[ks]),
                                                        __builtin_bit_cast(bf16x8_t, st.q[ks]), s, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = r < nval ? s[r] : -INFINITY;
        softmax_pv_mfma<F8>(a, st, s, vb);
    };

    for (c0 = 0; c0 < total; c0 = c1) {
        c1 = min(total, c0 + kShareTable);
        // (the previous window's list was last read before the barrier that
        // ended its stores)
        if (APS && threadIdx.x == 0) s_last[0] = 0;
        __syncthreads();                               // the previous table is no longer read
        for (int t = threadIdx.x; t < c1 - c0; t += blockDim.x) {
            // unit -> (sequence b, group, block of b): b is the largest with NG * prefix[b] <= u
            const int64_t u = u0 + c0 + t;
            int lo = 0, hi = B - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((int64_t)NG * s_pref[mid] <= u) lo = mid; else hi = mid - 1;
            }
            const int nb = s_pref[lo + 1] - s_pref[lo];
            const int64_t r = u - (int64_t)NG * s_pref[lo];
            const int grp = (int)(r / nb), blk = (int)(r % nb);
            const int row = (int)decode_row(a, lo);    // >= 0: only decode rows own blocks
            int id, valid;
            if (APR && blk == nb - 1) {
                // the newest token, from input row `row` (= lo)
                id = row;
                valid = 1 | kAppendUnit;
            } else {
                // in append mode the cached blocks hold the tokens before the newest
                id = a.block_table[(int64_t)lo * a.bt_stride + blk];
                valid = min(max(seq_len_of(a, lo) - (APR ? 1 : 0) - blk * kBlock, 0), kBlock);
            }
            s_tab[t] = int4{id, valid | (grp << 8), row, (nb - blk) | (blk == 0 ? kFirstBlock : 0)};
            if (APS && blk == nb - 1) s_last[1 + atomicAdd(&s_last[0], 1)] = t;
        }
        __syncthreads();
        if constexpr (APS) {
            store_newest_fp8<E5>(a, s_tab, s_last, W);
            __syncthreads();                           // stored before the window's blocks are read
        }
        if (c0 > 0 && qn_at < 0) prefetch_query();    // the segment running on ends in this table
        KvBuf<F8> buf[NBUF];
#pragma unroll
        for (int b = 0; b < NBUF; ++b) {
            issue(buf[b], c0 + b);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int j = c0; j < c1; j += NBUF) {
#pragma unroll
            for (int b = 0; b < NBUF; ++b) {
                if (b == 0 || j + b < c1) process(buf[b], j + b);
                issue(buf[b], j + b + NBUF);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // Records leave LDS as whole consecutive 16-byte pieces per lane (1 KB per
    // store instruction); the last segment's record, when cut, goes the same way.
    auto copy_out = [&](const float* src_lds, int slot) {
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(a.part + (((int64_t)blockIdx.x * 2 + slot) * W + wi) * G * kRec);
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(src_lds);
        for (int c = lane; c < G * kRec / 4; c += kWave) dst[c] = src[c];
    };
    if (!seg_whole && !seg_first) {
        finish_mfma<G, F8>(st, lane, nullptr, s_first + G * kRec, a.out_scale);
        copy_out(s_first + G * kRec, 1);
    } else {
        finish_segment();
    }
    if (first_in_lds) copy_out(s_first, 0);            // wave-uniform; the same wave wrote the areas
}

// ---- partitioned mode ------------------------------------------------------
template <typename Chunk, typename Elem, int G, bool QL, bool NT>
__global__ void __launch_bounds__(256)
decode_partition_kernel(DecodeArgs a) {
    constexpr bool MF = kMfmaWave<Elem, G>;
    __shared__ __attribute__((aligned(16))) float p_lds[MF ? 1 : kWavesPerGroup][MF ? 4 : kBlock * G];
    __shared__ __attribute__((aligned(16))) Elem q_lds[QL && !MF ? kWavesPerGroup : 1][QL && !MF ? G * kHeadDim : 8];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int Hkv = a.num_kv_heads;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerGroup + wave;
    const int kvh = (int)(item % Hkv);
    const int64_t rest = item / Hkv;
    const int part = (int)(rest % a.max_partitions);
    const int64_t b = rest / a.max_partitions;
    if (b >= a.num_seqs) return;
    const int64_t row = decode_row(a, b);
    if (row < 0) return;
    const int L = seq_len_of(a, b);
    const int PT = a.partition_tokens;
    const int nparts = L <= 0 ? 1 : min((L + PT - 1) / PT, a.max_partitions);
    if (part >= nparts) return;
    const int tok_begin = part * PT;
    const int tok_end = min(L, tok_begin + PT);
    const int nblk = tok_end > tok_begin ? (tok_end - tok_begin + kBlock - 1) / kBlock : 0;

    const int64_t h0 = row * a.num_heads + (int64_t)kvh * G;
    const int64_t r0 = ((b * Hkv + kvh) * a.max_partitions + part) * G;
    const int32_t* bt = a.block_table + b * a.bt_stride + tok_begin / kBlock;
    if constexpr (kMfmaWave<Elem, G>) {
        MfmaState st;
        load_query_mfma<G>(a, row, kvh, lane, st);
        attend_mfma<G, NT, kMfmaDepth>(a, kvh, bt, nblk, tok_begin, L, lane, st);
        if (nparts == 1) finish_mfma<G>(st, lane, reinterpret_cast<uint16_t*>(a.out) + h0 * kHeadDim, nullptr);
        else finish_mfma<G>(st, lane, nullptr, a.part + r0 * kRec);
    } else {
        WaveState<Chunk, Elem, G, QL> st;
        st.qs = q_lds[QL ? wave : 0];
        load_query<Chunk, Elem, G, QL>(a, row, kvh, lane, st);
        attend<Chunk, Elem, G, QL, NT, kPipelineDepth<Elem, G>>(a, kvh, bt, nblk, tok_begin, L, p_lds[wave], lane, st);
        if (nparts == 1) finish<Chunk, Elem, G, QL>(st, lane, reinterpret_cast<Elem*>(a.out) + h0 * kHeadDim, nullptr);
        else finish<Chunk, Elem, G, QL>(st, lane, nullptr, a.part + r0 * kRec);
    }
}

// Partial record of (sequence b, query head h, partition p): the G heads of
// one KV head and partition are consecutive records.
__device__ __forceinline__ int64_t partition_record(const DecodeArgs& a, int64_t b, int h, int p) {
    const int G = a.num_heads / a.num_kv_heads;
    return ((b * a.num_kv_heads + h / G) * a.max_partitions + p) * G + (h % G);
}

// ---- balanced stream mode --------------------------------------------------
// Number of blocks per KV head of each sequence, as an inclusive prefix in
// s_pref[0..B] (s_pref[0] = 0); computed by the whole workgroup.  Append mode
// (AP): the cached blocks of the L - 1 tokens before the newest, plus one unit
// for the newest token.
template <bool AP = false>
__device__ __forceinline__ void block_prefix(const DecodeArgs& a, int32_t* s_pref, int32_t* s_wsum) {
    const int B = a.num_seqs;
    const int nthr = blockDim.x;
    const int tid = threadIdx.x;
    const int per = (B + nthr - 1) / nthr;
    const int lo = min(tid * per, B), hi = min(lo + per, B);
    int sum = 0;
    for (int i = lo; i < hi; ++i) {
        const int L = seq_len_of(a, i);
        const int n = decode_row(a, i) < 0 ? 0 : AP ? (L > 0 ? (L - 1 + kBlock - 1) / kBlock + 1 : 0)
                                                    : (L + kBlock - 1) / kBlock;
        s_pref[i + 1] = n;
        sum += n;
    }
    // inclusive scan of the per-thread sums: within the wave, then across waves
    const int lane = tid & 63, wave = tid >> 6;
    int x = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) s_wsum[wave] = x;
    __syncthreads();
    int before = x - sum;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
    for (int i = lo; i < hi; ++i) {
        before += s_pref[i + 1];
        s_pref[i + 1] = before;
    }
    if (tid == 0) s_pref[0] = 0;
    __syncthreads();
}

__device__ __forceinline__ int64_t stream_quantum(const DecodeArgs& a, int64_t units) {
    const int64_t q = (units + a.num_wg - 1) / a.num_wg;
    return q > a.min_quantum ? q : (int64_t)a.min_quantum;
}

// F8: the caches hold fp8 codes, E4M3 or (E5) E5M2; query and output stay bf16.
// AP: append mode (matrix-core path only): bf16 reads the newest token from
// its input row; fp8 (F8 and AP) stores it into the cache first.
template <typename Chunk, typename Elem, int G, bool QL, bool NT, bool F8 = false, bool AP = false, bool E5 = false>
__global__ void __launch_bounds__(512)
decode_stream_kernel(DecodeArgs a) {
    // [num_seqs + 1] block prefix, then (matrix-core waves) G records per wave
    extern __shared__ __attribute__((aligned(16))) int32_t s_pref[];
    __shared__ int32_t s_wsum[8];
    constexpr bool MF = kMfmaWave<Elem, G>;
    __shared__ __attribute__((aligned(16))) float p_lds[MF ? 1 : 8][MF ? 4 : kBlock * G];
    __shared__ __attribute__((aligned(16))) Elem q_lds[QL && !MF ? 8 : 1][QL && !MF ? G * kHeadDim : 8];
    __shared__ int4 s_tab[MF ? kShareTable : 1];
    __shared__ int32_t s_last[F8 && AP ? kShareTable + 1 : 1];   // fp8 append: the window's last blocks
    block_prefix<AP && !F8>(a, s_pref, s_wsum);
    const int B = a.num_seqs;
    const int W = a.waves_per_group;
    const int NG = a.num_kv_heads / W;
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i <= B; i += blockDim.x) a.prefix[i] = s_pref[i];
    const int64_t units = (int64_t)s_pref[B] * NG;
    const int64_t Q = stream_quantum(a, units);
    const int64_t u0 = (int64_t)blockIdx.x * Q;
    const int64_t u1 = min(u0 + Q, units);
    const int wi = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    float* pl = p_lds[MF ? 0 : wi];
    static_assert(!AP || MF, "append mode: matrix-core path");
    if constexpr (F8 && AP) {
        // the slot of a sequence without tokens is -1 (the others' slots are
        // written with their newest rows)
        if (blockIdx.x == 0 && a.slot_out)
            for (int b = threadIdx.x; b < B; b += blockDim.x)
                if (s_pref[b + 1] == s_pref[b]) a.slot_out[b] = -1;
    }
    if constexpr (MF) {
        float* s_first = reinterpret_cast<float*>(s_pref + ((B + 1 + 3) & ~3)) + wi * 2 * G * kRec;
        stream_share_mfma<G, NT, F8 ? kFp8Depth : kMfmaDepth, F8, AP, E5>(a, s_pref, s_tab, u0, u1, W, NG, wi,
                                                                          lane, s_first, s_last);
        return;
    }

    for (int64_t u = u0; u < u1;) {
        // the sequence holding unit u: the largest b with NG * prefix[b] <= u
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)NG * s_pref[mid] <= u) lo = mid; else hi = mid - 1;
        }
        const int b = lo;
        const int nblk_b = s_pref[b + 1] - s_pref[b];
        const int64_t r = u - (int64_t)NG * s_pref[b];
        const int grp = (int)(r / nblk_b);
        const int blk0 = (int)(r % nblk_b);
        const int n = (int)min((int64_t)(nblk_b - blk0), u1 - u);
        const int kvh = grp * W + wi;
        const int L = seq_len_of(a, b);
        const int64_t row = decode_row(a, b);          // >= 0: only decode rows own blocks

        const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride + blk0;
        const bool whole = blk0 == 0 && n == nblk_b;
        Elem* out = reinterpret_cast<Elem*>(a.out) + (row * a.num_heads + (int64_t)kvh * G) * kHeadDim;
        float* rec = a.part + ((((int64_t)blockIdx.x * 2 + (u == u0 ? 0 : 1)) * W + wi) * G) * kRec;
        WaveState<Chunk, Elem, G, QL> st;
        st.qs = q_lds[QL ? wi : 0];
        load_query<Chunk, Elem, G, QL>(a, row, kvh, lane, st);
        attend<Chunk, Elem, G, QL, NT, kPipelineDepth<Elem, G>>(a, kvh, bt, n, blk0 * kBlock, L, pl, lane, st);
        finish<Chunk, Elem, G, QL>(st, lane, whole ? out : nullptr, whole ? nullptr : rec);
        u += n;
    }
}

// ---- merges ----------------------------------------------------------------
// Log-sum-exp merge of the pieces of one (sequence, head):
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
// One wave per (sequence, head), two dims per lane; `rec_of(p)` gives the
// record index of piece p of n.
// Up to kFew pieces: every load is issued at once -- lane p's (max, sum) of
// piece p and this lane's two dims of every piece -- so the merge takes one
// round trip to memory (2 kFew registers for the rows).
template <int kFew, typename Elem, typename RecOf>
__device__ __forceinline__ void merge_few(const float* part, int n, RecOf rec_of, int lane, Elem* o) {
    {
        float2 v[kFew];
#pragma unroll
        for (int q = 0; q < kFew; ++q)
            v[q] = q < n ? *reinterpret_cast<const float2*>(part + rec_of(q) * kRec + 2 * lane) : make_float2(0.f, 0.f);
        const float2 ml = lane < n ? *reinterpret_cast<const float2*>(part + rec_of(lane) * kRec + kHeadDim)
                                   : make_float2(-INFINITY, 0.f);
        float M = ml.x;
#pragma unroll
        for (int d = 1; d < kFew; d <<= 1) M = fmaxf(M, shfl_xor_f(M, d));   // lanes >= n hold -inf
        M = readlane_f(M, 0);
        const float w = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
        float lsum = w * ml.y, o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int d = 1; d < kFew; d <<= 1) lsum += shfl_xor_f(lsum, d);
        lsum = readlane_f(lsum, 0);
#pragma unroll
        for (int q = 0; q < kFew; ++q) {
            if (q < n) {
                const float wq = readlane_f(w, q);
                o0 = fmaf(wq, v[q].x, o0);
                o1 = fmaf(wq, v[q].y, o1);
            }
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        if constexpr (sizeof(Elem) == 2) {
            *reinterpret_cast<uint32_t*>(o + 2 * lane) = pack_bf16x2(o0 * inv, o1 * inv);
        } else {
            *reinterpret_cast<float2*>(o + 2 * lane) = make_float2(o0 * inv, o1 * inv);
        }
    }
}

// Two heads per wave, one per 32-lane half: lane half hh merges the pieces
// rec_of(q, hh) of its head, and lane l holds dims 4 (l % 32) .. +4 of it; o
// is the lane's head's output row.  n <= kFew <= 32 pieces, every load issued
// at once, so the merge is one round trip.
template <int kFew, typename Elem, typename RecOf>
__device__ __forceinline__ void merge_pair(const float* part, int n, RecOf rec_of, int lane, Elem* o) {
    const int hh = lane >> 5, ln = lane & 31;
    f32x4_t v[kFew];
#pragma unroll
    for (int q = 0; q < kFew; ++q)
        v[q] = q < n ? *reinterpret_cast<const f32x4_t*>(part + rec_of(q, hh) * kRec + 4 * ln)
                     : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float2 ml = ln < n ? *reinterpret_cast<const float2*>(part + rec_of(ln, hh) * kRec + kHeadDim)
                             : make_float2(-INFINITY, 0.f);
    float M = ml.x;
#pragma unroll
    for (int d = 1; d < kFew; d <<= 1) M = fmaxf(M, shfl_xor_f(M, d));   // within the half; lanes >= n hold -inf
    M = hh ? readlane_f(M, 32) : readlane_f(M, 0);
    const float w = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
    float lsum = w * ml.y;
#pragma unroll
    for (int d = 1; d < kFew; d <<= 1) lsum += shfl_xor_f(lsum, d);
    lsum = hh ? readlane_f(lsum, 32) : readlane_f(lsum, 0);
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int q = 0; q < kFew; ++q) {
        if (q < n) {
            const float wq = hh ? readlane_f(w, 32 + q) : readlane_f(w, q);
            o0 = fmaf(wq, v[q].x, o0);
            o1 = fmaf(wq, v[q].y, o1);
            o2 = fmaf(wq, v[q].z, o2);
            o3 = fmaf(wq, v[q].w, o3);
        }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if constexpr (sizeof(Elem) == 2) {
        *reinterpret_cast<u32x2_t*>(o + 4 * ln) =
            u32x2_t{pack_bf16x2(o0 * inv, o1 * inv), pack_bf16x2(o2 * inv, o3 * inv)};
    } else {
        *reinterpret_cast<f32x4_t*>(o + 4 * ln) = f32x4_t{o0 * inv, o1 * inv, o2 * inv, o3 * inv};
    }
}

template <typename Elem, typename RecOf>
__device__ __forceinline__ void merge_pieces(const float* part, int n, RecOf rec_of, int lane, Elem* o) {
    // 8 pieces or fewer (the usual case), up to 24 (long contexts cut over
    // many workgroups; 48 registers of rows keep the kernel at 8 waves per
    // SIMD), or a loop for more
    if (n <= 8) return merge_few<8>(part, n, rec_of, lane, o);
    if (n <= 24) return merge_few<24>(part, n, rec_of, lane, o);
    // pass over the pieces' (max, sum), 64 at a time, one per lane
    float M = -INFINITY;
    for (int p0 = 0; p0 < n; p0 += kWave) {
        const int p = p0 + lane;
        const float mp = p < n ? part[rec_of(p) * kRec + kHeadDim] : -INFINITY;
        M = fmaxf(M, mp);
    }
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) M = fmaxf(M, shfl_xor_f(M, d));
    float lsum = 0.f, o0 = 0.f, o1 = 0.f;
    for (int p0 = 0; p0 < n; p0 += kWave) {
        // this lane's piece weight and weighted sum, then every piece's rows
        // with weights broadcast by v_readlane (independent loads)
        const int p = p0 + lane;
        float w = 0.f;
        if (p < n) {
            const float2 ml = *reinterpret_cast<const float2*>(part + rec_of(p) * kRec + kHeadDim);
            w = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
            lsum = fmaf(w, ml.y, lsum);
        }
        const int cnt = min(kWave, n - p0);
        for (int q = 0; q < cnt; ++q) {
            const float wq = readlane_f(w, q);
            const float2 v = *reinterpret_cast<const float2*>(part + rec_of(p0 + q) * kRec + 2 * lane);
            o0 = fmaf(wq, v.x, o0);
            o1 = fmaf(wq, v.y, o1);
        }
    }
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) lsum += shfl_xor_f(lsum, d);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if constexpr (sizeof(Elem) == 2) {
        *reinterpret_cast<uint32_t*>(o + 2 * lane) = pack_bf16x2(o0 * inv, o1 * inv);
    } else {
        *reinterpret_cast<float2*>(o + 2 * lane) = make_float2(o0 * inv, o1 * inv);
    }
}

template <typename Elem>
__global__ void __launch_bounds__(256)
merge_partitions_kernel(DecodeArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int Hq = a.num_heads;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerGroup + wave;
    const int64_t b = item / Hq;
    const int h = (int)(item % Hq);
    if (b >= a.num_seqs) return;
    const int64_t row = decode_row(a, b);
    if (row < 0) return;
    const int L = seq_len_of(a, b);
    const int PT = a.partition_tokens;
    const int nparts = L <= 0 ? 1 : min((L + PT - 1) / PT, a.max_partitions);
    if (nparts <= 1) return;
    merge_pieces<Elem>(a.part, nparts, [&](int p) { return partition_record(a, b, h, p); }, lane,
                       reinterpret_cast<Elem*>(a.out) + (row * Hq + h) * kHeadDim);
}

// Append mode: sequence b's newest token (position seq_lens[b] - 1), row b of
// new_key / new_value, is written to its slot of the caches, and the slot to
// slot_out[b], with the slot rule of the page-table lookup (-1 when the request
// has no block for that position: nothing is written).  The decode launch
// before never reads that slot (it took the token from its input row), so the
// copy is done here, one wave per (sequence, KV head): lanes 0-15 the K head's
// 256 bytes, lanes 16-31 the V head's.
__device__ __forceinline__ void append_head(const DecodeArgs& a, int64_t b, int kvh, int lane) {
    const int p = a.seq_lens[b] - 1;
    int64_t slot = -1;
    if (p >= 0 && p / kBlock < a.bt_stride) {
        const int32_t physical = a.block_table[b * a.bt_stride + p / kBlock];
        if (physical >= 0) slot = (int64_t)physical * kBlock + p % kBlock;
    }
    if (kvh == 0 && lane == 0 && a.slot_out) a.slot_out[b] = slot;
    if (slot < 0 || slot >= a.num_blocks * kBlock || lane >= 32) return;
    const bool is_v = lane >= 16;
    const int64_t off = (int64_t)kvh * kHeadDim * 2 + (lane & 15) * 16;
    const char* src = (is_v ? a.new_value + b * a.new_value_stride : a.new_key + b * a.new_key_stride) + off;
    char* dst = reinterpret_cast<char*>(const_cast<void*>(is_v ? a.value_cache : a.key_cache)) +
                slot * ((int64_t)a.num_kv_heads * kHeadDim * 2) + off;
    *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(src);
}

// The stream mode's split merge: one wave per (sequence, query head), or (PR)
// per (sequence, two query heads of one KV head), a head to each half of the
// wave, which halves the waves of a large batch.  A pair whose sequence was cut
// into more than 8 pieces is merged one head after the other by the whole wave.
template <typename Elem, bool AP = false, bool PR = false>
__global__ void __launch_bounds__(256)
merge_stream_kernel(DecodeArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int Hq = a.num_heads;
    const int HI = PR ? Hq / 2 : Hq;                   // items per sequence
    const int64_t item = (int64_t)blockIdx.x * kWavesPerGroup + wave;
    const int64_t b = item / HI;
    const int hi = (int)(item % HI);
    if (b >= a.num_seqs) return;
    if constexpr (AP)
        if (hi < a.num_kv_heads) append_head(a, b, hi, lane);
    const int G = Hq / a.num_kv_heads;
    const int W = a.waves_per_group;
    const int NG = a.num_kv_heads / W;
    const int h0 = PR ? 2 * hi : hi;                   // the wave's (first) head
    const int kvh = h0 / G, hg = h0 % G, grp = kvh / W, wi = kvh % W;
    const int64_t row = decode_row(a, b);
    if (row < 0) return;
    const int32_t pb = a.prefix[b];
    const int nblk = a.prefix[b + 1] - pb;
    Elem* o = reinterpret_cast<Elem*>(a.out) + (row * Hq + h0) * kHeadDim;
    if (nblk == 0) {                                   // empty sequence: zeros
        if constexpr (PR) {
            Elem* oh = o + (lane >> 5) * kHeadDim + 4 * (lane & 31);
            if constexpr (sizeof(Elem) == 2) *reinterpret_cast<u32x2_t*>(oh) = u32x2_t{0u, 0u};
            else *reinterpret_cast<f32x4_t*>(oh) = f32x4_t{0.f, 0.f, 0.f, 0.f};
        } else {
            if constexpr (sizeof(Elem) == 2) *reinterpret_cast<uint32_t*>(o + 2 * lane) = 0u;
            else *reinterpret_cast<float2*>(o + 2 * lane) = make_float2(0.f, 0.f);
        }
        return;
    }
    const int64_t units = (int64_t)a.prefix[a.num_seqs] * NG;
    const int64_t Q = stream_quantum(a, units);
    const int64_t S = (int64_t)NG * pb + (int64_t)grp * nblk;
    const int64_t E = S + nblk;
    const int64_t w_lo = S / Q, w_hi = (E - 1) / Q;
    if (w_lo == w_hi) return;                          // one workgroup wrote it whole
    const bool lo_is_last = S != w_lo * Q;             // the piece in w_lo is that workgroup's second
    const int n = (int)(w_hi - w_lo + 1);
    auto rec = [&](int p, int x) {                     // piece p of head h0 + x
        const int64_t w = w_lo + p;
        const int slot = (p == 0 && lo_is_last) ? 1 : 0;
        return (((w * 2 + slot) * W + wi) * G + hg + x);
    };
    if constexpr (PR) {
        if (n <= 8) {
            merge_pair<8, Elem>(a.part, n, rec, lane, o + (lane >> 5) * kHeadDim);
        } else {
            merge_pieces<Elem>(a.part, n, [&](int p) { return rec(p, 0); }, lane, o);
            merge_pieces<Elem>(a.part, n, [&](int p) { return rec(p, 1); }, lane, o + kHeadDim);
        }
    } else {
        merge_pieces<Elem>(a.part, n, [&](int p) { return rec(p, 0); }, lane, o);
    }
}



// Dynamic LDS of the stream kernel: the block prefix, then (matrix-core waves)
// each wave's 2 x G records (first and last segment).
size_t stream_lds_bytes(int64_t num_seqs, int waves, int G, bool mf) {
    const size_t pref = (((size_t)num_seqs + 1 + 3) & ~(size_t)3) * sizeof(int32_t);
    return pref + (mf ? (size_t)waves * 2 * G * kRec * sizeof(float) : 0);
}

template <typename Chunk, typename Elem, int G, bool F8 = false, bool AP = false, bool E5 = false>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    constexpr bool QL = kQueryInLds<Elem, G>;
    if (a.mode == kDecodeStream) {
        const size_t lds = stream_lds_bytes(a.num_seqs, a.waves_per_group, G, kMfmaWave<Elem, G>);
        hipLaunchKernelGGL((decode_stream_kernel<Chunk, Elem, G, QL, kDecodeNT, F8, AP, E5>), dim3((unsigned)a.num_wg),
                           dim3(64 * a.waves_per_group), lds, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t mitems = (int64_t)a.num_seqs * a.num_heads;
        constexpr bool MAP = AP && !F8;                // the merge writes the newest rows (bf16 append)
        if (a.merge_pair) {
            hipLaunchKernelGGL((merge_stream_kernel<Elem, MAP, true>),
                               dim3((unsigned)((mitems / 2 + kWavesPerGroup - 1) / kWavesPerGroup)), dim3(256), 0,
                               stream, a);
        } else {
            hipLaunchKernelGGL((merge_stream_kernel<Elem, MAP>),
                               dim3((unsigned)((mitems + kWavesPerGroup - 1) / kWavesPerGroup)), dim3(256), 0,
                               stream, a);
        }
        return hipGetLastError();
    }
    if constexpr (F8 || AP) return hipErrorInvalidValue; // an fp8 cache and append mode: stream mode only
    const int64_t items = (int64_t)a.num_seqs * a.max_partitions * a.num_kv_heads;
    const int64_t grid = (items + kWavesPerGroup - 1) / kWavesPerGroup;
    hipLaunchKernelGGL((decode_partition_kernel<Chunk, Elem, G, QL, true>), dim3((unsigned)grid), dim3(256), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_partitions <= 1) return e;
    const int64_t mitems = (int64_t)a.num_seqs * a.num_heads;
    hipLaunchKernelGGL((merge_partitions_kernel<Elem>),
                       dim3((unsigned)((mitems + kWavesPerGroup - 1) / kWavesPerGroup)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename Chunk, typename Elem, bool F8 = false, bool AP = false, bool E5 = false>
hipError_t launch_group(const DecodeArgs& a, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_typed<Chunk, Elem, 1, F8, AP, E5>(a, stream);
        case 2: return launch_typed<Chunk, Elem, 2, F8, AP, E5>(a, stream);
        case 4: return launch_typed<Chunk, Elem, 4, F8, AP, E5>(a, stream);
        case 8: return launch_typed<Chunk, Elem, 8, F8, AP, E5>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename Chunk, typename Elem, int G, bool F8, bool AP, bool E5>
int stream_blocks_per_cu(int waves_per_group, int64_t num_seqs) {
    const size_t lds = stream_lds_bytes(num_seqs, waves_per_group, G, kMfmaWave<Elem, G>);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, decode_stream_kernel<Chunk, Elem, G, kQueryInLds<Elem, G>, kDecodeNT, F8, AP, E5>, 64 * waves_per_group,
            lds) != hipSuccess)
        return 0;
    return n;
}

template <typename Chunk, typename Elem, bool F8 = false, bool AP = false, bool E5 = false>
int stream_blocks_group(int group, int waves_per_group, int64_t num_seqs) {
    switch (group) {
        case 1: return stream_blocks_per_cu<Chunk, Elem, 1, F8, AP, E5>(waves_per_group, num_seqs);
        case 2: return stream_blocks_per_cu<Chunk, Elem, 2, F8, AP, E5>(waves_per_group, num_seqs);
        case 4: return stream_blocks_per_cu<Chunk, Elem, 4, F8, AP, E5>(waves_per_group, num_seqs);
        case 8: return stream_blocks_per_cu<Chunk, Elem, 8, F8, AP, E5>(waves_per_group, num_seqs);
        default: return 0;
    }
}

}  // namespace

// dtype: 0 fp32, 1 bf16, 2 E4M3 cache with bf16 query and output, 3 bf16 in
// append mode, 4 E5M2 cache with bf16 query and output, 5 and 6 the E4M3 and
// E5M2 caches in append mode.
// The append form runs on the matrix-core wave only: a build that moves the
// bf16 decode to the vector wave (PA_DECODE_MFMA_FROM > 1, for measurement)
// leaves it out, and its launches fail.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int group, hipStream_t stream) {
#if PA_DECODE_MFMA_FROM <= 1
    if (dtype == 3) return launch_group<ChunkBF16, uint16_t, false, true>(a, group, stream);
    if (dtype == 5) return launch_group<ChunkBF16, uint16_t, true, true>(a, group, stream);
    if (dtype == 6) return launch_group<ChunkBF16, uint16_t, true, true, true>(a, group, stream);
#else
    if (dtype == 3 || dtype == 5 || dtype == 6) return hipErrorInvalidDeviceFunction;
#endif
    if (dtype == 4) return launch_group<ChunkBF16, uint16_t, true, false, true>(a, group, stream);
    if (dtype == 2) return launch_group<ChunkBF16, uint16_t, true>(a, group, stream);
    if (dtype == 1) return launch_group<ChunkBF16, uint16_t>(a, group, stream);
    return launch_group<ChunkF32, float>(a, group, stream);
}

int decode_stream_blocks_per_cu(int dtype, int group, int waves_per_group, int num_seqs) {
#if PA_DECODE_MFMA_FROM <= 1
    if (dtype == 3) return stream_blocks_group<ChunkBF16, uint16_t, false, true>(group, waves_per_group, num_seqs);
    if (dtype == 5) return stream_blocks_group<ChunkBF16, uint16_t, true, true>(group, waves_per_group, num_seqs);
    if (dtype == 6)
        return stream_blocks_group<ChunkBF16, uint16_t, true, true, true>(group, waves_per_group, num_seqs);
#else
    if (dtype == 3) return stream_blocks_group<ChunkBF16, uint16_t>(group, waves_per_group, num_seqs);
    if (dtype == 5) return stream_blocks_group<ChunkBF16, uint16_t, true>(group, waves_per_group, num_seqs);
    if (dtype == 6) return stream_blocks_group<ChunkBF16, uint16_t, true, false, true>(group, waves_per_group, num_seqs);
#endif
    if (dtype == 4) return stream_blocks_group<ChunkBF16, uint16_t, true, false, true>(group, waves_per_group, num_seqs);
    if (dtype == 2) return stream_blocks_group<ChunkBF16, uint16_t, true>(group, waves_per_group, num_seqs);
    if (dtype == 1) return stream_blocks_group<ChunkBF16, uint16_t>(group, waves_per_group, num_seqs);
    return stream_blocks_group<ChunkF32, float>(group, waves_per_group, num_seqs);
}

}  // namespace pa
