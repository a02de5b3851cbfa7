// Paged decode attention for gfx950: one query token per sequence against its
// paged K/V, with the online softmax and a split of long contexts into
// partitions merged by log-sum-exp weights.
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
// Work decomposition (one wavefront = one (sequence, kv head, partition)):
//   * The G query heads of a KV head share every K/V row the wave loads, so
//     each cache byte is read once per call.
//   * A 16-token block of one KV head is 16 rows of 256 B (bf16), 2 KiB apart.
//     Two lane layouts read it with 16-byte loads:
//       K layout: lane = 4*t + c holds token t, dims {32j + 8c .. +8 : j<4}; a
//         quad of lanes covers one row, so <q_h, k_t> needs a 2-step quad
//         reduction only;
//       V layout: lane = 16*g + d holds dims 8d .. 8d+7 of tokens 4g .. 4g+3;
//         every load instruction covers 4 whole rows, and each lane's running
//         output is G x 8 fp32 values that need no exchange until the end.
//     The probabilities move from the K layout to the V layout through 64
//     floats of LDS per wave.
//   * The running max is shared by the whole wave per head; a wave-uniform
//     branch skips the max reduction and the rescale unless some score of the
//     block exceeds it.  Exponentials are base 2 with log2(e) folded into the
//     scale.
//   * Block ids are loaded once per 64 blocks (one per lane) and broadcast with
//     v_readlane; K/V loads of block i+1 are in flight while block i is used.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kWavesPerGroup = 4;

template <typename Chunk, typename Elem, int G, bool NT>
__global__ void __launch_bounds__(256)
decode_kernel(DecodeArgs a) {
    constexpr int D = kHeadDim;
    constexpr int NSEL = (G + 3) / 4;          // heads whose probability a K-layout lane produces
    constexpr int EPC = 8;                     // elements per chunk
    __shared__ __attribute__((aligned(16))) float p_lds[kWavesPerGroup][kBlock * G];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int Hkv = a.num_kv_heads;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerGroup + wave;
    const int kvh = (int)(item % Hkv);
    const int64_t rest = item / Hkv;
    const int part = (int)(rest % a.max_partitions);
    const int64_t b = rest / a.max_partitions;
    if (b >= a.num_seqs) return;
    // Lengths beyond the block table's row are cut to it, so that no table entry
    // outside the row is read even when seq_lens breaks the contract.
    const int L = min(a.seq_lens[b], a.bt_stride * kBlock);
    const int PT = a.partition_tokens;
    const int nparts = L <= 0 ? 1 : min((L + PT - 1) / PT, a.max_partitions);
    if (part >= nparts) return;
    const int tok_begin = part * PT;
    const int tok_end = min(L, tok_begin + PT);
    const int nblk = tok_end > tok_begin ? (tok_end - tok_begin + kBlock - 1) / kBlock : 0;

    const int64_t tok_stride = (int64_t)Hkv * D;                 // elements between tokens of a block
    const int64_t blk_stride = tok_stride * kBlock;              // elements between physical blocks

    // K layout
    const int t = lane >> 2;
    const int c = lane & 3;
    const uint32_t koff = (uint32_t)((t * tok_stride + (int64_t)kvh * D + c * EPC) * sizeof(Elem));
    // V layout
    const int g = lane >> 4;
    const int dch = lane & 15;
    const uint32_t voff = (uint32_t)((4 * g * tok_stride + (int64_t)kvh * D + dch * EPC) * sizeof(Elem));
    const uint32_t vrow = (uint32_t)(tok_stride * sizeof(Elem));

    // Query of the G heads sharing this KV head, in the K layout.
    Chunk q[G][4];
    {
        const Elem* qp = reinterpret_cast<const Elem*>(a.query) + b * a.q_stride + (int64_t)kvh * G * D;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) load_chunk<false>(q[h][j], qp + h * D + j * 32 + c * EPC);
    }

    float m[NSEL], l[NSEL];
#pragma unroll
    for (int r = 0; r < NSEL; ++r) { m[r] = -INFINITY; l[r] = 0.f; }
    float acc[G][EPC];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;

    const char* kc = reinterpret_cast<const char*>(a.key_cache);
    const char* vc = reinterpret_cast<const char*>(a.value_cache);
    const int32_t* bt = a.block_table + b * a.bt_stride + tok_begin / kBlock;
    float* pl = p_lds[wave];

    for (int cb = 0; cb < nblk; cb += kWave) {
        const int nb = min(kWave, nblk - cb);
        const int bid = lane < nb ? bt[cb + lane] : 0;

        auto issue = [&](Chunk (&kb)[4], Chunk (&vb)[4], int i) {
            // an id outside the pool (a caller error) is clamped into it: wrong
            // values, but no access outside the cache
            const int64_t phys = min(max((int64_t)__builtin_amdgcn_readlane(bid, i), (int64_t)0),
                                     a.num_blocks - 1);
            const char* kbase = kc + phys * blk_stride * (int64_t)sizeof(Elem);
            const char* vbase = vc + phys * blk_stride * (int64_t)sizeof(Elem);
#pragma unroll
            for (int j = 0; j < 4; ++j) load_chunk<NT>(kb[j], kbase + koff + j * 32 * sizeof(Elem));
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) load_chunk<NT>(vb[i4], vbase + voff + i4 * vrow);
        };

        auto process = [&](const Chunk (&kb)[4], const Chunk (&vb)[4], int i) {
            const int tok0 = tok_begin + (cb + i) * kBlock;
            const bool tail = tok0 + kBlock > tok_end;

            // scores of token t for every head of the group (quad reduction)
            float s[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float x = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) x = dot_chunk(q[h][j], kb[j], x);
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
            for (int r = 0; r < NSEL; ++r) grow |= ss[r] > m[r];
            if (__builtin_amdgcn_ballot_w64(grow)) {
                float alpha[NSEL];
#pragma unroll
                for (int r = 0; r < NSEL; ++r) {
                    float bm = ss[r];
                    bm = fmaxf(bm, dpp<kRowRor4>(bm));
                    bm = fmaxf(bm, dpp<kRowRor8>(bm));
                    bm = fmaxf(bm, shfl_xor_f(bm, 16));
                    bm = fmaxf(bm, shfl_xor_f(bm, 32));
                    const float mn = fmaxf(m[r], bm);
                    alpha[r] = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[r] - mn);
                    l[r] *= alpha[r];
                    m[r] = mn;
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float ah = readlane_f(alpha[h / 4], h % 4);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc[h][e] *= ah;
                }
            }

#pragma unroll
            for (int r = 0; r < NSEL; ++r) {
                if (c + 4 * r < G) {
                    const float p = __builtin_amdgcn_exp2f(ss[r] - m[r]);
                    l[r] += p;
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
                    for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(pr[h], vf[e], acc[h][e]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };

        Chunk ka[4], va[4], kb2[4], vb2[4];
        issue(ka, va, 0);
        int i = 0;
        for (; i + 1 < nb; i += 2) {
            issue(kb2, vb2, i + 1);
            process(ka, va, i);
            if (i + 2 < nb) issue(ka, va, i + 2);
            process(kb2, vb2, i + 1);
        }
        if (i < nb) process(ka, va, i);
    }

    // ---- epilogue: combine the per-lane partial sums
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            acc[h][e] += shfl_xor_f(acc[h][e], 16);
            acc[h][e] += shfl_xor_f(acc[h][e], 32);
        }
#pragma unroll
    for (int r = 0; r < NSEL; ++r) {
        l[r] += dpp<kRowRor4>(l[r]);
        l[r] += dpp<kRowRor8>(l[r]);
        l[r] += shfl_xor_f(l[r], 16);
        l[r] += shfl_xor_f(l[r], 32);
    }
    float lh[G], mh[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        lh[h] = readlane_f(l[h / 4], h % 4);
        mh[h] = readlane_f(m[h / 4], h % 4);
    }

    if (g == 0) {
        const int Hq = a.num_heads;
        if (nparts == 1) {
            Elem* o = reinterpret_cast<Elem*>(a.out) + (b * Hq + (int64_t)kvh * G) * D + dch * EPC;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = lh[h] > 0.f ? 1.f / lh[h] : 0.f;
                float f[EPC];
#pragma unroll
                for (int e = 0; e < EPC; ++e) f[e] = acc[h][e] * inv;
                store_chunk(o + h * D, f);
            }
        } else {
            const int P = a.max_partitions;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const int64_t slot = (b * Hq + (int64_t)kvh * G + h) * P + part;
                store_chunk(a.part_acc + slot * D + dch * EPC, acc[h]);
                if (dch == h) *reinterpret_cast<float2*>(a.part_ml + slot * 2) = make_float2(mh[h], lh[h]);
            }
        }
    }
}

// Log-sum-exp merge of the partitions of every (sequence, head) that was split:
// with M = max_p m_p, out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
// One wave per (sequence, head), two dims per lane.
template <typename Elem>
__global__ void __launch_bounds__(256)
merge_kernel(DecodeArgs a) {
    constexpr int D = kHeadDim;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int Hq = a.num_heads;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerGroup + wave;
    const int64_t b = item / Hq;
    const int h = (int)(item % Hq);
    if (b >= a.num_seqs) return;
    const int L = min(a.seq_lens[b], a.bt_stride * kBlock);
    const int PT = a.partition_tokens;
    const int nparts = L <= 0 ? 1 : min((L + PT - 1) / PT, a.max_partitions);
    if (nparts <= 1) return;
    const int P = a.max_partitions;
    const int64_t base = (b * Hq + h) * P;
    const float* ml = a.part_ml + base * 2;
    float M = -INFINITY;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
    float lsum = 0.f, o0 = 0.f, o1 = 0.f;
    const float* pa = a.part_acc + base * D + 2 * lane;
    for (int p = 0; p < nparts; ++p) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * p] - M);
        lsum = fmaf(w, ml[2 * p + 1], lsum);
        const float2 v = *reinterpret_cast<const float2*>(pa + (int64_t)p * D);
        o0 = fmaf(w, v.x, o0);
        o1 = fmaf(w, v.y, o1);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    Elem* o = reinterpret_cast<Elem*>(a.out) + (b * Hq + h) * D + 2 * lane;
    if constexpr (sizeof(Elem) == 2) {
        *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(o0 * inv, o1 * inv);
    } else {
        *reinterpret_cast<float2*>(o) = make_float2(o0 * inv, o1 * inv);
    }
}

template <typename Chunk, typename Elem, int G>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    const int64_t items = (int64_t)a.num_seqs * a.max_partitions * a.num_kv_heads;
    const int64_t grid = (items + kWavesPerGroup - 1) / kWavesPerGroup;
    hipLaunchKernelGGL((decode_kernel<Chunk, Elem, G, true>), dim3((unsigned)grid), dim3(256), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_partitions <= 1) return e;
    const int64_t mitems = (int64_t)a.num_seqs * a.num_heads;
    hipLaunchKernelGGL((merge_kernel<Elem>), dim3((unsigned)((mitems + kWavesPerGroup - 1) / kWavesPerGroup)),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename Chunk, typename Elem>
hipError_t launch_group(const DecodeArgs& a, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_typed<Chunk, Elem, 1>(a, stream);
        case 2: return launch_typed<Chunk, Elem, 2>(a, stream);
        case 4: return launch_typed<Chunk, Elem, 4>(a, stream);
        case 8: return launch_typed<Chunk, Elem, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, int group, hipStream_t stream) {
    if (dtype == 1) return launch_group<ChunkBF16, uint16_t>(a, group, stream);
    return launch_group<ChunkF32, float>(a, group, stream);
}

}  // namespace pa
