// Chunked-prefill attention for gfx950 on the matrix cores (MFMA).
//
// What is computed follows "AI Infra入门干货总结：大模型是如何高效推理的",
// section "Attention (FlashAttention, Scaled Dot-Product Attention)": for a
// request whose query_len rows are the last query_len positions of its
// seq_len tokens (cu_seqlens isolate requests of the flattened batch),
//   out = softmax(scale * Q K^T + M) V,  kv_head = q_head / (num_heads / num_kv_heads),
// K and V read from the paged cache through block_table, and M the causal mask
// (query row j sits at position seq_len - query_len + j and sees keys up to it).
// The online softmax (running max and sum, rescaled by 2^(m_old - m_new)) fuses
// the steps so that scores never leave the chip.
//
// Work decomposition:
//   * A workgroup owns 256 query rows of one (sequence, KV head): rows are
//     (token, grouped head) pairs, token-major, so G = num_heads/num_kv_heads
//     heads share every K/V tile and a tile spans 256/G tokens.  8 waves own
//     32 rows each (two 16-row MFMA tiles).
//   * K/V advance in tiles of 64 keys (4 cache blocks), double-buffered in LDS:
//     K row-major with a padded row (conflict-free 16-byte operand reads), V
//     transposed (dims x keys), as the P.V contraction runs over keys.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = the
//     wave's query rows held in registers): each lane's accumulator then holds
//     4 keys of ONE query row, which is exactly the lane layout of the B
//     operand of the next product, so the probabilities feed O^T += V^T P^T
//     without another pass through LDS.
//   * P is fed as two bf16 operands, hi = bf16(p) and lo = bf16(p - hi), so the
//     product keeps ~16 bits of p: a single bf16 rounding of p alone would use
//     most of the output's error budget on top of the bf16 output rounding.
//   * Causal masking selects -inf only on tiles that cross a row's limit; keys
//     past seq_len are zero-filled in LDS (stale cache slots may hold NaN, and
//     0 * NaN is NaN), and tiles wholly past a wave's rows are skipped.
//   * Workgroups are numbered heaviest tile first (later tiles of a chunk see
//     more keys), with the KV head as the fastest index, so the tiles of one
//     KV head land on one XCD and share its L2.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kRowsPerWave = 32;
static_assert(kWaves * kRowsPerWave == kPrefillRows, "tile rows");
constexpr int kKeys = 64;                    // keys per K/V tile
constexpr int kKStride = kHeadDim + 8;       // bf16 per K row in LDS (272 B)
constexpr int kVStride = kKeys + 4;          // bf16 per V^T row in LDS (136 B)
constexpr int kKTileElems = kKeys * kKStride;
constexpr int kVTileElems = kHeadDim * kVStride;
constexpr int kThreads = kWaves * kWave;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// hi/lo bf16 pair of a probability: hi = bf16(p), lo = bf16(p - hi).
__device__ __forceinline__ void split_bf16(float p, uint16_t& hi, uint16_t& lo) {
    const __bf16 h = (__bf16)p;
    hi = __builtin_bit_cast(uint16_t, h);
    lo = bf16_bits(p - (float)h);
}

// Prefix over sequences of the number of query tiles each needs (sequences with
// fewer than two query rows need none), in s_pref[0..B].
__device__ __forceinline__ void tile_prefix(const PrefillArgs& a, int tq, int32_t* s_pref, int32_t* s_wsum) {
    const int B = a.num_seqs;
    const int tid = threadIdx.x;
    const int per = (B + kThreads - 1) / kThreads;
    const int lo = min(tid * per, B), hi = min(lo + per, B);
    int sum = 0;
    for (int i = lo; i < hi; ++i) {
        const int q = a.cu_query_lens[i + 1] - a.cu_query_lens[i];
        const int n = q >= 2 ? (q + tq - 1) / tq : 0;
        s_pref[i + 1] = n;
        sum += n;
    }
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

template <int G>
__global__ void __launch_bounds__(kThreads)
prefill_kernel(PrefillArgs a) {
    constexpr int TQ = kPrefillRows / G;               // tokens per tile
    extern __shared__ __attribute__((aligned(16))) int32_t s_pref[];      // [num_seqs + 1]
    __shared__ int32_t s_wsum[kWaves];
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kKTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][kVTileElems];

    tile_prefix(a, TQ, s_pref, s_wsum);
    const int B = a.num_seqs;
    const int Hkv = a.num_kv_heads;
    const int T = s_pref[B];
    const int kvh = (int)(blockIdx.x % Hkv);
    const int t_rev = (int)(blockIdx.x / Hkv);
    if (t_rev >= T) return;                            // whole workgroup: no barrier is left behind
    const int t = T - 1 - t_rev;
    int lo = 0, hi = B - 1;                            // the largest b with s_pref[b] <= t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int tile = t - s_pref[b];
    const int q0 = a.cu_query_lens[b];
    const int qlen = a.cu_query_lens[b + 1] - q0;
    const int L = max(min(a.seq_lens[b], a.bt_stride * kBlock), 0);
    const int tok_begin = tile * TQ;
    const int ntok = min(TQ, qlen - tok_begin);
    const int prior = L - qlen;                        // position of query row 0
    const int kend_wg = a.causal ? max(min(L, prior + tok_begin + ntok), 0) : L;
    const int nkt = (kend_wg + kKeys - 1) / kKeys;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 15;                          // MFMA row/column within a 16-tile
    const int g = lane >> 4;                           // lane group
    const int Hq = a.num_heads;

    // ---- this lane's two query rows (one per 16-row tile) and their key limits
    int tq[2], kend[2];
    bool active[2];
    u32x4_t qop[2][4];                                 // B operand of S^T: dims 32ks + 8g .. +8
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int r = wave * kRowsPerWave + 16 * n + lr;
        tq[n] = r / G;
        active[n] = tq[n] < ntok;
        const int pos = prior + tok_begin + tq[n];
        kend[n] = !active[n] ? 0 : (a.causal ? max(min(L, pos + 1), 0) : L);
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.query) +
                             (int64_t)(q0 + tok_begin + (active[n] ? tq[n] : 0)) * a.q_stride +
                             (int64_t)(kvh * G + r % G) * kHeadDim + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qop[n][ks] = active[n] ? *reinterpret_cast<const u32x4_t*>(qp + 32 * ks) : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    // wave-wide key limits: tiles at or past kmax are skipped, tiles ending past
    // kmin need the mask
    int kmin = min(kend[0], kend[1]), kmax = max(kend[0], kend[1]);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        kmin = min(kmin, __shfl_xor(kmin, d, kWave));
        kmax = max(kmax, __shfl_xor(kmax, d, kWave));
    }

    float m[2] = {-INFINITY, -INFINITY};
    float lp[2] = {0.f, 0.f};                          // this lane's part of each row's sum
    f32x4_t oacc[8][2];                                // O^T: dims 16dt + 4g + r, row 16n + lr
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int n = 0; n < 2; ++n) oacc[dt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- K/V tile staging: 1024 16-byte chunks per tensor, two per thread
    const char* kc = reinterpret_cast<const char*>(a.key_cache);
    const char* vc = reinterpret_cast<const char*>(a.value_cache);
    const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
    const int64_t tok_bytes = (int64_t)Hkv * kHeadDim * 2;
    u32x4_t kreg[2], vreg[2];
    auto stage = [&](int kt) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = tid + j * kThreads;
            const int key = kt * kKeys + (c >> 4);
            const int part = c & 15;
            if (key < kend_wg) {
                const int64_t phys = min(max((int64_t)bt[key / kBlock], (int64_t)0), a.num_blocks - 1);
                const int64_t off = (phys * kBlock + key % kBlock) * tok_bytes + (int64_t)kvh * kHeadDim * 2 + part * 16;
                kreg[j] = *reinterpret_cast<const u32x4_t*>(kc + off);
                vreg[j] = *reinterpret_cast<const u32x4_t*>(vc + off);
            } else {
                kreg[j] = u32x4_t{0u, 0u, 0u, 0u};         // past the keys: zeros, never stale data
                vreg[j] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = tid + j * kThreads;
            const int key = c >> 4, part = c & 15;
            *reinterpret_cast<u32x4_t*>(&k_lds[buf][key * kKStride + part * 8]) = kreg[j];
            uint16_t* vt = &v_lds[buf][(part * 8) * kVStride + key];
            const u32x4_t w = vreg[j];
            vt[0 * kVStride] = (uint16_t)(w.x & 0xffffu);
            vt[1 * kVStride] = (uint16_t)(w.x >> 16);
            vt[2 * kVStride] = (uint16_t)(w.y & 0xffffu);
            vt[3 * kVStride] = (uint16_t)(w.y >> 16);
            vt[4 * kVStride] = (uint16_t)(w.z & 0xffffu);
            vt[5 * kVStride] = (uint16_t)(w.z >> 16);
            vt[6 * kVStride] = (uint16_t)(w.w & 0xffffu);
            vt[7 * kVStride] = (uint16_t)(w.w >> 16);
        }
    };

    if (nkt > 0) {
        stage(0);
        commit(0);
    }
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) stage(kt + 1);
        const int key0 = kt * kKeys;
        if (key0 < kmax) {
            // S^T = K Q^T over this tile: 4 key tiles x 2 row tiles x 4 dim steps
            f32x4_t sacc[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int n = 0; n < 2; ++n) sacc[mt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const uint16_t* kl = &k_lds[buf][lr * kKStride + 8 * g];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(kl + mt * 16 * kKStride + 32 * ks);
#pragma unroll
                    for (int n = 0; n < 2; ++n)
                        sacc[mt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), as_bf16x8(qop[n][ks]),
                                                                              sacc[mt][n], 0, 0, 0);
                }
            }

            // online softmax per row; lane holds keys 16mt + 4g + r of row 16n + lr
            const bool masked = key0 + kKeys > kmin;
            u32x4_t phi[2][2], plo[2][2];              // B operands of P^T: [row tile][key step]
            bool rescale = false;
            float alpha[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                float s[4][4];
                float mx = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float v = sacc[mt][n][r] * a.scale_log2;
                        if (masked && key0 + 16 * mt + 4 * g + r >= kend[n]) v = -INFINITY;
                        s[mt][r] = v;
                        mx = fmaxf(mx, v);
                    }
                mx = fmaxf(mx, shfl_xor_f(mx, 16));
                mx = fmaxf(mx, shfl_xor_f(mx, 32));
                const float mn = fmaxf(m[n], mx);
                const bool none = mn == -INFINITY;     // nothing visible yet in this row
                alpha[n] = none ? 1.f : __builtin_amdgcn_exp2f(m[n] - mn);
                rescale |= alpha[n] != 1.f;
                m[n] = mn;
                float sum = 0.f;
                uint16_t hb[4][4], lb[4][4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p = none ? 0.f : __builtin_amdgcn_exp2f(s[mt][r] - mn);
                        sum += p;
                        split_bf16(p, hb[mt][r], lb[mt][r]);
                    }
                lp[n] = lp[n] * alpha[n] + sum;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    // key slots: 4 keys of tile 2ks, then 4 keys of tile 2ks+1
                    phi[n][ks] = u32x4_t{(uint32_t)hb[2 * ks][0] | ((uint32_t)hb[2 * ks][1] << 16),
                                         (uint32_t)hb[2 * ks][2] | ((uint32_t)hb[2 * ks][3] << 16),
                                         (uint32_t)hb[2 * ks + 1][0] | ((uint32_t)hb[2 * ks + 1][1] << 16),
                                         (uint32_t)hb[2 * ks + 1][2] | ((uint32_t)hb[2 * ks + 1][3] << 16)};
                    plo[n][ks] = u32x4_t{(uint32_t)lb[2 * ks][0] | ((uint32_t)lb[2 * ks][1] << 16),
                                         (uint32_t)lb[2 * ks][2] | ((uint32_t)lb[2 * ks][3] << 16),
                                         (uint32_t)lb[2 * ks + 1][0] | ((uint32_t)lb[2 * ks + 1][1] << 16),
                                         (uint32_t)lb[2 * ks + 1][2] | ((uint32_t)lb[2 * ks + 1][3] << 16)};
                }
            }
            if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                    for (int n = 0; n < 2; ++n) oacc[dt][n] *= alpha[n];
            }

            // O^T += V^T P^T: 8 dim tiles x 2 key steps, hi and lo parts of P
            const uint16_t* vl = &v_lds[buf][lr * kVStride + 4 * g];
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const uint16_t* vrow = vl + dt * 16 * kVStride + 32 * ks;
                    const u32x2_t v0 = *reinterpret_cast<const u32x2_t*>(vrow);
                    const u32x2_t v1 = *reinterpret_cast<const u32x2_t*>(vrow + 16);
                    const u32x4_t va = u32x4_t{v0.x, v0.y, v1.x, v1.y};
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        oacc[dt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(phi[n][ks]),
                                                                              oacc[dt][n], 0, 0, 0);
                        oacc[dt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(plo[n][ks]),
                                                                              oacc[dt][n], 0, 0, 0);
                    }
                }
            }
        }
        if (kt + 1 < nkt) commit(buf ^ 1);
        __syncthreads();
    }

    // ---- normalise and store: lane holds dims 16dt + 4g .. +4 of row 16n + lr
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        float l = lp[n];
        l += shfl_xor_f(l, 16);
        l += shfl_xor_f(l, 32);
        if (!active[n]) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int r = wave * kRowsPerWave + 16 * n + lr;
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + (int64_t)(q0 + tok_begin + tq[n]) * Hq * kHeadDim +
                      (int64_t)(kvh * G + r % G) * kHeadDim + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const f32x4_t v = oacc[dt][n];
            *reinterpret_cast<u32x2_t*>(o + 16 * dt) =
                u32x2_t{pack_bf16x2(v.x * inv, v.y * inv), pack_bf16x2(v.z * inv, v.w * inv)};
        }
    }
}

template <int G>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
    const size_t lds = sizeof(int32_t) * ((size_t)a.num_seqs + 1);
    const int64_t grid = (int64_t)a.tiles_bound * a.num_kv_heads;
    hipLaunchKernelGGL((prefill_kernel<G>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_typed<1>(a, stream);
        case 2: return launch_typed<2>(a, stream);
        case 4: return launch_typed<4>(a, stream);
        case 8: return launch_typed<8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
