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
//     32 rows each, one 32-row MFMA tile.
//   * K/V advance in tiles of 64 keys (4 cache blocks), double-buffered in LDS:
//     K row-major with a padded row (conflict-free 16-byte operand reads), V
//     transposed (dims x keys), as the P.V contraction runs over keys, with the
//     keys of each 16-key group ordered so that an operand is one 16-byte read.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
//     wave's query rows held in registers): lane l then holds query row l % 32
//     and 16 of the tile's 32 keys per key tile, the lane pair (l, l ^ 32)
//     covering the row, so row maxima and sums take one lane swap.  Eight of
//     those scores form, in registers, the B operand of one 16-key step of
//     O^T += V^T P^T (the V^T operand follows the same key order), so P never
//     goes through LDS.  32x32x16 products sustain the matrix rate with one or
//     two independent accumulators per wave, where 16x16x32 products need
//     twelve or more (measured on MI355X).
//   * P.V runs in fp16 (v_mfma_f32_32x32x16_f16): V^T is staged to LDS as
//     fp16, exact for bf16 magnitudes below 2^16, and p in [0, 1] is rounded
//     once to fp16 (11 significant bits, subnormals kept).  A single bf16
//     rounding of p would use most of the output's error budget on top of the
//     bf16 output rounding.  A workgroup that stages a V magnitude of 2^16 or
//     more redoes its segment on an exact bf16 path that feeds P as two
//     operands, hi = p truncated to bf16 and lo = bf16(p - hi) (~16 bits of
//     p, twice the P.V products).
//   * Causal masking selects -inf only on tiles that cross a row's limit; keys
//     past seq_len are zero-filled in LDS (stale cache slots may hold NaN, and
//     0 * NaN is NaN).
//   * Work is balanced over the resident workgroups: the units of one KV
//     head are its (query tile, 64-key tile) pairs in (sequence, tile, key
//     tile) order, and each of the slots_per_kvh workgroups of a KV head takes
//     a contiguous share of them, one segment per query tile it touches.  The
//     shares are equal in a cost that adds a fixed set-up charge per query
//     tile to its key tiles, so that a workgroup whose share spans many short
//     tiles takes fewer units.  A tile inside one share writes its rows; the
//     segments of a tile that crosses a share boundary leave (max, sum,
//     unnormalised output) records per row, merged by a second kernel
//     (log-sum-exp weights, the same merge as split decode) over a compact
//     list of those tiles (slot: such tiles before it).
//   * The KV head is the fastest index of the workgroup number, so the shares
//     of one KV head land on one XCD and share its L2.
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = kPrefillWaves;
constexpr int kRowsPerWave = 32;
static_assert(kWaves * kRowsPerWave == kPrefillRows, "tile rows");
constexpr int kKeys = 64;                    // keys per K/V tile
constexpr int kKStride = kHeadDim + 8;       // bf16 per K row in LDS (272 B)
constexpr int kVStride = kKeys + 8;          // bf16 per V^T row in LDS (144 B)
constexpr int kKTileElems = kKeys * kKStride;
constexpr int kVTileElems = kHeadDim * kVStride;
constexpr int kThreads = kWaves * kWave;
// Thread groups of 256: each stages one 16-token block of a K/V tile per step,
// so every thread stages kBlkPerThr of the tile's 4 blocks.
constexpr int kThrGroups = kThreads / 256;
constexpr int kBlkPerThr = 4 / kThrGroups;
// V staging: a tile's 4 blocks x 2 quad pairs (quads 0 and 2, or 1 and 3, of a
// block) over the waves, kVPerThr of them per thread.
constexpr int kVPerThr = 8 / kWaves;
// Sets of staging registers.  With one (the default), a tile's loads are issued
// as the tile before it starts and committed at its end, a whole tile of
// compute later.  With two (8-wave workgroups only, a build parameter kept for
// measurement), they are issued two tiles before their commit; that costs 18
// more VGPRs and measured no faster once every wait covers only the loads it
// needs.
#ifndef PA_PREFILL_STAGE_SETS
#define PA_PREFILL_STAGE_SETS 1
#endif

constexpr int kStageSets = kThrGroups == 2 ? PA_PREFILL_STAGE_SETS : 1;
static_assert(kStageSets == 1 || kStageSets == 2, "staging sets");
// Merge workgroups per listed tile: one per wave block of 32 rows.
constexpr int kMergeParts = kPrefillRows / kRowsPerWave;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }
__device__ __forceinline__ f16x8_t as_f16x8(u32x4_t w) { return __builtin_bit_cast(f16x8_t, w); }

// Two fp32 -> two fp16 in one word (lo in bits 0-15), round to nearest even:
// one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}

constexpr int kRec = 132;                    // record floats per row: 128 O, max, sum, 2 unused
// A record's format flag (0: fp16 normalised rows, 1: fp32 unnormalised rows),
// after its (max, sum) pairs.
constexpr int kRecFlag = kPrefillRows * (kHeadDim + 2);
constexpr uint32_t kRsrcWord3 = 0x00020000u; // raw buffer, 32-bit data format
constexpr float kSlack = 8.f;                // log2 headroom of the softmax reference max

// Between the two 32-lane halves of the wave (lanes l and l ^ 32):
// permlane32_swap(x, x) returns each half broadcast to both.
__device__ __forceinline__ float max_across_halves(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return maximum(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Exclusive prefix over the workgroup's threads of `x` (every thread calls).
__device__ __forceinline__ int block_exclusive_scan(int x, int32_t* s_wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int y = x;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(y, d, kWave);
        if (lane >= d) y += t;
    }
    __syncthreads();                                   // s_wsum free from any earlier use
    if (lane == kWave - 1) s_wsum[wave] = y;
    __syncthreads();
    int before = y - x;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
    return before;
}

struct SeqShape {
    int q0, qlen, L;
};

// The same shape held in scalar registers (for a sequence index that is the
// same for the whole workgroup).
__device__ __forceinline__ SeqShape uniform(SeqShape sh) {
    sh.q0 = __builtin_amdgcn_readfirstlane(sh.q0);
    sh.qlen = __builtin_amdgcn_readfirstlane(sh.qlen);
    sh.L = __builtin_amdgcn_readfirstlane(sh.L);
    return sh;
}

__device__ __forceinline__ SeqShape seq_shape(const PrefillArgs& a, int b) {
    SeqShape sh;
    sh.q0 = a.cu_query_lens[b];
    sh.qlen = a.cu_query_lens[b + 1] - sh.q0;
    sh.L = max(min(a.seq_lens[b], a.bt_stride * kBlock), 0);
    return sh;
}

__device__ __forceinline__ int tiles_of(const SeqShape& sh, int tq) {
    return sh.qlen >= 2 ? (sh.qlen + tq - 1) / tq : 0;
}

// Key limit of query tile t (one past the last key any of its rows sees).
__device__ __forceinline__ int tile_kend(const PrefillArgs& a, const SeqShape& sh, int t, int tq) {
    if (!a.causal) return sh.L;
    const int last = min(sh.qlen, (t + 1) * tq);         // rows t*tq .. last-1
    return max(min(sh.L - sh.qlen + last, sh.L), 0);
}

// Work units of query tile t: its key tiles, and at least one, since a tile
// that sees no key still writes its (zero) rows.
__device__ __forceinline__ int tile_units(const PrefillArgs& a, const SeqShape& sh, int t, int tq) {
    return max(1, (tile_kend(a, sh, t, tq) + kKeys - 1) / kKeys);
}

// Set-up and finish of a segment (its query rows, the first tile's K/V round
// trip, the output or record writes, two barriers), in key-tile units: about
// two tiles' time, measured per workgroup on MI355X.
#ifndef PA_PREFILL_SEGMENT_UNITS
#define PA_PREFILL_SEGMENT_UNITS 2
#endif
constexpr int kSegUnits = PA_PREFILL_SEGMENT_UNITS;

// The slot whose share holds unit x: the largest s < slots with bnd[s] <= x
// (bnd[0] = 0 <= x).
__device__ __forceinline__ int slot_of(const int32_t* bnd, int slots, int x) {
    int lo = 0, hi = slots - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (bnd[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Does the tile of units [u0, u0 + n) cross a share boundary?
__device__ __forceinline__ bool cut(const int32_t* bnd, int slots, int u0, int n) {
    return slot_of(bnd, slots, u0) != slot_of(bnd, slots, u0 + n - 1);
}

// The batch's unit map, built by every workgroup.  Units are the (query tile,
// key tile) pairs of one KV head in (sequence, tile, key tile) order;
// s_pu[b] = first unit of sequence b (s_pu[B] = U).  The shares balance a
// cost in which each query tile also counts kSegUnits for its set-up and
// finish: the cost line is cut into slots_per_kvh shares of
// max(min_share, ceil(C / slots_per_kvh)), and a cut that falls in a tile's
// set-up moves to the tile's first unit, so that the tile stays whole.
// s_bnd[s] = first unit of slot s's share (s_bnd[slots_per_kvh] = U; trailing
// shares may be empty).  s_sp[b] = tiles before sequence b that cross a share
// boundary (s_sp[B] = total).
__device__ __forceinline__ void build_unit_map(const PrefillArgs& a, int tq, int32_t* s_pu, int32_t* s_sp,
                                               int32_t* s_bnd, int32_t* s_wsum) {
    const int B = a.num_seqs, slots = a.slots_per_kvh;
    const int nthr = blockDim.x;
    const int per = (B + nthr - 1) / nthr;
    const int lo = min((int)threadIdx.x * per, B), hi = min(lo + per, B);
    // units and query tiles per sequence; s_sp holds the tile prefix until the
    // boundaries are placed
    int units = 0, tiles = 0;
    for (int b = lo; b < hi; ++b) {
        const SeqShape sh = seq_shape(a, b);
        const int nt = tiles_of(sh, tq);
        int ub = 0;
        for (int t = 0; t < nt; ++t) ub += tile_units(a, sh, t, tq);
        s_pu[b + 1] = ub;
        s_sp[b + 1] = nt;
        units += ub;
        tiles += nt;
    }
    int run = block_exclusive_scan(units, s_wsum);
    int runt = block_exclusive_scan(tiles, s_wsum);
    for (int b = lo; b < hi; ++b) {
        run += s_pu[b + 1];
        s_pu[b + 1] = run;
        runt += s_sp[b + 1];
        s_sp[b + 1] = runt;
    }
    if (threadIdx.x == 0) s_pu[0] = s_sp[0] = 0;
    __syncthreads();
    const int U = s_pu[B];
    const int64_t C = (int64_t)U + (int64_t)kSegUnits * s_sp[B];
    const int64_t cs = max((int64_t)a.min_share, (C + slots - 1) / slots);
    for (int sl = threadIdx.x; sl <= slots; sl += nthr) {
        const int64_t x = (int64_t)sl * cs;
        int bnd = U;
        if (x < C) {
            // the sequence whose cost range holds x: the largest b with
            // s_pu[b] + kSegUnits * s_sp[b] <= x (it has tiles, as x < C)
            int l = 0, h = B - 1;
            while (l < h) {
                const int mid = (l + h + 1) >> 1;
                if ((int64_t)s_pu[mid] + (int64_t)kSegUnits * s_sp[mid] <= x) l = mid; else h = mid - 1;
            }
            const SeqShape sh = seq_shape(a, l);
            int64_t c = (int64_t)s_pu[l] + (int64_t)kSegUnits * s_sp[l];
            int u = s_pu[l];
            for (int t = 0, nt = tiles_of(sh, tq); t < nt; ++t) {
                const int n = tile_units(a, sh, t, tq);
                if (x < c + kSegUnits) { bnd = u; break; }
                if (x < c + kSegUnits + n) { bnd = u + (int)(x - c - kSegUnits); break; }
                c += kSegUnits + n;
                u += n;
            }
        }
        s_bnd[sl] = bnd;
    }
    __syncthreads();                                   // every read of the tile prefix is done
    int splits = 0;
    for (int b = lo; b < hi; ++b) {
        const SeqShape sh = seq_shape(a, b);
        int u = s_pu[b], sb = 0;
        for (int t = 0, nt = tiles_of(sh, tq); t < nt; ++t) {
            const int n = tile_units(a, sh, t, tq);
            sb += cut(s_bnd, slots, u, n);
            u += n;
        }
        s_sp[b + 1] = sb;
        splits += sb;
    }
    run = block_exclusive_scan(splits, s_wsum);
    for (int b = lo; b < hi; ++b) {
        run += s_sp[b + 1];
        s_sp[b + 1] = run;
    }
    __syncthreads();
}

// The largest b with pref[b] <= x (pref non-decreasing, pref[0] = 0 <= x).
__device__ __forceinline__ int find_seq(const int32_t* pref, int B, int x) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pref[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <int G>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
prefill_kernel(PrefillArgs a) {
    constexpr int TQ = kPrefillRows / G;               // tokens per tile
    extern __shared__ __attribute__((aligned(16))) int32_t s_dyn[];
    int32_t* s_pu = s_dyn;                             // [num_seqs + 1] unit prefix
    int32_t* s_sp = s_dyn + a.num_seqs + 1;            // [num_seqs + 1] split-tile prefix
    __shared__ int32_t s_wsum[kWaves];
    __shared__ int32_t s_bnd[kPrefillMaxSlots + 1];    // first unit of each slot's share
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kKTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][kVTileElems];

    build_unit_map(a, TQ, s_pu, s_sp, s_bnd, s_wsum);
    const int B = a.num_seqs;
    const int Hkv = a.num_kv_heads;
    const int slots = a.slots_per_kvh;
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.split_count = s_sp[B] * Hkv;
    const int kvh = (int)(blockIdx.x % Hkv);
    const int slot = (int)(blockIdx.x / Hkv);
    // values read from LDS are the same in every lane: kept in scalar registers
    const int ub = __builtin_amdgcn_readfirstlane(s_bnd[slot]);
    const int ue = __builtin_amdgcn_readfirstlane(s_bnd[slot + 1]);
    if (ub >= ue) return;                              // whole workgroup: no barrier is left behind

    // the tile holding unit ub
    int b = __builtin_amdgcn_readfirstlane(find_seq(s_pu, B, ub));
    SeqShape sh = uniform(seq_shape(a, b));
    int nt = tiles_of(sh, TQ), tile = 0;
    int tu0 = __builtin_amdgcn_readfirstlane(s_pu[b]);  // first unit of the tile
    int split_before = __builtin_amdgcn_readfirstlane(s_sp[b]);
    for (int n = tile_units(a, sh, 0, TQ); ub >= tu0 + n; n = tile_units(a, sh, tile, TQ)) {
        split_before += cut(s_bnd, slots, tu0, n);
        tu0 += n;
        ++tile;
    }

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 31;                          // MFMA row/column within a 32-tile
    const int h = lane >> 5;                           // lane half
    const int Hq = a.num_heads;

    // One segment per query tile the share touches: the key tiles of the
    // share that belong to that tile.
    for (int u = ub, first = 1;; first = 0) {
        const int units = tile_units(a, sh, tile, TQ);
        const int kend_wg = tile_kend(a, sh, tile, TQ);
        const int nkt = (kend_wg + kKeys - 1) / kKeys;
        const int kt_begin = u - tu0;
        const int seg_end = min(ue, tu0 + units) - tu0;
        const int kt_end = min(seg_end, nkt);
        const bool split = tu0 < ub || tu0 + units > ue; // the tile reaches past this share
        const int q0 = sh.q0, qlen = sh.qlen, L = sh.L;
        const int tok_begin = tile * TQ;
        const int ntok = min(TQ, qlen - tok_begin);
        const int prior = L - qlen;                        // position of query row 0

        // ---- this lane's query row and its key limit.  Lane l of the wave holds
        // row 32 * wave + l % 32; its two lanes (l, l ^ 32) each hold half of
        // every tile's keys (h = l / 32 selects which).
        const int r = wave * kRowsPerWave + lr;
        const int tq = r / G;
        const bool active = tq < ntok;
        const int kend = !active ? 0 : (a.causal ? max(min(L, prior + tok_begin + tq + 1), 0) : L);
        // wave-wide key limit: tiles ending past kmin need the mask.  (A tile
        // wholly past the wave's rows is still computed, its scores all masked:
        // skipping it would merge two versions of the accumulators at the join,
        // which costs register copies on every tile.)
        int kmin = kend;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) kmin = min(kmin, __shfl_xor(kmin, d, kWave));

        float m;
        float lp;                                          // this lane's part of the row's sum
        f32x16_t oacc[4];                                  // O^T: oacc[dt][4b + e] = dim 32dt + 8b + 4h + e

        // ---- K/V tile staging.  K: 1024 16-byte chunks (row, 16-byte part), two per
        // thread, stored row-major.  V^T: each 16-key group of a row (one cache
        // block) is stored as two 16-byte chunks, keys 0-3 and 8-11, then 4-7
        // and 12-15: the 8 keys that lane half h feeds to one P.V step (see
        // pv_products), so each operand is one 16-byte read, and rows 144 bytes
        // apart put the 16 rows such a read covers per cycle on all banks.
        // Thread (dim pair dp, wave w) loads, of block w / 2 (w / 2 and
        // w / 2 + 2 with 4 waves), the 4-byte (dims 2dp, 2dp+1) word of keys
        // 4q .. 4q + 3 and 4q + 8 .. 4q + 11 (q = w % 2) -- a wave reads whole
        // 256-byte rows -- and writes one chunk to each of its two V^T rows.  A
        // wave's loads of tile kt fall in a fixed set of cache blocks of the
        // tile, at offsets within the block that do not change from tile to
        // tile; each block is read through a buffer resource whose size is its
        // valid keys' rows, so that keys past the range read as zeros (never
        // stale data) without a branch or a per-lane test.
        const char* kc = reinterpret_cast<const char*>(a.key_cache);
        const char* vc = reinterpret_cast<const char*>(a.value_cache);
        const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
        const uint32_t tok_bytes = (uint32_t)Hkv * kHeadDim * 2;
        const int64_t blk_bytes = (int64_t)kBlock * tok_bytes;
        const uint32_t head_off = (uint32_t)kvh * kHeadDim * 2;
        const int dp = tid & 63, kq = tid >> 6;
        const int w4 = __builtin_amdgcn_readfirstlane(tid >> 8);   // the same for a whole wave
        const uint32_t koff = ((tid >> 4) & 15) * tok_bytes + head_off + (tid & 15) * 16;
        const int vq = kq & 1;                             // V quad pair, the same for a whole wave
        const uint32_t voff = 4 * vq * tok_bytes + head_off + dp * 4;
        auto v_block = [&](int jv) { return __builtin_amdgcn_readfirstlane((kq >> 1) + (kWaves / 2) * jv); };
        // staging registers, kStageSets sets of them (the set chosen at compile
        // time, see run)
        u32x4_t kreg[kStageSets][kBlkPerThr];
        uint32_t vw[kStageSets][kVPerThr][8];
        // Block ids, per staging set: bid[S] holds (lanes 0-3) the ids of the
        // next tile staged into set S, loaded when the set's previous tile was
        // staged, and broadcast with v_readlane, so that a tile's 10 loads issue
        // back to back.  Every load of the loop (ids and K/V) is issued
        // unconditionally -- tiles past the segment read through empty buffer
        // resources, which return zeros without touching memory -- so that the
        // number of loads issued after any one of them is the same on every
        // path, and each wait covers exactly the loads it needs.
        const int nblk_wg = (kend_wg + kBlock - 1) / kBlock;
        const rsrc_t rbt = __builtin_amdgcn_make_buffer_rsrc((void*)bt, (short)0, nblk_wg * 4, kRsrcWord3);
        int bid[kStageSets];
        auto load_ids = [&](int kt, auto set) {
            constexpr int S = decltype(set)::value;
            bid[S] = __builtin_amdgcn_raw_buffer_load_b32(rbt, (4 * kt + (lane & 3)) * 4, 0, 0);
        };
        // The segment's first block ids are loaded before the query rows, so
        // that the wait for them (before the first tile's K/V loads) does not
        // cover the query loads as well: the query latency then overlaps the
        // first tile's.
        using Set0 = std::integral_constant<int, 0>;
        using Set1 = std::integral_constant<int, 1>;
        load_ids(kt_begin, Set0{});
        __builtin_amdgcn_sched_barrier(0);
        // B operand of S^T, dim step ks: dims 16ks + 8h .. +8.  Loaded on every
        // path (a load under a branch leaves the wait counts unknown, and the
        // loop would then wait on every load in flight): an inactive row reads
        // the tile's first token, and its limit kend = 0 masks every score, so
        // its p are all 0.  The values are not otherwise touched before the
        // first product, so their wait falls there, behind the K/V prologue.
        u32x4_t qop[8];
        {
            const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.query) +
                                 (int64_t)(q0 + tok_begin + (active ? tq : 0)) * a.q_stride +
                                 (int64_t)(kvh * G + r % G) * kHeadDim + 8 * h;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) qop[ks] = *reinterpret_cast<const u32x4_t*>(qp + 16 * ks);
        }
        auto stage = [&](int kt, auto set) {
            constexpr int S = decltype(set)::value;
            const bool live = kt < kt_end;                 // wave-uniform
#pragma unroll
            for (int j = 0; j < kBlkPerThr; ++j) {
                const int blk = 4 * kt + w4 + kThrGroups * j;
                const int64_t id = __builtin_amdgcn_readlane(bid[S], w4 + kThrGroups * j);
                const int64_t off = min(max(id, (int64_t)0), a.num_blocks - 1) * blk_bytes;
                const int nrec = __builtin_amdgcn_readfirstlane(
                    live ? min(max(kend_wg - blk * kBlock, 0), kBlock) * (int)tok_bytes : 0);
                const rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + off), (short)0, nrec, kRsrcWord3);
                kreg[S][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)koff, 0, 0));
            }
#pragma unroll
            for (int jv = 0; jv < kVPerThr; ++jv) {
                const int vb = v_block(jv);
                const int blk = 4 * kt + vb;
                const int64_t id = __builtin_amdgcn_readlane(bid[S], vb);
                const int64_t off = min(max(id, (int64_t)0), a.num_blocks - 1) * blk_bytes;
                const int nrec = __builtin_amdgcn_readfirstlane(
                    live ? min(max(kend_wg - blk * kBlock, 0), kBlock) * (int)tok_bytes : 0);
                const rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + off), (short)0, nrec, kRsrcWord3);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    vw[S][jv][i] = __builtin_amdgcn_raw_buffer_load_b32(
                        rv, (int)(voff + ((i & 3) + 8 * (i >> 2)) * tok_bytes), 0, 0);
            }
        };
        // V^T goes to LDS as bf16 (exact path) or fp16 (fast path).  The fp16
        // copy is exact for every bf16 magnitude below 2^16 (fp16 subnormals
        // included, up to a rounding far below the output's); vmax tracks the
        // largest magnitude staged so that a workgroup that met a larger one
        // can redo its segment on the exact path.
        float vmax = 0.f;
        auto commit = [&](int kbuf, int vbuf, auto half, auto set) {
            constexpr bool kHalf = decltype(half)::value;
            constexpr int S = decltype(set)::value;
#pragma unroll
            for (int j = 0; j < kBlkPerThr; ++j) {
                const int c = tid + j * kThreads;
                *reinterpret_cast<u32x4_t*>(&k_lds[kbuf][(c >> 4) * kKStride + (c & 15) * 8]) = kreg[S][j];
            }
#pragma unroll
            for (int jv = 0; jv < kVPerThr; ++jv) {
                const uint32_t* w = vw[S][jv];
                u32x4_t even, odd;                         // V^T rows 2dp and 2dp + 1
                if constexpr (kHalf) {
                    float e[8], o[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        e[i] = bf16_lo(w[i]);
                        o[i] = bf16_hi(w[i]);
                        vmax = maximum(vmax, maximum(fabsf(e[i]), fabsf(o[i])));
                    }
                    even = u32x4_t{pack_f16x2(e[0], e[1]), pack_f16x2(e[2], e[3]), pack_f16x2(e[4], e[5]),
                                   pack_f16x2(e[6], e[7])};
                    odd = u32x4_t{pack_f16x2(o[0], o[1]), pack_f16x2(o[2], o[3]), pack_f16x2(o[4], o[5]),
                                  pack_f16x2(o[6], o[7])};
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        even[i] = (w[2 * i] & 0xffffu) | (w[2 * i + 1] << 16);
                        odd[i] = (w[2 * i] >> 16) | (w[2 * i + 1] & 0xffff0000u);
                    }
                }
                uint16_t* vt = &v_lds[vbuf][(2 * dp) * kVStride + 8 * (2 * v_block(jv) + vq)];
                *reinterpret_cast<u32x4_t*>(vt) = even;
                *reinterpret_cast<u32x4_t*>(vt + kVStride) = odd;
            }
        };

        // ---- the pieces of a key tile.
        // S^T = K Q^T over the tile in K buffer kbuf: 2 key tiles of 32 x 8 dim
        // steps of 16.  sacc[mt][4b + e] is the score of key 32mt + 8b + 4h + e.
        auto s_products = [&](int kbuf, f32x16_t (&sacc)[2]) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v) sacc[mt][v] = 0.f;
            // operands read one step ahead of the products that use them
            const uint16_t* kl = &k_lds[kbuf][lr * kKStride + 8 * h];
            auto k_operand = [&](int i) {                  // step i: dim step i / 2, key tile i % 2
                return *reinterpret_cast<const u32x4_t*>(kl + (i & 1) * 32 * kKStride + 16 * (i >> 1));
            };
            u32x4_t ka[2];
            ka[0] = k_operand(0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i + 1 < 16) ka[(i + 1) & 1] = k_operand(i + 1);
                sacc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[i & 1]), as_bf16x8(qop[i >> 1]),
                                                                      sacc[i & 1], 0, 0, 0);
            }
        };
        // Online softmax of tile kt's scores.  The max is taken on raw scores
        // (scale > 0) and the scale folded into the exponent: p = 2^(s *
        // scale_log2 - m).  The reference m is raised only when a tile's maximum
        // exceeds it by more than kSlack (log2 units), so p <= 2^kSlack (exact in
        // fp16 and fp32) and the accumulator rescale is rare after the first
        // tiles; the result is the same softmax, as O and l share the reference.
        // P^T as the B operand of key step s (keys 16s .. 16s+15): the 8 scores
        // sacc[s / 2][8 (s % 2) .. +8] of this lane, i.e. keys 16s + 8c + 4h + e
        // for c, e -- the k order the V^T operand follows.  Fast path: p rounded
        // once to fp16.  Exact path: hi = p truncated to bf16, lo = bf16(p - hi).
        auto softmax = [&](int kt, f32x16_t (&sacc)[2], u32x4_t (&phi)[4], u32x4_t (&plo)[4], auto half) {
            constexpr bool kHalf = decltype(half)::value;
            const int key0 = kt * kKeys;
            if (key0 + kKeys > kmin) {                     // a row's limit falls in this tile
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (key0 + 32 * mt + 8 * (v >> 2) + 4 * h + (v & 3) >= kend) sacc[mt][v] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int v = 0; v < 16; v += 4)
                    mx = maximum(maximum(mx, maximum(sacc[mt][v], sacc[mt][v + 1])),
                                 maximum(sacc[mt][v + 2], sacc[mt][v + 3]));
            mx = max_across_halves(mx);
            const float mtile = mx * a.scale_log2;
            const bool bump = mtile > m + kSlack;
            const float mn = bump ? mtile : m;
            const bool none = mn == -INFINITY;             // nothing visible yet in this row
            const float msafe = none ? 0.f : mn;           // then every score is -inf and p = 0
            const float alpha = bump ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
            const bool rescale = bump && m != -INFINITY;
            m = mn;
            float sum = 0.f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][8 * (s & 1) + e], a.scale_log2, -msafe));
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    if constexpr (kHalf) {
                        // the row sum adds the fp16 p that P.V uses
                        hw[e2] = pack_f16x2(pv[2 * e2], pv[2 * e2 + 1]);
                        sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, hw[e2]), f16x2_t{1.f16, 1.f16}, sum,
                                                     false);
                    } else {
                        // p - hi is exact in fp32 and lo keeps p to ~2^-16 relative
                        const uint32_t u0 = __float_as_uint(pv[2 * e2]), u1 = __float_as_uint(pv[2 * e2 + 1]);
                        hw[e2] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
                        lw[e2] = pack_bf16x2(pv[2 * e2] - __uint_as_float(u0 & 0xffff0000u),
                                             pv[2 * e2 + 1] - __uint_as_float(u1 & 0xffff0000u));
                        sum += pv[2 * e2] + pv[2 * e2 + 1];
                    }
                }
                phi[s] = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
                if constexpr (!kHalf) plo[s] = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
            }
            lp = lp * alpha + sum;
            if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
            }
        };
        // O^T += V^T P^T with the tile in V buffer vbuf: 4 key steps x 4 dim tiles
        // of 32 (x hi and lo parts of P on the exact path).  The V^T operand of
        // (dim tile dt, key step s): dim 32dt + l % 32, keys 16s + 4h .. +4 and
        // 16s + 8 + 4h .. +4, i.e. chunk 2s + h of the row (see the staging).
        auto pv_products = [&](int vbuf, const u32x4_t (&phi)[4], const u32x4_t (&plo)[4], auto half) {
            constexpr bool kHalf = decltype(half)::value;
            const uint16_t* vl = &v_lds[vbuf][lr * kVStride + 8 * h];
            auto v_operand = [&](int i) {                  // step i: key step i / 4, dim tile i % 4
                return *reinterpret_cast<const u32x4_t*>(vl + (i & 3) * 32 * kVStride + 16 * (i >> 2));
            };
            u32x4_t va[2];
            va[0] = v_operand(0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i + 1 < 16) va[(i + 1) & 1] = v_operand(i + 1);
                const int dt = i & 3, s = i >> 2;
                const u32x4_t vop = va[i & 1];
                if constexpr (kHalf) {
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vop), as_f16x8(phi[s]), oacc[dt], 0, 0, 0);
                } else {
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vop), as_bf16x8(phi[s]), oacc[dt], 0, 0,
                                                                       0);
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vop), as_bf16x8(plo[s]), oacc[dt], 0, 0,
                                                                       0);
                }
            }
        };
        auto init_row = [&]() {
            m = -INFINITY;
            lp = 0.f;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
        };

        // One pass over the segment's key tiles.  Fast path: P is rounded once to fp16
        // (11 significant bits) against V^T in fp16.  Exact path: P is fed as two
        // bf16 operands against V^T in bf16, keeping ~16 bits of p; a single
        // bf16 rounding of p would use most of the output's error budget on top
        // of the bf16 output rounding.  ids_loaded: the ids of the segment's
        // first tile are already in bid[0] (the first pass; the exact pass
        // reloads them).
        auto run = [&](auto half, auto ids_loaded) {
            constexpr bool kIdsLoaded = decltype(ids_loaded)::value;
            init_row();
            if constexpr (kStageSets == 2) {
                if constexpr (!kIdsLoaded) load_ids(kt_begin, Set0{});
                load_ids(kt_begin + 1, Set1{});
                stage(kt_begin, Set0{});
                load_ids(kt_begin + 2, Set0{});
                commit(0, 0, half, Set0{});
                stage(kt_begin + 1, Set1{});
                load_ids(kt_begin + 3, Set1{});
            } else {
                if constexpr (!kIdsLoaded) load_ids(kt_begin, Set0{});
                stage(kt_begin, Set0{});
                load_ids(kt_begin + 1, Set0{});
                commit(0, 0, half, Set0{});
            }
            __syncthreads();

            // One key tile.  With one staging set, tile kt + 1 is loaded now and
            // committed at the end of this tile.  With two, tile kt + 1 is already
            // in set `held` and tile kt + 2 is loaded into the other set now, to be
            // committed at the end of the next tile.
            auto tile = [&](int kt, auto held) {
                constexpr int A = decltype(held)::value;
                using Other = std::integral_constant<int, 1 - A>;
                const int buf = (kt - kt_begin) & 1;
                if constexpr (kStageSets == 2) {
                    stage(kt + 2, Other{});
                    load_ids(kt + 4, Other{});
                } else {
                    stage(kt + 1, Set0{});
                    load_ids(kt + 2, Set0{});
                }
                f32x16_t sacc[2];
                u32x4_t phi[4], plo[4];
                s_products(buf, sacc);
                softmax(kt, sacc, phi, plo, half);
                pv_products(buf, phi, plo, half);
                if (kt + 1 < kt_end)
                    commit(buf ^ 1, buf ^ 1, half, std::integral_constant<int, kStageSets == 2 ? A : 0>{});
                __syncthreads();
            };
            for (int kt = kt_begin; kt < kt_end; kt += 2) {
                tile(kt, Set1{});
                if (kt + 1 < kt_end) tile(kt + 1, Set0{});
            }
        };

        run(std::true_type{}, std::true_type{});
        // a V magnitude beyond fp16 (or a NaN, which the exact path propagates)
        const bool exact = __syncthreads_or(!(vmax <= 65504.f));
        if (exact) run(std::false_type{}, std::false_type{});
        // ---- finish: lane holds dims 32dt + 8b + 4h .. +4 of its row.
        //  * A tile within the share normalises its rows to bf16 and writes them
        //    through LDS (the K/V buffers are free once every wave has passed the
        //    last barrier of the loop): each wave stages its 32 rows, then writes
        //    4 whole rows per store instruction, 16 bytes a lane.
        //  * A segment of a tile that crosses a share boundary writes its record
        //    (rows, max, sum) in the workgroup's record 0 if the segment is its
        //    first, else in record 1, in the order of the accumulator fragments.
        //    Fast path: the rows normalised by their sum, in fp16 (every V
        //    magnitude was below 65504, so is every normalised value; 11
        //    significant bits); store (dt, b) of a wave covers 512 consecutive
        //    bytes.  Exact path: the unnormalised rows in fp32, 1 KB per store.
        //    A flag after the record's (max, sum) pairs says which.  The segment
        //    holding the tile's first unit lists the tile for the merge kernel.
        {
            const float l = sum_across_halves(lp);
            if (!split) {
                const float inv = l > 0.f ? 1.f / l : 0.f;
                uint16_t* st = (wave < 4 ? &k_lds[0][0] : &v_lds[0][0]) + (wave & 3) * kRowsPerWave * kKStride;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int b4 = 0; b4 < 4; ++b4) {
                        const f32x16_t& v = oacc[dt];
                        *reinterpret_cast<u32x2_t*>(st + lr * kKStride + 32 * dt + 8 * b4 + 4 * h) =
                            u32x2_t{pack_bf16x2(v[4 * b4] * inv, v[4 * b4 + 1] * inv),
                                    pack_bf16x2(v[4 * b4 + 2] * inv, v[4 * b4 + 3] * inv)};
                    }
                // the wave reads back only what it wrote: LDS keeps one wave's
                // accesses in order, and the compiler keeps the reads after the
                // writes
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int j = 0; j < kRowsPerWave / 4; ++j) {
                    const int wr = 4 * j + (lane >> 4);        // row within the wave
                    const int rr = wave * kRowsPerWave + wr;
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + wr * kKStride + 8 * (lane & 15));
                    if (rr / G < ntok) {
                        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) +
                                      (int64_t)(q0 + tok_begin + rr / G) * Hq * kHeadDim +
                                      (int64_t)(kvh * G + rr % G) * kHeadDim + 8 * (lane & 15);
                        *reinterpret_cast<u32x4_t*>(o) = v;
                    }
                }
                __syncthreads();                           // staging read before the next segment's commit
            } else {
                float* rec = a.part + ((int64_t)blockIdx.x * 2 + (first ? 0 : 1)) * kPrefillRows * kRec;
                if (active) {
                    if (!exact) {
                        const float inv = l > 0.f ? 1.f / l : 0.f;
                        uint32_t* rh = reinterpret_cast<uint32_t*>(rec);
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                            for (int b4 = 0; b4 < 4; ++b4) {
                                const f32x16_t& v = oacc[dt];
                                *reinterpret_cast<u32x2_t*>(rh + ((wave * 16 + 4 * dt + b4) * kWave + lane) * 2) =
                                    u32x2_t{pack_f16x2(v[4 * b4] * inv, v[4 * b4 + 1] * inv),
                                            pack_f16x2(v[4 * b4 + 2] * inv, v[4 * b4 + 3] * inv)};
                            }
                    } else {
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                            for (int b4 = 0; b4 < 4; ++b4)
                                *reinterpret_cast<f32x4_t*>(rec + ((wave * 16 + 4 * dt + b4) * kWave + lane) * 4) =
                                    f32x4_t{oacc[dt][4 * b4], oacc[dt][4 * b4 + 1], oacc[dt][4 * b4 + 2],
                                            oacc[dt][4 * b4 + 3]};
                    }
                    if (h == 0) *reinterpret_cast<float2*>(rec + kPrefillRows * kHeadDim + 2 * r) = make_float2(m, l);
                }
                if (tid == 0) rec[kRecFlag] = exact ? 1.f : 0.f;
            }
        }
        // list entry: first slot, slots | (record of the first slot) << 24, first
        // row, (tokens << 8) | KV head
        if (split && u == tu0 && tid == 0) {
            const int s1 = slot_of(s_bnd, slots, tu0 + units - 1);
            a.split_list[split_before * Hkv + kvh] =
                int4{slot, (s1 - slot + 1) | ((tu0 != ub) << 24), q0 + tok_begin, (ntok << 8) | kvh};
        }

        u = tu0 + seg_end;
        if (u >= ue) break;
        split_before += split;
        tu0 += units;
        ++tile;
        while (tile >= nt && b + 1 < B) {                  // next sequence with query tiles
            ++b;
            sh = uniform(seq_shape(a, b));
            nt = tiles_of(sh, TQ);
            tile = 0;
        }
    }
}

// Log-sum-exp merge of the segments of every listed query tile: per row,
// M = max_p m_p, out = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p, taken in
// one pass with a running max.  One workgroup per 32-row wave block of a
// listed (tile, KV head); the records hold each block's rows in accumulator
// fragment order (16 fragments of 64 lanes x 4 values, fp16 normalised rows
// or fp32 unnormalised ones by the record's flag), so thread t reads
// fragments t / 64 + 4i (i < 4) of lane t % 64, contiguous per wave and
// fragment, and stages its bf16 results in LDS so that whole rows leave
// together.
template <int G>
__global__ void __launch_bounds__(256)
prefill_merge_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_out[kRowsPerWave * kKStride];
    const int e = (int)(blockIdx.x / kMergeParts);
    if (e >= *a.split_count) return;
    const int4 d = a.split_list[e];
    const int s0 = d.x, np = d.y & 0xffffff, rec0 = d.y >> 24, row0 = d.z, ntok = d.w >> 8, kvh = d.w & 255;
    const int w = (int)(blockIdx.x % kMergeParts);     // wave block: rows 32w .. 32w + 31
    if ((w * kRowsPerWave) / G >= ntok) return;        // rows are token-major: the whole block is inactive
    const int Hkv = a.num_kv_heads;
    const int t = threadIdx.x, lane = t & 63, j = t >> 6;
    const int lr = lane & 31, h = lane >> 5;
    const int r = w * kRowsPerWave + lr;
    float mrun = -INFINITY, lrun = 0.f;
    f32x4_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < np; ++p) {
        // segment p: slot s0 + p, record rec0 for p = 0 (the tile may start
        // inside that slot's share), else record 0
        const int64_t wg = (int64_t)(s0 + p) * Hkv + kvh;
        const float* rec = a.part + (wg * 2 + (p == 0 ? rec0 : 0)) * kPrefillRows * kRec;
        const float2 ml = *reinterpret_cast<const float2*>(rec + kPrefillRows * kHeadDim + 2 * r);
        f32x4_t ov[4];
        if (rec[kRecFlag] == 0.f) {                    // fp16 rows normalised by their sum
            // read as an fp16 x 4 vector: hipcc 7.2 compiles a bit cast of one
            // component of a loaded vector (v.y) from the vector's first component
            const f16x4_t* rh = reinterpret_cast<const f16x4_t*>(rec);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ov[i] = __builtin_convertvector(rh[(w * 16 + j + 4 * i) * kWave + lane], f32x4_t) * ml.y;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ov[i] = *reinterpret_cast<const f32x4_t*>(rec + ((w * 16 + j + 4 * i) * kWave + lane) * 4);
        }
        const float mn = fmaxf(mrun, ml.x);
        const float wa = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - mn);
        const float wb = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - mn);
        lrun = wa * lrun + wb * ml.y;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = wa * o[i] + wb * ov[i];
        mrun = mn;
    }
    const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
    // fragment (dt, b) = j + 4i holds dims 32dt + 8b + 4h .. +4 of row lr
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int f = j + 4 * i, dt = f >> 2, b4 = f & 3;
        *reinterpret_cast<u32x2_t*>(&s_out[lr * kKStride + 32 * dt + 8 * b4 + 4 * h]) =
            u32x2_t{pack_bf16x2(o[i].x * inv, o[i].y * inv), pack_bf16x2(o[i].z * inv, o[i].w * inv)};
    }
    __syncthreads();
    // 32 rows of 256 bytes: 16 threads a row, 16 rows per pass
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int wr = 16 * pass + (t >> 4);
        const int rr = w * kRowsPerWave + wr;
        if (rr / G < ntok) {
            uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + (int64_t)(row0 + rr / G) * a.num_heads * kHeadDim +
                            (int64_t)(kvh * G + rr % G) * kHeadDim + 8 * (t & 15);
            *reinterpret_cast<u32x4_t*>(out) = *reinterpret_cast<const u32x4_t*>(&s_out[wr * kKStride + 8 * (t & 15)]);
        }
    }
}

template <int G>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
    const size_t lds = 2 * sizeof(int32_t) * ((size_t)a.num_seqs + 1);
    const int64_t grid = (int64_t)a.slots_per_kvh * a.num_kv_heads;
    hipLaunchKernelGGL((prefill_kernel<G>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // a listed tile crosses one of the slots_per_kvh - 1 share boundaries of its
    // KV head, each of which lies in one tile
    const int64_t listed = (int64_t)(a.slots_per_kvh - 1) * a.num_kv_heads;
    if (listed == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_merge_kernel<G>), dim3((unsigned)(kMergeParts * listed)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int G>
int blocks_per_cu(int num_seqs) {
    int n = 0;
    const size_t lds = 2 * sizeof(int32_t) * ((size_t)num_seqs + 1);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_kernel<G>, kThreads, lds) != hipSuccess) return 0;
    return n;
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

int prefill_blocks_per_cu(int group, int num_seqs) {
    switch (group) {
        case 1: return blocks_per_cu<1>(num_seqs);
        case 2: return blocks_per_cu<2>(num_seqs);
        case 4: return blocks_per_cu<4>(num_seqs);
        case 8: return blocks_per_cu<8>(num_seqs);
        default: return 0;
    }
}

}  // namespace pa
