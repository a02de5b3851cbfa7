// Device helpers shared by the gfx950 kernels of libpa.so: element storage
// types, 8-element chunks (one 16-byte or two 16-byte loads per lane), bf16
// conversions and wave-level lane exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kBlock = 16;       // tokens per physical cache block
constexpr int kHeadDim = 128;    // head_dim this build implements

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 in one word (lo in bits 0-15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Eight consecutive elements of one K/V/Q row, as one lane holds them.
struct ChunkBF16 {
    u32x4_t w;                                   // 8 x bf16 = 16 bytes
    static constexpr int kBytes = 16;
};
struct ChunkF32 {
    f32x4_t a, b;                                // 8 x fp32 = 32 bytes
    static constexpr int kBytes = 32;
};

template <bool NT>
__device__ __forceinline__ void load_chunk(ChunkBF16& c, const void* p) {
    if constexpr (NT) c.w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    else c.w = *reinterpret_cast<const u32x4_t*>(p);
}
template <bool NT>
__device__ __forceinline__ void load_chunk(ChunkF32& c, const void* p) {
    const f32x4_t* q = reinterpret_cast<const f32x4_t*>(p);
    if constexpr (NT) { c.a = __builtin_nontemporal_load(q); c.b = __builtin_nontemporal_load(q + 1); }
    else { c.a = q[0]; c.b = q[1]; }
}

__device__ __forceinline__ void to_f32(const ChunkBF16& c, float f[8]) {
    f[0] = bf16_lo(c.w.x); f[1] = bf16_hi(c.w.x);
    f[2] = bf16_lo(c.w.y); f[3] = bf16_hi(c.w.y);
    f[4] = bf16_lo(c.w.z); f[5] = bf16_hi(c.w.z);
    f[6] = bf16_lo(c.w.w); f[7] = bf16_hi(c.w.w);
}
__device__ __forceinline__ void to_f32(const ChunkF32& c, float f[8]) {
    f[0] = c.a.x; f[1] = c.a.y; f[2] = c.a.z; f[3] = c.a.w;
    f[4] = c.b.x; f[5] = c.b.y; f[6] = c.b.z; f[7] = c.b.w;
}

// Reinterpret one 32-bit word as two bf16.  It takes the word by value: clang
// (ROCm 7.2) mis-lowers __builtin_bit_cast applied directly to an ext-vector
// component such as w.y, reading component 0 instead.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t word) { return __builtin_bit_cast(bf16x2_t, word); }

// <q, k> over one chunk, accumulated into acc.  bf16 products are exact in
// fp32; v_dot2_f32_bf16 adds two of them per instruction.
__device__ __forceinline__ float dot_chunk(const ChunkBF16& q, const ChunkBF16& k, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w.x), as_bf16x2(k.w.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w.y), as_bf16x2(k.w.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w.z), as_bf16x2(k.w.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w.w), as_bf16x2(k.w.w), acc, false);
    return acc;
}
__device__ __forceinline__ float dot_chunk(const ChunkF32& q, const ChunkF32& k, float acc) {
    acc = fmaf(q.a.x, k.a.x, acc); acc = fmaf(q.a.y, k.a.y, acc);
    acc = fmaf(q.a.z, k.a.z, acc); acc = fmaf(q.a.w, k.a.w, acc);
    acc = fmaf(q.b.x, k.b.x, acc); acc = fmaf(q.b.y, k.b.y, acc);
    acc = fmaf(q.b.z, k.b.z, acc); acc = fmaf(q.b.w, k.b.w, acc);
    return acc;
}

// Store eight fp32 values as one row chunk of the output dtype.
__device__ __forceinline__ void store_chunk(uint16_t* p, const float f[8]) {
    u32x4_t w;
    w.x = pack_bf16x2(f[0], f[1]); w.y = pack_bf16x2(f[2], f[3]);
    w.z = pack_bf16x2(f[4], f[5]); w.w = pack_bf16x2(f[6], f[7]);
    *reinterpret_cast<u32x4_t*>(p) = w;
}
__device__ __forceinline__ void store_chunk(float* p, const float f[8]) {
    reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{f[0], f[1], f[2], f[3]};
    reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{f[4], f[5], f[6], f[7]};
}

// Store a chunk's bits unchanged.
__device__ __forceinline__ void store_chunk_raw(uint16_t* p, const ChunkBF16& c) {
    *reinterpret_cast<u32x4_t*>(p) = c.w;
}
__device__ __forceinline__ void store_chunk_raw(float* p, const ChunkF32& c) {
    reinterpret_cast<f32x4_t*>(p)[0] = c.a;
    reinterpret_cast<f32x4_t*>(p)[1] = c.b;
}

// ---- lane exchanges ---------------------------------------------------------
// DPP controls (CDNA): quad_perm selects within groups of 4 lanes, row_ror
// rotates within rows of 16 lanes.
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]: partner lane ^ 1
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]: partner lane ^ 2
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
    int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// IEEE-754 maximum (a NaN operand gives NaN): v_maximum3_f32 on gfx950, with
// no quieting of the operands first.
__device__ __forceinline__ float maximum(float x, float y) { return __builtin_elementwise_maximum(x, y); }

// Across the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48), with
// the gfx950 lane swaps (VALU, no LDS round trip): permlane32_swap(x, x)
// returns the two 32-lane halves each broadcast to both, permlane16_swap(x, x)
// the even and odd 16-lane rows each broadcast to their pair.
__device__ __forceinline__ float max_across_rows(float x) {
    auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = maximum(__uint_as_float(h[0]), __uint_as_float(h[1]));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_rows(float x) {
    auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// ---- fp8 encoding (the fp8 scatters, and the decode's fp8 append form) ----
// Each element x is stored as the OCP E4M3 (E5 = false) or E5M2 (E5 = true)
// code of x / scale: the division in float32 (correctly rounded), magnitudes
// beyond the format's largest finite value (448; 57344) saturated to it, NaN
// kept, then the hardware conversion to the nearest code, ties to even.
template <bool E5, bool HI>
__device__ __forceinline__ int cvt_pk_fp8(float a, float b, int old) {
    if constexpr (E5)
        return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
    else
        return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// 16 source elements (two chunks) -> their 16 codes of x / scale.
template <typename Chunk, bool E5>
__device__ __forceinline__ u32x4_t fp8_codes(const Chunk& x0, const Chunk& x1, float scale) {
    constexpr float kMax = E5 ? 57344.f : 448.f;
    float f[16];
    to_f32(x0, f);
    to_f32(x1, f + 8);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float y = f[e] / scale;
        f[e] = __builtin_fabsf(y) > kMax ? __builtin_copysignf(kMax, y) : y;
    }
    u32x4_t w;
    int p0 = cvt_pk_fp8<E5, false>(f[0], f[1], 0);
    p0 = cvt_pk_fp8<E5, true>(f[2], f[3], p0);
    int p1 = cvt_pk_fp8<E5, false>(f[4], f[5], 0);
    p1 = cvt_pk_fp8<E5, true>(f[6], f[7], p1);
    int p2 = cvt_pk_fp8<E5, false>(f[8], f[9], 0);
    p2 = cvt_pk_fp8<E5, true>(f[10], f[11], p2);
    int p3 = cvt_pk_fp8<E5, false>(f[12], f[13], 0);
    p3 = cvt_pk_fp8<E5, true>(f[14], f[15], p3);
    w.x = (uint32_t)p0; w.y = (uint32_t)p1; w.z = (uint32_t)p2; w.w = (uint32_t)p3;
    return w;
}

}  // namespace pa
