// Probes for gfx950: a streaming read and a streaming copy of a flat buffer,
// and a matrix-core rate probe.  They carry none of the attention arithmetic.  Decode attention is
// bound by HBM reads (the article "AI Infra入门干货总结：大模型是如何高效推理的",
// section "Attention (FlashAttention, Scaled Dot-Product Attention)", on the
// memory wall of reading the KV cache), so its roofline needs the bandwidth a
// plain read reaches on the same GPU, and the copy gives the hardware traffic
// counters a transfer of known size to be scaled by.
#include "device_common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

// Each thread reads 16-byte vectors, kProbeUnroll of them in flight, over a
// grid-stride loop.  The XOR of everything read is stored only if it equals a
// value no input produces by chance, so the loads cannot be dropped and
// nothing is written in practice.
__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u) sink[0] = x;
}

__global__ void __launch_bounds__(kProbeThreads)
stream_copy_kernel(u32x4_t* __restrict__ dst, const u32x4_t* __restrict__ src, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        u32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Matrix-core rate: every wave runs `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 accumulations (the instruction of the prefill's
// S^T product; four chains keep it at its rate), 4 * 32768 flops a round.
// The accumulators are reduced and stored only if the sum equals a value no
// input produces, so the products cannot be dropped.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(kProbeThreads)
mfma_rate_kernel(uint32_t* __restrict__ sink, int32_t iters) {
    bf16x8_t x, y;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = (__bf16)(0.001f * (float)(threadIdx.x + e));
        y[e] = (__bf16)(0.002f * (float)(blockIdx.x % 7 + e));
    }
    f32x16_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) c[j][v] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += c[j][v];
    if (s == 1234567.f) sink[0] = __float_as_uint(s);
}

int grid_for(int64_t n16, int32_t workgroups) {
    if (workgroups > 0) return workgroups;
    const int64_t want = (n16 + kProbeThreads - 1) / kProbeThreads;
    return (int)(want < 4096 ? (want > 0 ? want : 1) : 4096);   // 16 workgroups per CU at most
}

}  // namespace

hipError_t launch_mfma_probe(uint32_t* sink, int32_t workgroups, int32_t iters, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(kProbeThreads), 0, stream, sink, iters);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups,
                              hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid_for(n16, workgroups)), dim3(kProbeThreads), 0,
                       stream, (const u32x4_t*)src, n16, sink);
    return hipGetLastError();
}

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, int32_t workgroups,
                              hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(stream_copy_kernel, dim3(grid_for(n16, workgroups)), dim3(kProbeThreads), 0,
                       stream, (u32x4_t*)dst, (const u32x4_t*)src, n16);
    return hipGetLastError();
}

}  // namespace pa
