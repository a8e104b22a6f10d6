// peaks.hip -- achievable-peak probes for the benchmark (not part of libdsa's ABI).
//
// Two kernels measure what this GPU delivers, next to its published peaks:
//   * a streaming read: every thread folds 16-byte words of a large buffer into one word, 8 loads in
//     flight per thread, grid-stride over the buffer (HBM read bandwidth);
//   * a bf16 matrix-core loop: every wave runs 4 independent chains of v_mfma_f32_32x32x16_bf16 on
//     register operands (dense bf16 MFMA throughput at the clock the chip holds under load).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                            uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kReadThreads;
    size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; u++) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kReadUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(size_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

constexpr int kMfmaThreads = 256;
constexpr int kChains = 4;

__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
        b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; c++) acc[c] = f32x16{};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int c = 0; c < kChains; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) s += acc[c][r];
    sink[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from src with `blocks` workgroups of 256 threads; sink holds
// blocks * 256 words.
hipError_t peak_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t st) {
    read_kernel<<<blocks, kReadThreads, 0, st>>>((const u32x4*)src, bytes / 16, sink);
    return hipGetLastError();
}

// blocks workgroups of 4 waves, each wave `iters` x 4 MFMAs of 32x32x16 (32768 flops each); sink
// holds blocks * 256 floats.  Flops: blocks * 4 * iters * 4 * 32768.
hipError_t peak_mfma_bf16(int iters, float* sink, int blocks, hipStream_t st) {
    mfma_kernel<<<blocks, kMfmaThreads, 0, st>>>(iters, sink);
    return hipGetLastError();
}

}  // extern "C"
