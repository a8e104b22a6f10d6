// common.h -- device helpers shared by the libdsa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

constexpr int kWave = 64;
constexpr int kIdxDim = 128;   // indexer key/query width
constexpr int kDqk = 576;      // latent key width (512 latent + 64 decoupled RoPE)
constexpr int kDv = 512;       // value width

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

// Cache addressing as plain values, passed to kernels by value.
struct CacheView {
    const void* data;
    const float* scale;
    int64_t num_rows;
    int64_t seq_stride;
    const int32_t* page_table;
    int32_t pt_stride;
    int32_t page_size;
};

// Storage row of logical token s of sequence b, or -1 when the page number is out of range.
__device__ __forceinline__ int64_t cache_row(const CacheView& c, int b, int64_t s) {
    if (c.page_table == nullptr) return (int64_t)b * c.seq_stride + s;
    int64_t page = c.page_table[(int64_t)b * c.pt_stride + s / c.page_size];
    int64_t row = page * c.page_size + s % c.page_size;
    return (page >= 0 && row < c.num_rows) ? row : -1;
}

// ---- number formats (exact decodes) -----------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// OCP e4m3fn -> f32, exact: normal codes rebias the exponent (7 -> 127); subnormals are m * 2^-9.
__device__ __forceinline__ float e4m3_bits_to_f32(uint8_t b) {
    uint32_t sign = (uint32_t)(b & 0x80) << 24;
    uint32_t e = (b >> 3) & 0xf, m = b & 0x7;
    if (e == 0xf && m == 0x7) return __uint_as_float(0x7fc00000u | sign);
    if (e == 0) { float v = (float)m * 0.001953125f; return sign ? -v : v; }
    return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

__device__ __forceinline__ float load_elem(const void* base, int dtype, int64_t i) {
    if (dtype == DSA_F32) return ((const float*)base)[i];
    if (dtype == DSA_BF16) return bf16_bits_to_f32(((const uint16_t*)base)[i]);
    return e4m3_bits_to_f32(((const uint8_t*)base)[i]);
}

// f32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---- wave helpers --------------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    for (int o = 32; o >= 1; o >>= 1) { uint32_t w = __shfl_xor(v, o, kWave); v = v > w ? v : w; }
    return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    for (int o = 32; o >= 1; o >>= 1) { uint32_t w = __shfl_xor(v, o, kWave); v = v < w ? v : w; }
    return v;
}

}  // namespace dsa
