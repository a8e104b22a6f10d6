// cache_write.hip -- the write path that feeds the DSA steps, for gfx950: rotary position embedding
// of the new keys and queries, storage in the caches' number formats (bf16, or e4m3 with one scale
// per 128-wide row), and the append of new tokens to contiguous or paged caches.
//
// Page "一文讀懂DeepSeek-V3.2核心技術DSA", "DSA 的四步工作流程", first step: the query and key
// projections carry rotary position information before the indexer and the attention use them.
// Page "DeepSeek 稀疏注意力路线", section "DeepSeek-V3：MLA 基座", "核心机制（直觉）": MLA keeps that
// information in a decoupled channel of its own (the 64 dims after the 512 latent dims of a row).
// Page "DeepSeek 稀疏注意力路线", "两阶段流程" item 1: the indexer runs in fp8.
//
// Rotation: pair i of the span [off, off + d) of a row at position p turns by p * base^(-2i/d)
// radians; pairs are (off + 2i, off + 2i + 1) (interleaved) or (off + i, off + i + d/2) (split).
// The angle, its cosine and sine and the rotation are computed in double, and each result is
// rounded once to binary32 before it is stored:
//   f32 as is; bf16 round to nearest even; fp8 per row: s = max(amax, 1e-12) / 448 and
//   code = e4m3(x / s), round to nearest even, saturating at 448 (binary32 arithmetic throughout).
// This path is bound by HBM traffic; the double-precision angles are computed once per (token,
// pair) and shared by all heads of the token.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kCwThreads = 256;
constexpr int kCwWaves = kCwThreads / kWave;
constexpr int kMaxIdxPairs = kIdxDim / 2;   // 64
constexpr int kMaxMlaPairs = kDqk / 2;      // 288

// e4m3fn code of v, the nearest value with ties to the even code; magnitudes of 448 and above
// give 448 (the largest finite value).  -0 and negative values that round to zero keep the sign.
__device__ __forceinline__ uint32_t f32_to_e4m3_bits(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    if (!(a < 448.0f)) return sign | 0x7eu;
    if (a < 0.015625f) {                                 // below 2^-6: subnormal steps of 2^-9
        const uint32_t m = (uint32_t)__builtin_rintf(a * 512.0f);   // 0 .. 8 (8 = smallest normal)
        return sign | m;
    }
    int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;       // 2^e <= a < 2^(e+1), e in [-6, 8]
    uint32_t q = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));   // 8 .. 16
    if (q == 16u) { q = 8u; e++; }
    return sign | ((uint32_t)(e + 7) << 3) | (q - 8u);
}

// cos and sin of p * base^(-2i/d), in double.
__device__ __forceinline__ void rope_cs(int64_t p, int i, const RopeView& r, double& c, double& s) {
    const double th = pow(r.base, -2.0 * i / r.dim);
    sincos((double)p * th, &s, &c);
}

// For element e of a row: whether it is rotated, its pair number, its partner and whether it is
// the first element of the pair.
__device__ __forceinline__ bool rope_pair(int e, const RopeView& r, int& i, int& partner, bool& first) {
    if (r.dim == 0 || e < r.off || e >= r.off + r.dim) return false;
    const int j = e - r.off;
    if (r.inter) {
        i = j >> 1;
        first = (j & 1) == 0;
        partner = first ? e + 1 : e - 1;
    } else {
        const int h = r.dim >> 1;
        first = j < h;
        i = first ? j : j - h;
        partner = first ? e + h : e - h;
    }
    return true;
}

__device__ __forceinline__ float load_src(const void* base, int dtype, int64_t i) {
    return dtype == DSA_F32 ? ((const float*)base)[i] : bf16_bits_to_f32(((const uint16_t*)base)[i]);
}

// Elements 2 * lane and 2 * lane + 1 of N rows of 128 (rows[r]) as binary32, one vector load per row.
// The dtype is tested once: a load under a per-load branch makes the compiler wait for each one.
template <int N>
__device__ __forceinline__ void load_rows128(const void* base, int dtype, const int64_t (&rows)[N], float (&x)[N][2]) {
    const int lane = lane_id();
    if (dtype == DSA_F32) {
        const float2* b2 = (const float2*)base;
#pragma unroll
        for (int r = 0; r < N; r++) {
            const float2 v = b2[rows[r] * (kIdxDim / 2) + lane];
            x[r][0] = v.x;
            x[r][1] = v.y;
        }
    } else {
        const uint32_t* b1 = (const uint32_t*)base;
#pragma unroll
        for (int r = 0; r < N; r++) {
            const uint32_t w = b1[rows[r] * (kIdxDim / 2) + lane];
            x[r][0] = bf16_bits_to_f32((uint16_t)(w & 0xffffu));
            x[r][1] = bf16_bits_to_f32((uint16_t)(w >> 16));
        }
    }
}

// Store one wave's row of 128 binary32 values (element 2 * lane + u in v[u]) in dtype; fp8 also
// writes the row's scale.
__device__ __forceinline__ void store_row128(const float (&v)[2], int dtype, void* dst, float* scale,
                                             int64_t row) {
    const int lane = lane_id();
    if (dtype == DSA_F32) {
        ((float2*)dst)[row * (kIdxDim / 2) + lane] = make_float2(v[0], v[1]);
    } else if (dtype == DSA_BF16) {
        ((uint32_t*)dst)[row * (kIdxDim / 2) + lane] =
            (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    } else {
        const float amax = wave_max(fmaxf(fabsf(v[0]), fabsf(v[1])));
        const float s = fmaxf(amax, 1e-12f) / 448.0f;
        ((uint16_t*)dst)[row * (kIdxDim / 2) + lane] =
            (uint16_t)(f32_to_e4m3_bits(v[0] / s) | (f32_to_e4m3_bits(v[1] / s) << 8));
        if (lane == 0) scale[row] = s;
    }
}

// Storage row of token (b, p) for a write, or -1 when the token has no slot in the cache.
__device__ __forceinline__ int64_t write_row(const CacheView& c, int b, int num_seqs, int p) {
    if (b < 0 || b >= num_seqs || p < 0) return -1;
    if (c.page_table == nullptr) {
        if (p >= c.seq_stride) return -1;
        const int64_t r = (int64_t)b * c.seq_stride + p;
        return r < c.num_rows ? r : -1;
    }
    if (p / c.page_size >= c.pt_stride) return -1;
    return cache_row(c, b, p);   // -1 for a page outside the cache
}

// One wave per new token: the indexer key row (128) and the latent row (576).  The source rows
// are loaded first (they do not depend on where the token goes), then the destination rows are
// looked up.
__global__ __launch_bounds__(kCwThreads) void cache_append_kernel(
    const void* __restrict__ k_new, int k_dtype, const void* __restrict__ lat_new, int lat_dtype,
    const int32_t* __restrict__ seq, const int32_t* __restrict__ pos, int T, int num_seqs, RopeView k_rope,
    RopeView lat_rope, CacheView kc, int kc_dtype, CacheView lc) {
    constexpr int kLatPerLane = kDqk / kWave;   // 9
    __shared__ float rowk[kCwWaves][kIdxDim];
    __shared__ float rowl[kCwWaves][kDqk];
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kCwWaves + wave;
    if (t >= T) return;
    float xk[1][2] = {{0.0f, 0.0f}};
    float xl[kLatPerLane];
    if (k_new != nullptr) {
        const int64_t rows[1] = {t};
        load_rows128(k_new, k_dtype, rows, xk);
    }
    if (lat_new != nullptr) {
        if (lat_dtype == DSA_F32) {
            const float* src = (const float*)lat_new + (int64_t)t * kDqk;
#pragma unroll
            for (int j = 0; j < kLatPerLane; j++) xl[j] = src[lane + kWave * j];
        } else {
            const uint16_t* src = (const uint16_t*)lat_new + (int64_t)t * kDqk;
            uint16_t v[kLatPerLane];
#pragma unroll
            for (int j = 0; j < kLatPerLane; j++) v[j] = src[lane + kWave * j];
#pragma unroll
            for (int j = 0; j < kLatPerLane; j++) xl[j] = bf16_bits_to_f32(v[j]);
        }
    }
    const int b = seq[t], p = pos[t];
    if (k_new != nullptr) {
        const int64_t r = write_row(kc, b, num_seqs, p);
        if (r >= 0) {
            float* x = rowk[wave];
            x[2 * lane] = xk[0][0];
            x[2 * lane + 1] = xk[0][1];
            __builtin_amdgcn_wave_barrier();
            float v[2];
#pragma unroll
            for (int u = 0; u < 2; u++) {
                const int e = 2 * lane + u;
                int i, q;
                bool first;
                if (rope_pair(e, k_rope, i, q, first)) {
                    double c, s;
                    rope_cs(p, i, k_rope, c, s);
                    const double xe = x[e], xq = x[q];
                    v[u] = (float)(first ? xe * c - xq * s : xq * s + xe * c);
                } else {
                    v[u] = x[e];
                }
            }
            store_row128(v, kc_dtype, (void*)kc.data, (float*)kc.scale, r);
        }
    }
    if (lat_new != nullptr) {
        const int64_t r = write_row(lc, b, num_seqs, p);
        if (r >= 0) {
            float* x = rowl[wave];
#pragma unroll
            for (int j = 0; j < kLatPerLane; j++) x[lane + kWave * j] = xl[j];
            __builtin_amdgcn_wave_barrier();
            uint16_t* dst = (uint16_t*)lc.data + r * kDqk;
#pragma unroll
            for (int j = 0; j < kLatPerLane; j++) {
                const int e = lane + kWave * j;
                int i, q;
                bool first;
                float v = x[e];
                if (rope_pair(e, lat_rope, i, q, first)) {
                    double c, s;
                    rope_cs(p, i, lat_rope, c, s);
                    const double xe = x[e], xq = x[q];
                    v = (float)(first ? xe * c - xq * s : xq * s + xe * c);
                }
                dst[e] = f32_to_bf16_bits(v);
            }
        }
    }
}

// Workgroup (t, s): slice s of query token t's heads (gridDim.y slices, so that short batches still
// fill the GPU).  The token's angle tables go to LDS, then the slice's indexer query rows (out of
// place, to f32 / bf16 / fp8 with a scale per row) and MLA query rows (bf16, rotated in place on
// the span).  Loads are batched so that each wave keeps many in flight: indexer rows kIdxBatch at a
// time per wave (row base + 4r + wave), and the MLA span as (row, pair) items spread over all
// threads, each thread loading all of its items before it computes any.
constexpr int kIdxBatch = 8;
constexpr int kPairBatch = 8;

__global__ __launch_bounds__(kCwThreads) void rope_queries_kernel(
    const void* __restrict__ qi_in, int qi_dtype, int Hi, void* __restrict__ qi_out, int qo_dtype,
    float* __restrict__ qo_scale, RopeView ri, uint16_t* __restrict__ qm, int Hm, RopeView rm,
    const int32_t* __restrict__ pos) {
    __shared__ double cs_i[kMaxIdxPairs][2];
    __shared__ double cs_m[kMaxMlaPairs][2];
    __shared__ float rowq[kCwWaves][kIdxBatch][kIdxDim];
    const int t = blockIdx.x, sl = blockIdx.y, ns = gridDim.y;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int64_t p = pos[t];
    const int hi_lo = (int)((int64_t)sl * Hi / ns), hi_hi = (int)((int64_t)(sl + 1) * Hi / ns);
    const int hm_lo = (int)((int64_t)sl * Hm / ns), hm_hi = (int)((int64_t)(sl + 1) * Hm / ns);
    // the two angle tables on different waves (indexer: wave 0, MLA: from wave 1 on)
    if (qi_in != nullptr && tid < ri.dim / 2) rope_cs(p, tid, ri, cs_i[tid][0], cs_i[tid][1]);
    if (qm != nullptr)
        for (int i = tid - kWave; i >= 0 && i < rm.dim / 2; i += kCwThreads - kWave) rope_cs(p, i, rm, cs_m[i][0], cs_m[i][1]);
    __syncthreads();
    if (qi_in != nullptr) {
        for (int h0 = hi_lo + wave; h0 < hi_hi; h0 += kCwWaves * kIdxBatch) {
            const int nr = min(kIdxBatch, (hi_hi - h0 + kCwWaves - 1) / kCwWaves);   // rows h0 + 4r < hi_hi
            float xr[kIdxBatch][2];
            int64_t rows[kIdxBatch];
#pragma unroll
            for (int r = 0; r < kIdxBatch; r++)
                rows[r] = (int64_t)t * Hi + h0 + kCwWaves * min(r, nr - 1);   // clamped: in range
            load_rows128(qi_in, qi_dtype, rows, xr);
#pragma unroll
            for (int r = 0; r < kIdxBatch; r++) {
                rowq[wave][r][2 * lane] = xr[r][0];
                rowq[wave][r][2 * lane + 1] = xr[r][1];
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int r = 0; r < kIdxBatch; r++) {
                if (r >= nr) break;
                const float* x = rowq[wave][r];
                float v[2];
#pragma unroll
                for (int u = 0; u < 2; u++) {
                    const int e = 2 * lane + u;
                    int i, q;
                    bool first;
                    if (rope_pair(e, ri, i, q, first)) {
                        const double c = cs_i[i][0], s = cs_i[i][1], xe = x[e], xq = x[q];
                        v[u] = (float)(first ? xe * c - xq * s : xq * s + xe * c);
                    } else {
                        v[u] = x[e];
                    }
                }
                store_row128(v, qo_dtype, qi_out, qo_scale, rows[r]);
            }
            __builtin_amdgcn_wave_barrier();   // every lane has read the batch before the next is written
        }
    }
    if (qm != nullptr && rm.dim > 0) {
        uint16_t* base = qm + ((int64_t)t * Hm + hm_lo) * kDqk;
        const int np = rm.dim / 2, hm_n = hm_hi - hm_lo;
        if (rm.off % 8 == 0 && rm.dim % 16 == 0 && ((uintptr_t)qm & 15u) == 0) {
            // 16-byte items: interleaved spans, 8 consecutive elements (4 pairs) of a row; split
            // spans, 8 consecutive first-half elements and their 8 second-half partners
            const int per_row = rm.inter ? rm.dim / 8 : rm.dim / 16;
            const int items = hm_n * per_row;
            for (int it0 = tid; it0 < items; it0 += kCwThreads * kPairBatch) {
                uint4 va[kPairBatch], vb[kPairBatch];
#pragma unroll
                for (int j = 0; j < kPairBatch; j++) {
                    const int it = min(it0 + j * kCwThreads, items - 1);
                    const int h = it / per_row, c = it - h * per_row;
                    const uint16_t* rp = base + (int64_t)h * kDqk + rm.off + 8 * c;
                    va[j] = *(const uint4*)rp;
                    if (!rm.inter) vb[j] = *(const uint4*)(rp + np);
                }
#pragma unroll
                for (int j = 0; j < kPairBatch; j++) {
                    const int it = it0 + j * kCwThreads;
                    if (it >= items) break;
                    const int h = it / per_row, c = it - h * per_row;
                    uint16_t* rp = base + (int64_t)h * kDqk + rm.off + 8 * c;
                    const uint32_t wa[4] = {va[j].x, va[j].y, va[j].z, va[j].w};
                    uint32_t oa[4], ob[4];
                    if (rm.inter) {
#pragma unroll
                        for (int k = 0; k < 4; k++) {   // word k = pair 4c + k: (low half, high half)
                            const int i = 4 * c + k;
                            const double cc = cs_m[i][0], ss = cs_m[i][1];
                            const double x0 = bf16_bits_to_f32((uint16_t)(wa[k] & 0xffffu));
                            const double x1 = bf16_bits_to_f32((uint16_t)(wa[k] >> 16));
                            oa[k] = (uint32_t)f32_to_bf16_bits((float)(x0 * cc - x1 * ss)) |
                                    ((uint32_t)f32_to_bf16_bits((float)(x0 * ss + x1 * cc)) << 16);
                        }
                        *(uint4*)rp = make_uint4(oa[0], oa[1], oa[2], oa[3]);
                    } else {
                        const uint32_t wb[4] = {vb[j].x, vb[j].y, vb[j].z, vb[j].w};
#pragma unroll
                        for (int k = 0; k < 4; k++) {   // words k of both halves: pairs 8c + 2k, 8c + 2k + 1
                            uint32_t ra = 0, rb = 0;
#pragma unroll
                            for (int u = 0; u < 2; u++) {
                                const int i = 8 * c + 2 * k + u;
                                const double cc = cs_m[i][0], ss = cs_m[i][1];
                                const double x0 = bf16_bits_to_f32((uint16_t)(wa[k] >> (16 * u)));
                                const double x1 = bf16_bits_to_f32((uint16_t)(wb[k] >> (16 * u)));
                                ra |= (uint32_t)f32_to_bf16_bits((float)(x0 * cc - x1 * ss)) << (16 * u);
                                rb |= (uint32_t)f32_to_bf16_bits((float)(x0 * ss + x1 * cc)) << (16 * u);
                            }
                            oa[k] = ra;
                            ob[k] = rb;
                        }
                        *(uint4*)rp = make_uint4(oa[0], oa[1], oa[2], oa[3]);
                        *(uint4*)(rp + np) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
                    }
                }
            }
        } else {
            // any other span: (row, pair) items, two 2-byte elements each; each item is read and
            // written by one thread only, so the in-place update needs no ordering between threads
            const int items = hm_n * np;
            for (int it0 = tid; it0 < items; it0 += kCwThreads * kPairBatch) {
                float xa[kPairBatch], xb[kPairBatch];
#pragma unroll
                for (int j = 0; j < kPairBatch; j++) {
                    const int it = min(it0 + j * kCwThreads, items - 1);
                    const int h = it / np, i = it - h * np;
                    const int a = rm.inter ? rm.off + 2 * i : rm.off + i;
                    const int b = rm.inter ? a + 1 : a + np;
                    xa[j] = bf16_bits_to_f32(base[(int64_t)h * kDqk + a]);
                    xb[j] = bf16_bits_to_f32(base[(int64_t)h * kDqk + b]);
                }
#pragma unroll
                for (int j = 0; j < kPairBatch; j++) {
                    const int it = it0 + j * kCwThreads;
                    if (it >= items) break;
                    const int h = it / np, i = it - h * np;
                    const int a = rm.inter ? rm.off + 2 * i : rm.off + i;
                    const int b = rm.inter ? a + 1 : a + np;
                    const double c = cs_m[i][0], s = cs_m[i][1], x0 = xa[j], x1 = xb[j];
                    base[(int64_t)h * kDqk + a] = f32_to_bf16_bits((float)(x0 * c - x1 * s));
                    base[(int64_t)h * kDqk + b] = f32_to_bf16_bits((float)(x0 * s + x1 * c));
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_cache_append(const void* k_new, int k_dtype, const void* lat_new, int lat_dtype,
                               const int32_t* seq, const int32_t* pos, int T, int num_seqs, const RopeView& k_rope,
                               const RopeView& lat_rope, const CacheView& kc, int kc_dtype, const CacheView& lc,
                               hipStream_t st) {
    if (T == 0) return hipSuccess;
    const int blocks = (T + kCwWaves - 1) / kCwWaves;
    cache_append_kernel<<<blocks, kCwThreads, 0, st>>>(k_new, k_dtype, lat_new, lat_dtype, seq, pos, T, num_seqs,
                                                       k_rope, lat_rope, kc, kc_dtype, lc);
    return hipGetLastError();
}

hipError_t launch_rope_queries(const void* qi_in, int qi_dtype, int Hi, void* qi_out, int qo_dtype, float* qo_scale,
                               const RopeView& ri, uint16_t* qm, int Hm, const RopeView& rm, const int32_t* pos,
                               int T, hipStream_t st) {
    if (T == 0) return hipSuccess;
    // head slices per token: enough workgroups to spread a short batch over the GPU
    const int slices = max(1, min(8, (1024 + T - 1) / T));
    rope_queries_kernel<<<dim3(T, slices), kCwThreads, 0, st>>>(qi_in, qi_dtype, Hi, qi_out, qo_dtype, qo_scale, ri, qm,
                                                                Hm, rm, pos);
    return hipGetLastError();
}

}  // namespace dsa
