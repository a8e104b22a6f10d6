// topk.hip -- per-query top-k selection for gfx950.
//
// Selection rule (page "一文讀懂DeepSeek-V3.2核心技術DSA", section "DSA 的四步工作流程", top-k
// step): the k positions with the largest indexer scores; a context of at most k tokens selects
// every token.  Equal scores go to the lower position, so the selected set is unique.
//
// One workgroup per query row.  Scores map to order-preserving unsigned keys (-0 is folded onto
// +0 first, so equal reals give equal keys).  A radix select finds the exact k-th largest key
// `thr`: the bits above the common prefix of the row's min and max key are skipped, then 11-bit
// digits are resolved with LDS histograms, each pass keeping only keys that match the prefix found
// so far.  The passes stop early once the bin holding the k-th key is needed whole (usually after
// two passes).  A final ordered compaction writes every key above the threshold plus the
// lowest-position keys equal to it (compared on the resolved bits), in ascending position order,
// which makes the output deterministic.  Rows of up to kCap scores are cached in LDS; longer rows
// are re-read from global memory (L2) on each pass.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kTkBlock = 512;
constexpr int kTkWaves = kTkBlock / 64;
constexpr int kCap = 32768;   // keys cached in LDS (128 KiB)

constexpr int kUnroll = 4;     // 16-byte loads in flight per thread
constexpr int kDigitBits = 11; // radix digit width
constexpr int kBins = 1 << kDigitBits;
constexpr int kHistCopies = 2;

__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;                            // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);       // monotone in the real value
}

// f(i, key) for every position i < n of a score row in global memory (each i once, in no set order).
template <typename F>
__device__ __forceinline__ void for_each_raw(const float* __restrict__ srow, int n, bool vec, F&& f) {
    const int tid = threadIdx.x;
    if (!vec) {
        for (int i = tid; i < n; i += kTkBlock) f(i, order_key(srow[i]));
        return;
    }
    for (int base = 0; base < n; base += kTkBlock * 4 * kUnroll) {
        float4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int i = base + 4 * (u * kTkBlock + tid);
            if (i + 3 < n) {
                v[u] = *(const float4*)(srow + i);
            } else {
                v[u].x = i < n ? srow[i] : 0.0f;
                v[u].y = i + 1 < n ? srow[i + 1] : 0.0f;
                v[u].z = i + 2 < n ? srow[i + 2] : 0.0f;
                v[u].w = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int i = base + 4 * (u * kTkBlock + tid);
            if (i < n) f(i, order_key(v[u].x));
            if (i + 1 < n) f(i + 1, order_key(v[u].y));
            if (i + 2 < n) f(i + 2, order_key(v[u].z));
            if (i + 3 < n) f(i + 3, order_key(v[u].w));
        }
    }
}

// The same over the keys cached in LDS (16-byte reads; the cache is 16-byte aligned).
template <typename F>
__device__ __forceinline__ void for_each_cached(const uint32_t* keys, int n, F&& f) {
    const int tid = threadIdx.x;
    for (int i = 4 * tid; i < n; i += 4 * kTkBlock) {
        const uint4 v = *(const uint4*)(keys + i);
        f(i, v.x);
        if (i + 1 < n) f(i + 1, v.y);
        if (i + 2 < n) f(i + 2, v.z);
        if (i + 3 < n) f(i + 3, v.w);
    }
}

__global__ __launch_bounds__(kTkBlock) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                        BatchView bv, int k, int32_t* __restrict__ out,
                                                        int cap) {
    extern __shared__ __align__(16) uint32_t keys[];   // [cap]
    __shared__ uint32_t hist[kHistCopies][kBins];   // copies shared by alternate waves (fewer collisions)
    __shared__ uint32_t red[2][kTkWaves];
    __shared__ uint32_t sel[3];
    __shared__ uint32_t wcnt[2][kTkWaves];

    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int32_t* orow = out + (int64_t)t * k;
    const int n = max(0, min(bv.q_len[t], bv.max_len));
    if (n <= k) {
        for (int i = tid; i < k; i += kTkBlock) orow[i] = i < n ? i : -1;
        return;
    }
    const float* srow = scores + (int64_t)t * ld;
    const bool cached = n <= cap;

    // keys (cached in LDS when the row fits) and their min / max; the row is read with 16-byte loads,
    // kUnroll of them in flight per thread, when it is 16-byte aligned
    const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
    uint32_t lo = 0xffffffffu, hi = 0u;
    for_each_raw(srow, n, vec, [&](int i, uint32_t kk) {
        if (cached) keys[i] = kk;
        lo = min(lo, kk);
        hi = max(hi, kk);
    });
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) { red[0][wave] = lo; red[1][wave] = hi; }
    __syncthreads();
    lo = red[0][0];
    hi = red[1][0];
    for (int w = 1; w < kTkWaves; w++) { lo = min(lo, red[0][w]); hi = max(hi, red[1][w]); }

    auto key_at = [&](int i) -> uint32_t { return cached ? keys[i] : order_key(srow[i]); };

    uint32_t prefix = lo;            // bits resolved so far (under `mask`)
    uint32_t mask = 0xffffffffu;
    uint32_t remaining = (uint32_t)k; // keys still to take among those matching the prefix
    if (lo != hi) {
        const int top = 31 - __clz(lo ^ hi);                 // highest bit where keys differ
        mask = ~((2u << top) - 1u);                          // top == 31 gives 0
        prefix = lo & mask;
        int pos = top;
        while (pos >= 0) {
            const int width = min(kDigitBits, pos + 1);
            const int shift = pos + 1 - width;
            const uint32_t dmask = (1u << width) - 1u;
            for (int i = tid; i < kHistCopies * kBins; i += kTkBlock) (&hist[0][0])[i] = 0u;
            __syncthreads();
            uint32_t* myhist = hist[wave % kHistCopies];
            auto count = [&](int, uint32_t kk) {
                if ((kk & mask) == prefix) atomicAdd(&myhist[(kk >> shift) & dmask], 1u);
            };
            if (cached) for_each_cached(keys, n, count);
            else for_each_raw(srow, n, vec, count);
            __syncthreads();
            {
                // the digit d with (count above d) < remaining <= (count at or above d): thread t
                // owns bins [4t, 4t + 4); a suffix scan over the block gives the keys above them
                constexpr int kPerThread = kBins / kTkBlock;
                uint32_t c[kPerThread], local = 0u;
#pragma unroll
                for (int j = 0; j < kPerThread; j++) {
                    c[j] = 0u;
#pragma unroll
                    for (int h = 0; h < kHistCopies; h++) c[j] += hist[h][kPerThread * tid + j];
                    local += c[j];
                }
                uint32_t suf = local;                      // sum over this wave's lanes >= lane
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t v = __shfl_down(suf, o, 64);
                    if (lane + o < 64) suf += v;
                }
                if (lane == 0) red[0][wave] = suf;
                __syncthreads();
                uint32_t acc = suf - local;                // keys in bins above this thread's bins
                for (int w = wave + 1; w < kTkWaves; w++) acc += red[0][w];
                if (acc < remaining && remaining <= acc + local) {
#pragma unroll
                    for (int j = kPerThread - 1; j >= 0; j--) {
                        if (remaining <= acc + c[j]) {
                            sel[0] = kPerThread * tid + j;
                            sel[1] = acc;
                            sel[2] = c[j];
                            break;
                        }
                        acc += c[j];
                    }
                }
            }
            __syncthreads();
            const uint32_t d = sel[0], above = sel[1], inbin = sel[2];
            remaining -= above;
            prefix |= d << shift;
            mask |= dmask << shift;
            pos = shift - 1;
            __syncthreads();
            // every key of this bin is needed: the selection is settled without the lower bits
            if (inbin == remaining) break;
        }
    }
    // On the resolved bits (`mask`), `prefix` is now the k-th largest key: all keys above it are
    // taken, and the `remaining` lowest-position keys equal to it (all of them after an early
    // exit, where the bin holds exactly `remaining` keys).
    const uint32_t thr = prefix, need_eq = remaining;

    // ordered compaction: wave w owns positions [beg, end), in steps of 64
    const int seg = (((n + kTkWaves - 1) / kTkWaves) + 63) & ~63;
    const int beg = min(n, wave * seg), end = min(n, beg + seg);
    uint32_t cgt = 0, ceq = 0;
    for (int base = beg; base < end; base += 64) {
        const int i = base + lane;
        const uint32_t kk = i < end ? key_at(i) & mask : 0u;
        cgt += __popcll(__ballot(i < end && kk > thr));
        ceq += __popcll(__ballot(i < end && kk == thr));
    }
    if (lane == 0) { wcnt[0][wave] = cgt; wcnt[1][wave] = ceq; }
    __syncthreads();
    uint32_t gt_before = 0, eq_before = 0;
    for (int w = 0; w < wave; w++) { gt_before += wcnt[0][w]; eq_before += wcnt[1][w]; }
    uint32_t pos = gt_before + min(eq_before, need_eq);
    uint32_t eq_rank = eq_before;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int base = beg; base < end; base += 64) {
        const int i = base + lane;
        const uint32_t kk = i < end ? key_at(i) & mask : 0u;
        const bool gt = i < end && kk > thr;
        const bool eq = i < end && kk == thr;
        const uint64_t beq = __ballot(eq);
        const bool take = gt || (eq && eq_rank + (uint32_t)__popcll(beq & lt_mask) < need_eq);
        const uint64_t btake = __ballot(take);
        const uint32_t at = pos + (uint32_t)__popcll(btake & lt_mask);
        if (take && at < (uint32_t)k) orow[at] = i;
        pos += __popcll(btake);
        eq_rank += __popcll(beq);
    }
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t ld, const BatchView& bv, int k, int32_t* idx,
                       hipStream_t st) {
    if (bv.T == 0) return hipSuccess;
    const int cap = bv.max_len > k ? min(bv.max_len, kCap) : 0;
    const size_t shm = (size_t)((cap + 3) & ~3) * sizeof(uint32_t);   // whole 16-byte reads stay inside
    if (shm > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shm);
        if (e != hipSuccess) return e;
    }
    topk_kernel<<<bv.T, kTkBlock, shm, st>>>(scores, ld, bv, k, idx, cap);
    return hipGetLastError();
}

}  // namespace dsa
