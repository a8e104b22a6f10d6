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
// which makes the output deterministic.
//
// Working set: rows of up to kCap scores are cached in LDS as keys.  Longer rows are read from
// global memory for the min/max and the first digit pass; then the candidates -- keys at or above
// the bin of the k-th key, at most k plus that bin -- are gathered with their positions into LDS
// in position order, and every later pass and the compaction run on them.  (Should the candidates
// not fit, the row is simply re-read from global memory on each pass.)
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kTkBlock = 512;
constexpr int kTkWaves = kTkBlock / 64;
constexpr int kCap = 32768;          // keys cached in LDS (128 KiB)
constexpr int kCandCap = kCap / 2;   // candidates of a long row: keys + positions (128 KiB)
constexpr int kLdsWords = kCap;      // dynamic LDS words of a launch whose rows may exceed kCap

constexpr int kUnroll = 16;    // 16-byte loads in flight per thread
constexpr int kDigitBits = 11; // radix digit width
constexpr int kBins = 1 << kDigitBits;
constexpr int kHistCopies = 2;
constexpr int kGatherKeys = 16;  // consecutive keys per thread per step of the candidate gather

enum { kModeCached = 0, kModeGlobal = 1, kModeCand = 2 };

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

// The same over keys held in LDS (16-byte reads; the array is 16-byte aligned).
template <typename F>
__device__ __forceinline__ void for_each_lds(const uint32_t* keys, int n, F&& f) {
    const int tid = threadIdx.x;
    for (int i = 4 * tid; i < n; i += 4 * kTkBlock) {
        const uint4 v = *(const uint4*)(keys + i);
        f(i, v.x);
        if (i + 1 < n) f(i + 1, v.y);
        if (i + 2 < n) f(i + 2, v.z);
        if (i + 3 < n) f(i + 3, v.w);
    }
}

// kGatherKeys consecutive scores starting at i0 (positions past n read as 0, never used)
__device__ __forceinline__ void load_run(const float* __restrict__ srow, int n, bool vec, int i0,
                                         float (&v)[kGatherKeys]) {
    if (vec && i0 + kGatherKeys <= n) {
#pragma unroll
        for (int j = 0; j < kGatherKeys; j += 4) {
            const float4 f = *(const float4*)(srow + i0 + j);
            v[j] = f.x; v[j + 1] = f.y; v[j + 2] = f.z; v[j + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kGatherKeys; j++) v[j] = i0 + j < n ? srow[i0 + j] : 0.0f;
    }
}

// Inclusive prefix sum over the wave's 64 lanes with DPP moves (no LDS round trips): shifts
// within each row of 16 lanes, then the last lane of row 0 / rows 0-1 is broadcast into the rows
// above it.  Lanes whose source is out of range take 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return (uint32_t)x;
}

// Ordered compaction: every working-set entry with (key & mask) > thr, plus the first need_eq
// entries with (key & mask) == thr, in entry order.  Wave w owns entries [beg, end); an iteration
// covers 256 entries as four groups of 64 consecutive ones (one per lane), so each group's slots
// come from a ballot and a popcount, and the four loads of an iteration are in flight together.
template <typename KeyAt, typename PosAt>
__device__ __forceinline__ void compact(KeyAt&& key_at, PosAt&& pos_at, int nw, uint32_t mask, uint32_t thr,
                                        uint32_t need_eq, int k, int32_t* __restrict__ orow,
                                        uint32_t (&wcnt)[2][kTkWaves]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = (((nw + kTkWaves - 1) / kTkWaves) + 255) & ~255;
    const int beg = min(nw, wave * seg), end = min(nw, beg + seg);
    uint32_t cgt = 0, ceq = 0;
    for (int base = beg; base < end; base += 256) {
        uint32_t kk[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int i = base + 64 * j + lane;
            kk[j] = i < end ? key_at(i) & mask : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int i = base + 64 * j + lane;
            cgt += __popcll(__ballot(i < end && kk[j] > thr));
            ceq += __popcll(__ballot(i < end && kk[j] == thr));
        }
    }
    if (lane == 0) { wcnt[0][wave] = cgt; wcnt[1][wave] = ceq; }
    __syncthreads();
    uint32_t gt_before = 0, eq_before = 0;
    for (int w = 0; w < wave; w++) { gt_before += wcnt[0][w]; eq_before += wcnt[1][w]; }
    uint32_t pos = gt_before + min(eq_before, need_eq);   // output slot of this wave's next take
    uint32_t eq_rank = eq_before;                          // equal entries before this wave's next
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int base = beg; base < end; base += 256) {
        uint32_t kk[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int i = base + 64 * j + lane;
            kk[j] = i < end ? key_at(i) & mask : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int i = base + 64 * j + lane;
            const bool gt = i < end && kk[j] > thr;
            const bool eq = i < end && kk[j] == thr;
            const uint64_t beq = __ballot(eq);
            const bool take = gt || (eq && eq_rank + (uint32_t)__popcll(beq & lt_mask) < need_eq);
            const uint64_t btake = __ballot(take);
            const uint32_t at = pos + (uint32_t)__popcll(btake & lt_mask);
            if (take && at < (uint32_t)k) orow[at] = pos_at(i);
            pos += __popcll(btake);
            eq_rank += __popcll(beq);
        }
    }
}

__global__ __launch_bounds__(kTkBlock) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                        BatchView bv, int k, int32_t* __restrict__ out) {
    // cached rows: keys[kCap]; long rows: candidate keys [0, kCandCap) + positions [kCandCap, kCap)
    extern __shared__ __align__(16) uint32_t lds[];
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
    uint32_t* keys = lds;
    int32_t* cpos = (int32_t*)(lds + kCandCap);
    int mode = n <= kCap ? kModeCached : kModeGlobal;
    int nw = n;   // size of the working set

    // keys (cached in LDS when the row fits) and their min / max; the row is read with 16-byte loads,
    // kUnroll of them in flight per thread, when it is 16-byte aligned
    const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
    uint32_t lo = 0xffffffffu, hi = 0u;
    {
        const bool cache = mode == kModeCached;
        for_each_raw(srow, n, vec, [&](int i, uint32_t kk) {
            if (cache) keys[i] = kk;
            lo = min(lo, kk);
            hi = max(hi, kk);
        });
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) { red[0][wave] = lo; red[1][wave] = hi; }
    __syncthreads();
    lo = red[0][0];
    hi = red[1][0];
    for (int w = 1; w < kTkWaves; w++) { lo = min(lo, red[0][w]); hi = max(hi, red[1][w]); }
    __syncthreads();

    auto key_at = [&](int i) -> uint32_t { return mode == kModeGlobal ? order_key(srow[i]) : lds[i]; };
    auto pos_at = [&](int i) -> int { return mode == kModeCand ? cpos[i] : i; };

    uint32_t prefix = lo;            // bits resolved so far (under `mask`)
    uint32_t mask = 0xffffffffu;
    uint32_t remaining = (uint32_t)k; // keys still to take among those matching the prefix

    // Ordered gather of the candidates (keys with (key & mask) >= prefix) of a long row into LDS:
    // thread t takes keys [base + 16 t, +16) of each step, a block-wide prefix sum gives their
    // slots, and the next step's scores are loaded while this one is processed.  Returns false
    // (and keeps the row in global memory) if there are more than kCandCap.
    auto gather = [&]() -> bool {
        uint32_t total = 0;
        constexpr int kStep = kTkBlock * kGatherKeys;
        float cur[kGatherKeys], nxt[kGatherKeys];
        load_run(srow, n, vec, kGatherKeys * tid, cur);
        for (int base = 0; base < n; base += kStep) {
            const int i0 = base + kGatherKeys * tid;
            if (base + kStep < n) load_run(srow, n, vec, i0 + kStep, nxt);
            uint32_t kk[kGatherKeys], c = 0;
#pragma unroll
            for (int j = 0; j < kGatherKeys; j++) {
                kk[j] = order_key(cur[j]);
                c += (i0 + j < n && (kk[j] & mask) >= prefix) ? 1u : 0u;
            }
            const uint32_t incl = wave_incl_scan(c);   // inclusive prefix over the wave's lanes
            if (lane == 63) red[0][wave] = incl;
            __syncthreads();
            uint32_t at = total + incl - c;
            for (int w = 0; w < kTkWaves; w++) {
                const uint32_t s = red[0][w];
                if (w < wave) at += s;
                total += s;
            }
#pragma unroll
            for (int j = 0; j < kGatherKeys; j++) {
                if (i0 + j < n && (kk[j] & mask) >= prefix) {
                    if (at < (uint32_t)kCandCap) {
                        lds[at] = kk[j];
                        cpos[at] = i0 + j;
                    }
                    at++;
                }
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kGatherKeys; j++) cur[j] = nxt[j];
        }
        if (total > (uint32_t)kCandCap) return false;
        nw = (int)total;
        return true;
    };

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
            if (mode == kModeGlobal) for_each_raw(srow, nw, vec, count);
            else for_each_lds(lds, nw, count);
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
                const uint32_t incl = wave_incl_scan(local);
                const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
                const uint32_t suf = wtot - incl + local;  // sum over this wave's lanes >= lane
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
            // a long row continues on its candidates: every key above the bin and the bin itself
            if (mode == kModeGlobal && gather()) mode = kModeCand;
            // every key of this bin is needed: the selection is settled without the lower bits
            if (inbin == remaining) break;
        }
    }
    // On the resolved bits (`mask`), `prefix` is now the k-th largest key: all keys above it are
    // taken, and the `remaining` lowest-position keys equal to it (all of them after an early
    // exit, where the bin holds exactly `remaining` keys).  (All keys equal: the first k.)
    const uint32_t thr = prefix, need_eq = remaining;

    compact(key_at, pos_at, nw, mask, thr, need_eq, k, orow, wcnt);
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t ld, const BatchView& bv, int k, int32_t* idx,
                       hipStream_t st) {
    if (bv.T == 0) return hipSuccess;
    // LDS for the longest row: its keys (rounded up so whole 16-byte reads stay inside), or the
    // candidate area when rows may exceed the key cache
    size_t words = 0;
    if (bv.max_len > k) words = bv.max_len > kCap ? (size_t)kLdsWords : (size_t)((bv.max_len + 3) & ~3);
    const size_t shm = words * sizeof(uint32_t);
    if (shm > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shm);
        if (e != hipSuccess) return e;
    }
    topk_kernel<<<bv.T, kTkBlock, shm, st>>>(scores, ld, bv, k, idx);
    return hipGetLastError();
}

}  // namespace dsa
