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

constexpr int kUnroll = 8;     // 16-byte loads in flight per thread, rows cached in LDS
constexpr int kUnrollLong = 16; // the same for rows read from global memory on every pass
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

// f4(i, keys) for every aligned group of four positions i .. i+3 < n of a score row in global memory
// (16-byte loads, kUnroll of them in flight per thread), then f1(i, key) for the tail positions;
// each position once, in no set order.  Rows that are not 16-byte aligned use f1 throughout.
template <int U, typename F4, typename F1>
__device__ __forceinline__ void for_each_raw4(const float* __restrict__ srow, int n, bool vec, F4&& f4, F1&& f1) {
    const int tid = threadIdx.x;
    int done = 0;
    if (vec) {
        const int n4 = n >> 2;
        const float4* s4 = (const float4*)srow;
        for (int base = 0; base < n4; base += U * kTkBlock) {
            // every load is issued (clamped to the last vector) so that they all stay in flight
            // together; positions past the end are skipped below
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int j = base + u * kTkBlock + tid;
                v[u] = s4[j < n4 ? j : n4 - 1];
            }
            if (base + U * kTkBlock <= n4) {  // uniform: a whole batch, no guards
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const int j = base + u * kTkBlock + tid;
                    f4(4 * j, uint4{order_key(v[u].x), order_key(v[u].y), order_key(v[u].z), order_key(v[u].w)});
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const int j = base + u * kTkBlock + tid;
                    if (j < n4) f4(4 * j, uint4{order_key(v[u].x), order_key(v[u].y), order_key(v[u].z), order_key(v[u].w)});
                }
            }
        }
        done = 4 * n4;
    }
    for (int i = done + tid; i < n; i += kTkBlock) f1(i, order_key(srow[i]));
}

template <typename F>
__device__ __forceinline__ void for_each_raw(const float* __restrict__ srow, int n, bool vec, F&& f) {
    for_each_raw4<kUnrollLong>(srow, n, vec,
                               [&](int i, const uint4& kk) { f(i, kk.x); f(i + 1, kk.y); f(i + 2, kk.z); f(i + 3, kk.w); }, f);
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

// Wave-wide min / max with the same DPP pattern as wave_incl_scan: after the four row shifts the
// last lane of each 16-lane row holds its row's result, the two broadcasts carry it up, and lane
// 63 ends with the wave's result, which readlane hands to every lane.  Out-of-range sources read
// the identity (`old`).
__device__ __forceinline__ uint32_t wave_reduce_max(uint32_t v) {
    int x = (int)v;
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ uint32_t wave_reduce_min(uint32_t v) {
    int x = (int)v;
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x111, 0xf, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x112, 0xf, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x114, 0xf, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x118, 0xf, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x142, 0xa, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

// Ordered compaction: every working-set entry with (key & mask) > thr, plus the first need_eq
// entries with (key & mask) == thr, in entry order.  Wave w owns entries [beg, end) (beg a multiple
// of 256); a step covers 256 entries, lane L holding entries base + 4L .. +3 (one 16-byte read).
// The first pass counts the wave's entries above / equal to the threshold; in the second, an
// inclusive DPP scan over the lanes' packed (above, equal) counts gives every lane the output slot
// of its first take -- equal entries are taken in entry order while the running count of earlier
// equal entries is below need_eq.
template <typename Key4, typename Pos4>
__device__ __forceinline__ void compact(Key4&& key4, Pos4&& pos4, int nw, uint32_t mask, uint32_t thr,
                                        uint32_t need_eq, int k, int32_t* __restrict__ orow,
                                        uint32_t (&wcnt)[2][kTkWaves], int wlo, uint32_t* first_win) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = (((nw + kTkWaves - 1) / kTkWaves) + 255) & ~255;
    const int beg = min(nw, wave * seg), end = min(nw, beg + seg);
    uint32_t cgt = 0, ceq = 0;
    for (int base = beg; base < end; base += 256) {
        const int i0 = base + 4 * lane;
        const uint4 kk = key4(i0, end);
        const uint32_t v[4] = {kk.x & mask, kk.y & mask, kk.z & mask, kk.w & mask};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const bool ok = i0 + j < end;
            cgt += (ok && v[j] > thr) ? 1u : 0u;
            ceq += (ok && v[j] == thr) ? 1u : 0u;
        }
    }
    cgt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cgt), 63);
    ceq = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(ceq), 63);
    if (lane == 0) { wcnt[0][wave] = cgt; wcnt[1][wave] = ceq; }
    __syncthreads();
    uint32_t gt_before = 0, eq_before = 0;
    for (int w = 0; w < wave; w++) { gt_before += wcnt[0][w]; eq_before += wcnt[1][w]; }
    uint32_t pos = gt_before + min(eq_before, need_eq);   // output slot of this wave's next take
    uint32_t eq_rank = eq_before;                          // equal entries before this wave's next
    for (int base = beg; base < end; base += 256) {
        const int i0 = base + 4 * lane;
        const uint4 kk = key4(i0, end);
        const int4 pp = pos4(i0);
        const uint32_t v[4] = {kk.x & mask, kk.y & mask, kk.z & mask, kk.w & mask};
        const int p[4] = {pp.x, pp.y, pp.z, pp.w};
        uint32_t g = 0, e = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const bool ok = i0 + j < end;
            g += (ok && v[j] > thr) ? 1u : 0u;
            e += (ok && v[j] == thr) ? 1u : 0u;
        }
        const uint32_t own = g | (e << 16);                 // at most 256 of each per step
        const uint32_t incl = wave_incl_scan(own);
        const uint32_t excl = incl - own;
        const uint32_t quota = need_eq > eq_rank ? need_eq - eq_rank : 0u;   // equal entries still to take
        uint32_t eq_seen = excl >> 16;
        uint32_t at = pos + (excl & 0xffffu) + min(eq_seen, quota);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const bool ok = i0 + j < end;
            bool take = ok && v[j] > thr;
            if (ok && v[j] == thr) {
                take = eq_seen < quota;
                eq_seen++;
            }
            if (take) {
                if (at < (uint32_t)k) {
                    // positions in the window [wlo, n) are written with the window block; the
                    // first of them marks where that block starts
                    if (p[j] < wlo) orow[at] = p[j];
                    else atomicMin(first_win, at);
                }
                at++;
            }
        }
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        pos += (tot & 0xffffu) + min(tot >> 16, quota);
        eq_rank += tot >> 16;
    }
}

// Query t selects its best kt = clamp(kq[t], 0, k) positions (k when kq is null; all when n <= kt)
// and adds its last `window` positions; the union is written in ascending order to a row of
// `width` = k + window entries, -1 padded.  The plain top-k is kq = null, window = 0.
__global__ __launch_bounds__(kTkBlock) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                        BatchView bv, int k, const int32_t* __restrict__ kq,
                                                        int window, int width, int32_t* __restrict__ out) {
    // cached rows: keys[kCap]; long rows: candidate keys [0, kCandCap) + positions [kCandCap, kCap)
    extern __shared__ __align__(16) uint32_t lds[];
    __shared__ uint32_t hist[kHistCopies][kBins];   // copies shared by alternate waves (fewer collisions)
    __shared__ uint32_t red[2][kTkWaves];
    __shared__ uint32_t sel[3];
    __shared__ uint32_t wcnt[2][kTkWaves];
    __shared__ uint32_t first_win;

    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int32_t* orow = out + (int64_t)t * width;
    const int n = max(0, min(bv.q_len[t], bv.max_len));
    const int kt = kq != nullptr ? max(0, min(kq[t], k)) : k;
    const int wn = min(window, n), wlo = n - wn;   // the window: positions [wlo, n)
    if (n <= kt) {
        for (int i = tid; i < width; i += kTkBlock) orow[i] = i < n ? i : -1;
        return;
    }
    if (kt == 0) {
        for (int i = tid; i < width; i += kTkBlock) orow[i] = i < wn ? wlo + i : -1;
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
    if (mode == kModeCached) {
        for_each_raw4<kUnroll>(
            srow, n, vec,
            [&](int i, const uint4& kk) {
                *(uint4*)(keys + i) = kk;
                lo = min(lo, min(min(kk.x, kk.y), min(kk.z, kk.w)));
                hi = max(hi, max(max(kk.x, kk.y), max(kk.z, kk.w)));
            },
            [&](int i, uint32_t kk) {
                keys[i] = kk;
                lo = min(lo, kk);
                hi = max(hi, kk);
            });
    } else {
        for_each_raw4<kUnrollLong>(
            srow, n, vec,
            [&](int, const uint4& kk) {
                lo = min(lo, min(min(kk.x, kk.y), min(kk.z, kk.w)));
                hi = max(hi, max(max(kk.x, kk.y), max(kk.z, kk.w)));
            },
            [&](int, uint32_t kk) {
                lo = min(lo, kk);
                hi = max(hi, kk);
            });
    }
    lo = wave_reduce_min(lo);
    hi = wave_reduce_max(hi);
    if (lane == 0) { red[0][wave] = lo; red[1][wave] = hi; }
    __syncthreads();
    lo = red[0][0];
    hi = red[1][0];
    for (int w = 1; w < kTkWaves; w++) { lo = min(lo, red[0][w]); hi = max(hi, red[1][w]); }
    __syncthreads();

    // entries i .. i+3 of the working set (positions at or past `end` are never used)
    auto key4 = [&](int i, int end) -> uint4 {
        if (mode != kModeGlobal) return *(const uint4*)(lds + i);
        if (vec && i + 3 < end)
            return uint4{order_key(srow[i]), order_key(srow[i + 1]), order_key(srow[i + 2]), order_key(srow[i + 3])};
        return uint4{i < end ? order_key(srow[i]) : 0u, i + 1 < end ? order_key(srow[i + 1]) : 0u,
                     i + 2 < end ? order_key(srow[i + 2]) : 0u, 0u};
    };
    auto pos4 = [&](int i) -> int4 {
        if (mode == kModeCand) return *(const int4*)(cpos + i);
        return int4{i, i + 1, i + 2, i + 3};
    };

    uint32_t prefix = lo;            // bits resolved so far (under `mask`)
    uint32_t mask = 0xffffffffu;
    uint32_t remaining = (uint32_t)kt; // keys still to take among those matching the prefix

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

    if (tid == 0) first_win = (uint32_t)kt;   // ordered before compact's writes by its barrier
    compact(key4, pos4, nw, mask, thr, need_eq, kt, orow, wcnt, wlo, &first_win);
    if (wn > 0 || width > kt) {
        // the selected positions below the window fill slots [0, c); then the window, then padding
        __syncthreads();
        const int c = (int)first_win;
        for (int i = tid; i < width - c; i += kTkBlock) orow[c + i] = i < wn ? wlo + i : -1;
    }
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t ld, const BatchView& bv, int k, const int32_t* kq, int window,
                       int32_t* idx, hipStream_t st) {
    if (bv.T == 0) return hipSuccess;
    // LDS for the longest row: its keys (rounded up so whole 16-byte reads stay inside), or the
    // candidate area when rows may exceed the key cache
    size_t words = 0;
    // (with a per-query k any query may select, so the key cache is sized for every row)
    if (bv.max_len > (kq != nullptr ? 0 : k))
        words = bv.max_len > kCap ? (size_t)kLdsWords : (size_t)((bv.max_len + 3) & ~3);
    const size_t shm = words * sizeof(uint32_t);
    if (shm > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shm);
        if (e != hipSuccess) return e;
    }
    topk_kernel<<<bv.T, kTkBlock, shm, st>>>(scores, ld, bv, k, kq, window, k + window, idx);
    return hipGetLastError();
}

}  // namespace dsa
