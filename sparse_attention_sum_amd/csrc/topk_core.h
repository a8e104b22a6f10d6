// topk_core.h -- per-query top-k selection for gfx950: the device code of one row's selection,
// shared by the top-k kernels (topk.hip) and the fused indexer -> top-k kernel (indexer_topk.hip).
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
//
// Rows longer than kTwoPassMin, given a workspace, take two passes instead: slices of the row, one
// workgroup each, keep their own best k as candidates, and one workgroup per row selects from their
// union (see TkSlices).  A working set in LDS of which at most an eighth is taken is compacted
// through bitmasks (compact_sparse), a denser one of up to 32 entries per thread in one block-wide
// scan (compact_dense; the final selection of a row without a window is then staged in LDS and
// written with 16-byte stores), and a row read from global memory with a scan per 256 entries
// (compact).
#pragma once

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
constexpr int kTwoPassMin = 32768;   // rows longer than this go through two passes (given a workspace)

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

// The same over keys held in LDS (16-byte reads; the array is 16-byte aligned).  Four reads are
// issued before any f: one at a time, each read also queued behind the LDS atomics of the f calls
// before it.  Reads past the end are clamped to the last aligned group (in bounds, not used).
template <typename F>
__device__ __forceinline__ void for_each_lds(const uint32_t* keys, int n, F&& f) {
    constexpr int U = 4;
    const int tid = threadIdx.x;
    const int last = max(n - 1, 0) & ~3;
    for (int i0 = 4 * tid; i0 < n; i0 += 4 * kTkBlock * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) v[u] = *(const uint4*)(keys + min(i0 + 4 * kTkBlock * u, last));
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int i = i0 + 4 * kTkBlock * u;
            if (i < n) {
                f(i, v[u].x);
                if (i + 1 < n) f(i + 1, v[u].y);
                if (i + 2 < n) f(i + 2, v[u].z);
                if (i + 3 < n) f(i + 3, v[u].w);
            }
        }
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
template <typename Key4, typename Pos4, typename Emit>
__device__ __forceinline__ void compact(Key4&& key4, Pos4&& pos4, int nw, uint32_t mask, uint32_t thr,
                                        uint32_t need_eq, int k, uint32_t (&wcnt)[2][kTkWaves], Emit&& emit) {
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
        const uint32_t raw[4] = {kk.x, kk.y, kk.z, kk.w};
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
                if (at < (uint32_t)k) emit(at, p[j], raw[j]);
                at++;
            }
        }
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        pos += (tot & 0xffffu) + min(tot >> 16, quota);
        eq_rank += tot >> 16;
    }
}

// Ordered compaction of a working set in LDS of at most E * kTkBlock entries in one step: thread t
// owns entries [E t, E t + E) (E / 4 16-byte reads issued together), one block-wide scan over the
// threads' packed counts (above | equal << 16) gives each thread its first output slot and the number
// of equal entries before its own, and the thread emits its taken entries in entry order -- equal
// entries while fewer than need_eq precede them, so the result is the same as compact()'s.
// nw <= E * kTkBlock <= 65535 keeps the packed sums apart.
template <int E, typename Pos4, typename Emit>
__device__ __forceinline__ void compact_dense(const uint32_t* keys, int nw, uint32_t mask, uint32_t thr,
                                              uint32_t need_eq, int k, uint32_t (&wcnt)[2][kTkWaves], Pos4&& pos4,
                                              Emit&& emit) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i0 = E * tid;
    const int last = max(nw - 1, 0) & ~3;   // reads past the end are clamped (in bounds, not used)
    uint32_t v[E];
#pragma unroll
    for (int j = 0; j < E; j += 4) {
        const uint4 kk = *(const uint4*)(keys + min(i0 + j, last));
        v[j] = kk.x;
        v[j + 1] = kk.y;
        v[j + 2] = kk.z;
        v[j + 3] = kk.w;
    }
    uint32_t g = 0, e = 0;
#pragma unroll
    for (int j = 0; j < E; j++) {
        const bool ok = i0 + j < nw;
        g += (ok && (v[j] & mask) > thr) ? 1u : 0u;
        e += (ok && (v[j] & mask) == thr) ? 1u : 0u;
    }
    const uint32_t own = g | (e << 16);
    const uint32_t incl = wave_incl_scan(own);
    if (lane == 63) wcnt[0][wave] = incl;
    __syncthreads();
    uint32_t before = incl - own;
    for (int w = 0; w < wave; w++) before += wcnt[0][w];
    const uint32_t gt_before = before & 0xffffu;
    uint32_t eq_seen = before >> 16;
    uint32_t at = gt_before + min(eq_seen, need_eq);
    if (g == 0 && (e == 0 || eq_seen >= need_eq)) return;   // nothing to take
#pragma unroll
    for (int j = 0; j < E; j += 4) {
        const int4 pp = pos4(min(i0 + j, last));
        const int p[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const int x = j + jj;
            const bool ok = i0 + x < nw;
            const uint32_t m = v[x] & mask;
            bool take = ok && m > thr;
            if (ok && m == thr) {
                take = eq_seen < need_eq;
                eq_seen++;
            }
            if (take) {
                if (at < (uint32_t)k) emit(at, p[jj], v[x]);
                at++;
            }
        }
    }
}

// Ordered compaction of a working set held in LDS of which few entries are taken (keys[i]; entry
// i is position pos_of(i)), through bitmasks instead of per-step scans: each wave marks 64
// consecutive entries per ballot (above the threshold / equal to it), one block-wide scan over the
// packed per-word counts (above | equal << 16) gives every word its first output slot and the number
// of equal entries before it, and the thread owning a word emits its taken entries in entry order.
// Equal entries are taken while fewer than need_eq precede them, so the result is the same as
// compact()'s.  A thread walks its word's taken entries one by one, which pays where they are
// sparse (rows at least 8x longer than k); nw <= 64 * kTkBlock, `bits` holds 2 * 64-bit words per 64 entries.
template <typename PosOf, typename Emit>
__device__ __forceinline__ void compact_sparse(const uint32_t* keys, int nw, uint32_t mask, uint32_t thr,
                                               uint32_t need_eq, int k, uint64_t* bits,
                                               uint32_t (&wcnt)[2][kTkWaves], PosOf&& pos_of, Emit&& emit) {
    constexpr int kMarkUnroll = 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwords = (nw + 63) >> 6;
    // 1. marks: bits[2c] = entries 64c .. 64c+63 above thr, bits[2c + 1] = equal to thr
    for (int c0 = wave; c0 < nwords; c0 += kTkWaves * kMarkUnroll) {
        uint32_t v[kMarkUnroll];
#pragma unroll
        for (int u = 0; u < kMarkUnroll; u++) v[u] = keys[min(64 * (c0 + u * kTkWaves) + lane, max(nw - 1, 0))] & mask;
#pragma unroll
        for (int u = 0; u < kMarkUnroll; u++) {
            const int c = c0 + u * kTkWaves;
            const bool ok = 64 * c + lane < nw;
            const uint64_t g = __ballot(ok && v[u] > thr);
            const uint64_t e = __ballot(ok && v[u] == thr);
            if (lane == 0 && c < nwords) {
                bits[2 * c] = g;
                bits[2 * c + 1] = e;
            }
        }
    }
    __syncthreads();
    // 2. word tid: its first slot and the equal entries before it
    uint64_t g = 0, e = 0;
    if (tid < nwords) {
        g = bits[2 * tid];
        e = bits[2 * tid + 1];
    }
    const uint32_t own = (uint32_t)__popcll(g) | ((uint32_t)__popcll(e) << 16);   // sums stay < 2^16 each
    const uint32_t incl = wave_incl_scan(own);
    if (lane == 63) wcnt[0][wave] = incl;
    __syncthreads();
    uint32_t before = incl - own;
    for (int w = 0; w < wave; w++) before += wcnt[0][w];
    const uint32_t gt_before = before & 0xffffu, eq_before = before >> 16;
    uint64_t take = g;
    if (e != 0) {
        const uint32_t quota = need_eq > eq_before ? need_eq - eq_before : 0u;
        if (quota >= (uint32_t)__popcll(e)) {
            take |= e;
        } else {
            for (uint32_t r = 0; r < quota; r++) {   // the lowest `quota` equal entries of the word
                const uint64_t low = e & (~e + 1);
                take |= low;
                e ^= low;
            }
        }
    }
    // 3. emit in entry order
    uint32_t at = gt_before + min(eq_before, need_eq);
    while (take != 0) {
        const int i = 64 * tid + __builtin_ctzll(take);
        take &= take - 1;
        if (at < (uint32_t)k) emit(at, pos_of(i), keys[i]);
        at++;
    }
}

// Long rows in two passes (workspace): slice s of row t (positions [s * len, (s + 1) * len)) keeps
// its own best kt entries as (key, position) candidates -- the row's best kt are among the union of
// the slices' best kt under the same order -- and one workgroup per row then selects from at most
// nslices * kt candidates, which it holds in LDS in position order.
struct TkSlices {
    uint32_t* ckey;      // [T][nslices][k] candidate keys
    int32_t* cpos;       // [T][nslices][k] candidate positions
    int32_t* ccnt;       // [T][nslices] candidates per slice
    int nslices, slice_len;
};

// The candidates' layout in a workspace: keys, positions, counts, each 256-byte aligned.
inline size_t slices_bytes(int T, int nslices, int k) {
    const size_t half = ((size_t)T * nslices * k * 4 + 255) & ~(size_t)255;
    return 2 * half + (size_t)T * nslices * 4;
}
inline TkSlices slices_in(void* ws, int T, int nslices, int k, int slice_len) {
    const size_t half = ((size_t)T * nslices * k * 4 + 255) & ~(size_t)255;
    TkSlices sl;
    sl.ckey = (uint32_t*)ws;
    sl.cpos = (int32_t*)((uint8_t*)ws + half);
    sl.ccnt = (int32_t*)((uint8_t*)ws + 2 * half);
    sl.nslices = nslices;
    sl.slice_len = slice_len;
    return sl;
}

// Shared memory of one row's selection, besides the dynamic key / candidate area.
struct TkShared {
    __align__(16) uint32_t hist[kHistCopies][kBins];   // copies shared by alternate waves (fewer collisions)
    uint32_t red[2][kTkWaves];
    uint32_t sel[3];
    uint32_t wcnt[2][kTkWaves];
    uint32_t first_win;
    int coff[kTkWaves + 1];
};

// Query t selects its best kt = clamp(kq[t], 0, k) positions (k when kq is null; all when n <= kt)
// and adds its last `window` positions; the union is written in ascending order to a row of
// `width` = k + window entries, -1 padded.  The plain top-k is kq = null, window = 0.
// PASS 0: the whole row in one workgroup; PASS 1: one slice of a row -> candidates; PASS 2: the
// selection from a row's candidates.
// PRE: the row (PASS 1: the slice) is already in lds as keys, and pre_lo / pre_hi are this thread's
// min / max of the keys it stored (the fused indexer -> top-k kernel); otherwise the scores are read
// from `scores`.  lds: cached rows keys[kCap]; long rows candidate keys [0, kCandCap) + positions
// [kCandCap, kCap).
template <int PASS, bool PRE>
__device__ __forceinline__ void topk_row(uint32_t* lds, TkShared& sh, int t, int slice,
                                         const float* __restrict__ scores, int64_t ld, const BatchView& bv, int k,
                                         const int32_t* __restrict__ kq, int window, int width,
                                         int32_t* __restrict__ out, const TkSlices& sl, uint32_t pre_lo,
                                         uint32_t pre_hi) {
    auto& hist = sh.hist;
    auto& red = sh.red;
    auto& sel = sh.sel;
    auto& wcnt = sh.wcnt;
    auto& first_win = sh.first_win;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int32_t* orow = out + (int64_t)t * width;
    const int n = max(0, min(bv.q_len[t], bv.max_len));
    const int kt = kq != nullptr ? max(0, min(kq[t], k)) : k;
    const int wn = min(window, n), wlo = n - wn;   // the window: positions [wlo, n)
    if (n <= kt) {   // (pass 1 writes nothing: pass 2 takes the same exit)
        if (PASS != 1)
            for (int i = tid; i < width; i += kTkBlock) orow[i] = i < n ? i : -1;
        return;
    }
    if (kt == 0) {
        if (PASS != 1)
            for (int i = tid; i < width; i += kTkBlock) orow[i] = i < wn ? wlo + i : -1;
        return;
    }
    // pass 1: this workgroup's slice [s0, s0 + nrow) of the row
    const int s0 = PASS == 1 ? slice * sl.slice_len : 0;
    const int nrow = PASS == 1 ? min(sl.slice_len, n - s0) : n;
    const int64_t cbase = ((int64_t)t * sl.nslices + slice) * k;   // pass 1: this slice's candidate slots
    const int kts = PASS == 1 ? min(kt, nrow) : kt;                // pass 1: the slice keeps its best kts
    const float* srow = scores + (int64_t)t * ld + s0;
    if (PASS == 1) {
        if (nrow <= kts) {   // a slice no longer than kt: every entry is a candidate (nrow <= 0: none)
            for (int i = tid; i < nrow; i += kTkBlock) {
                sl.ckey[cbase + i] = PRE ? lds[i] : order_key(srow[i]);
                sl.cpos[cbase + i] = s0 + i;
            }
            if (tid == 0) sl.ccnt[(int64_t)t * sl.nslices + slice] = max(nrow, 0);
            return;
        }
    }
    uint32_t* keys = lds;
    int32_t* cpos = (int32_t*)(lds + kCandCap);
    int mode = PASS == 2 ? kModeCand : (PRE || nrow <= kCap) ? kModeCached : kModeGlobal;
    int nw = nrow;   // size of the working set

    // keys (cached in LDS when the row fits) and their min / max; the row is read with 16-byte loads,
    // kUnroll of them in flight per thread, when it is 16-byte aligned
    const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
    uint32_t lo = 0xffffffffu, hi = 0u;
    if (PRE) {
        lo = pre_lo;
        hi = pre_hi;
    } else if (PASS == 2) {
        // the row's candidates, slice after slice (each in position order), into LDS
        auto& coff = sh.coff;
        if (tid == 0) {
            int acc = 0;
            for (int sI = 0; sI < sl.nslices; sI++) {
                coff[sI] = acc;
                acc += min(max(sl.ccnt[(int64_t)t * sl.nslices + sI], 0), k);   // (a count is never above k)
            }
            coff[sl.nslices] = acc;
        }
        __syncthreads();
        nw = coff[sl.nslices];
        // the row's workspace slots in order: slot q = s * k + j holds candidate j of slice s when
        // j < ccnt[s], and it goes to list entry coff[s] + j.  Loads run over contiguous slots
        // (kUnroll in flight per thread); a slot's slice comes from offsets held in registers.
        int cb[kTkWaves + 1];
#pragma unroll
        for (int s2 = 0; s2 <= kTkWaves; s2++) cb[s2] = coff[min(s2, sl.nslices)];
        const int tot = sl.nslices * k;
        const int64_t src0 = (int64_t)t * sl.nslices * k;
        for (int q0 = tid; q0 < tot; q0 += kTkBlock * kUnroll) {
            uint32_t kk[kUnroll];
            int32_t pp[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                const int q = min(q0 + u * kTkBlock, tot - 1);
                kk[u] = sl.ckey[src0 + q];
                pp[u] = sl.cpos[src0 + q];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                const int q = q0 + u * kTkBlock;
                int d0 = cb[0], d1 = cb[1], base = 0;
#pragma unroll
                for (int s2 = 1; s2 < kTkWaves; s2++)
                    if (s2 < sl.nslices && q >= s2 * k) {
                        d0 = cb[s2];
                        d1 = cb[s2 + 1];
                        base = s2 * k;
                    }
                const int d = d0 + (q - base);
                if (q < tot && d < d1) {
                    keys[d] = kk[u];
                    cpos[d] = pp[u];
                    lo = min(lo, kk[u]);
                    hi = max(hi, kk[u]);
                }
            }
        }
    } else if (mode == kModeCached) {
        for_each_raw4<kUnroll>(
            srow, nrow, vec,
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
            srow, nrow, vec,
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
    uint32_t remaining = (uint32_t)kts; // keys still to take among those matching the prefix

    // Ordered gather of the candidates (keys with (key & mask) >= prefix) of a long row into LDS:
    // thread t takes keys [base + 16 t, +16) of each step, a block-wide prefix sum gives their
    // slots, and the next step's scores are loaded while this one is processed.  Returns false
    // (and keeps the row in global memory) if there are more than kCandCap.
    auto gather = [&]() -> bool {
        uint32_t total = 0;
        constexpr int kStep = kTkBlock * kGatherKeys;
        float cur[kGatherKeys], nxt[kGatherKeys];
        load_run(srow, nrow, vec, kGatherKeys * tid, cur);
        for (int base = 0; base < nrow; base += kStep) {
            const int i0 = base + kGatherKeys * tid;
            if (base + kStep < nrow) load_run(srow, nrow, vec, i0 + kStep, nxt);
            uint32_t kk[kGatherKeys], c = 0;
#pragma unroll
            for (int j = 0; j < kGatherKeys; j++) {
                kk[j] = order_key(cur[j]);
                c += (i0 + j < nrow && (kk[j] & mask) >= prefix) ? 1u : 0u;
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
                if (i0 + j < nrow && (kk[j] & mask) >= prefix) {
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
            for (int i = 4 * tid; i < kHistCopies * kBins; i += 4 * kTkBlock) *(uint4*)(&hist[0][0] + i) = uint4{0u, 0u, 0u, 0u};
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
                static_assert(kPerThread == 4 && kHistCopies == 2, "a thread's bins: one 16-byte read per copy");
                uint32_t c[kPerThread], local = 0u;
                const uint4 c0 = *(const uint4*)&hist[0][kPerThread * tid];
                const uint4 c1 = *(const uint4*)&hist[1][kPerThread * tid];
                c[0] = c0.x + c1.x;
                c[1] = c0.y + c1.y;
                c[2] = c0.z + c1.z;
                c[3] = c0.w + c1.w;
                local = (c[0] + c[1]) + (c[2] + c[3]);
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

    // a working set in LDS of which at most an eighth is taken is compacted through bitmasks (kept
    // in the histogram's space, which the selection no longer needs)
    static_assert(2 * (kCap / 64) * 2 <= kHistCopies * kBins, "bitmasks must fit the histogram space");
    auto pos_of = [&](int i) -> int { return mode == kModeCand ? cpos[i] : i; };
    // working sets in LDS: at least 8x longer than the count taken -> bitmasks; up to 16 or 32 entries
    // per thread -> one block-wide scan; otherwise (long rows read from global memory) a scan per step
    auto compact_any = [&](int kk, auto&& emit) {
        if (mode != kModeGlobal && nw >= 8 * kk)
            compact_sparse(lds, nw, mask, thr, need_eq, kk, reinterpret_cast<uint64_t*>(&hist[0][0]), wcnt, pos_of, emit);
        else if (mode != kModeGlobal && nw <= 16 * kTkBlock)
            compact_dense<16>(lds, nw, mask, thr, need_eq, kk, wcnt, pos4, emit);
        else if (mode != kModeGlobal && nw <= 32 * kTkBlock)
            compact_dense<32>(lds, nw, mask, thr, need_eq, kk, wcnt, pos4, emit);
        else
            compact(key4, pos4, nw, mask, thr, need_eq, kk, wcnt, emit);
    };
    if (PASS == 1) {   // the slice's best kts as candidates, in position order
        compact_any(kts, [&](uint32_t at, int pos, uint32_t key) {
            sl.ckey[cbase + at] = key;
            sl.cpos[cbase + at] = s0 + pos;
        });
        if (tid == 0) sl.ccnt[(int64_t)t * sl.nslices + slice] = kts;
        return;
    }
    // no window, a dense working set in LDS and a 16-byte aligned row: the selection is staged in
    // the histogram space (free now; the dense compaction does not use it) and written with one
    // 16-byte store per four entries, instead of a 4-byte store per entry from the compaction's
    // threads (top-k at decode 64 x 8192 13.1 -> 12.5 us)
    if (wn == 0 && mode != kModeGlobal && nw < 8 * kt && nw <= 32 * kTkBlock && kt <= kHistCopies * kBins &&
        (reinterpret_cast<uintptr_t>(orow) & 15) == 0) {
        int32_t* stage = reinterpret_cast<int32_t*>(&hist[0][0]);
        auto put = [&](uint32_t at, int pos, uint32_t) { stage[at] = pos; };
        if (nw <= 16 * kTkBlock)
            compact_dense<16>(lds, nw, mask, thr, need_eq, kt, wcnt, pos4, put);
        else
            compact_dense<32>(lds, nw, mask, thr, need_eq, kt, wcnt, pos4, put);
        __syncthreads();
        for (int i = 4 * tid; i < kt; i += 4 * kTkBlock) {
            if (i + 3 < kt) *(int4*)(orow + i) = *(const int4*)(stage + i);
            else for (int j = i; j < kt; j++) orow[j] = stage[j];
        }
        for (int i = kt + tid; i < width; i += kTkBlock) orow[i] = -1;
        return;
    }
    if (tid == 0) first_win = (uint32_t)kt;   // ordered before compact's writes by its barrier
    // positions in the window [wlo, n) are written with the window block; the first of them marks
    // where that block starts
    compact_any(kt, [&](uint32_t at, int pos, uint32_t) {
        if (pos < wlo) orow[at] = pos;
        else atomicMin(&first_win, at);
    });
    if (wn > 0 || width > kt) {
        // the selected positions below the window fill slots [0, c); then the window, then padding
        __syncthreads();
        const int c = (int)first_win;
        for (int i = tid; i < width - c; i += kTkBlock) orow[c + i] = i < wn ? wlo + i : -1;
    }
}

}  // namespace
}  // namespace dsa
