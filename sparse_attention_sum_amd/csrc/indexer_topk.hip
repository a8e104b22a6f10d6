// indexer_topk.hip -- the lightning indexer fused with the first pass of the two-pass top-k, for long
// decode rows, so that the scores never leave the chip (page "DeepSeek 稀疏注意力路线（V3 / V3.2 /
// V4）", section "两阶段流程", items 1-2: the indexer scores every past token and only the top-k of
// those scores are kept; page "一文讀懂DeepSeek-V3.2核心技術DSA", "DSA 的四步工作流程", steps 2-3).
//
// One workgroup of 8 waves per (sequence, slice of its positions).  For every group of the sequence's
// query tokens (one, or two for two-token decode, sharing each key fetch):
//   1. the slice's keys stream from HBM straight into MFMA operands (v_mfma_f32_32x32x64_f8f6f4), each
//      wave keeping PF 32-key subtiles in flight; the score of every position is computed with the
//      same instructions as the decode indexer (indexer_fp8.h), so it is the same binary32 value, and
//      stored in LDS as the top-k's order-preserving key;
//   2. the slice's best k (key, position) pairs are selected from LDS by the top-k's own code
//      (topk_row, topk_core.h) and written to the workspace as candidates.
// The top-k's merge pass (launch_topk_merge) then selects each row's k from the union of its slices'
// candidates, exactly as after the unfused first pass: the selection is bit-identical to
// dsa_indexer_scores followed by dsa_topk.
#include "indexer_fp8.h"
#include "topk_core.h"

namespace dsa {
namespace {

constexpr int kFuMinPage = 16;   // smallest page size taken (the slice's page table lives in LDS)
constexpr int kFuSplitMin = 8192;   // a row that fits one slice is split only into slices this long

// PASS 1: the slice's best k go to the workspace as candidates (a merge pass follows).  PASS 0: the
// slice is the whole row (n <= 32768 / QG): the selection is final and written to idx [T][k].
template <int NHS, int QG, int PASS>
__global__ __launch_bounds__(kTkBlock) void indexer_topk_kernel(const uint8_t* __restrict__ q,
                                                                const float* __restrict__ q_scale,
                                                                const float* __restrict__ w, CacheView kc,
                                                                BatchView bv, float scale, int k, TkSlices sl,
                                                                int32_t* __restrict__ idx) {
    constexpr int H = 32 * NHS;
    // subtiles in flight per wave (registers: 17 per subtile).  Four for one query: measured at decode
    // 64 x 131072 (fused stage 223.9-225.5 us against 228.7-228.8 with six, 248-249 with eight) and in
    // the 64 x 65536 forward (190.6-191.0 against 192.8-194.2 us); the scores are the same either way.
    constexpr int PF = QG == 1 ? 4 : 3;
    // LDS: the scores of QG rows over the slice as keys, then the slice's page table
    extern __shared__ __align__(16) uint32_t lds[];
    __shared__ TkShared sh;
    __shared__ __align__(16) float wsh[QG][H];   // w * q_scale of the pass's queries

    const int slice = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    const int slen = sl.slice_len;
    const int s0 = slice * slen;
    int qb = bv.cu_q[b], qe = bv.cu_q[b + 1];
    qb = max(0, min(qb, bv.T));
    qe = max(qb, min(qe, bv.T));
    if (qb >= qe) return;

    // paged layout: the slice's pages (their first storage row, -1 when the page is invalid)
    const bool paged = kc.page_table != nullptr;
    const int ps = kc.page_size;
    const int first_page = paged ? s0 / ps : 0;
    int32_t* ptab = (int32_t*)(lds + QG * slen);
    if (paged) {
        const int npages = (s0 + slen - 1) / ps - first_page + 1;
        for (int i = tid; i < npages; i += kTkBlock) {
            const int pi = first_page + i;
            const int64_t page = pi < kc.pt_stride ? kc.page_table[(int64_t)b * kc.pt_stride + pi] : -1;
            const int64_t row0 = page * ps;
            ptab[i] = (page >= 0 && row0 < kc.num_rows) ? (int32_t)page : -1;
        }
    }

    for (int t0 = qb; t0 < qe; t0 += QG) {
        const int nq = min(QG, qe - t0);
        // positions of this slice each row needs: rows with n <= k take every position in the merge
        int n[QG], nrow[QG];
        int nstream = 0;
#pragma unroll
        for (int u = 0; u < QG; u++) {
            n[u] = u < nq ? max(0, min(bv.q_len[t0 + u], bv.max_len)) : 0;
            nrow[u] = n[u] > k ? max(0, min(slen, n[u] - s0)) : 0;
            nstream = max(nstream, nrow[u]);
        }
        __syncthreads();   // the previous group's selection is done with wsh and the key area
        for (int i = tid; i < QG * H; i += kTkBlock) {
            const int u = i / H, j = i % H;
            const int t = t0 + min(u, nq - 1);
            const float sc = q_scale ? q_scale[(int64_t)t * H + j] : 1.0f;
            wsh[u][j] = u < nq ? w[(int64_t)t * H + j] * sc : 0.0f;
        }
        __syncthreads();   // wsh and the page table

        uint32_t lo[QG], hi[QG];
#pragma unroll
        for (int u = 0; u < QG; u++) { lo[u] = 0xffffffffu; hi[u] = 0u; }
        const int nsub = (nstream + 31) / 32;
        const int nmy = nsub > wave ? (nsub - wave + kTkWaves - 1) / kTkWaves : 0;   // this wave's subtiles
        if (nmy > 0) {
            // this wave's query operands: head 32 hs + c, dims 64 g + [0, 64)
            i32x8 qf[QG][NHS][2];
#pragma unroll
            for (int u = 0; u < QG; u++) {
                const int t = t0 + (u < nq ? u : 0);
#pragma unroll
                for (int hs = 0; hs < NHS; hs++) {
                    const uint8_t* src = q + ((int64_t)t * H + 32 * hs + c) * kIdxDim + 64 * g;
                    qf[u][hs][0] = *(const i32x8*)(src);
                    qf[u][hs][1] = *(const i32x8*)(src + 32);
                }
            }
            // wave w takes subtiles w, w + 8, w + 16, ... of the slice; every load is issued, from a
            // position clamped to the last one streamed (in bounds; its score is not stored)
            i32x8 kf[PF][2];
            float ks[PF];
            uint32_t okm = 0;   // bit j: ring slot j holds a valid key row
            auto issue = [&](int j, int i) {
                const int pos = min(32 * (wave + kTkWaves * min(i, nmy - 1)) + c, nstream - 1);
                const int s = s0 + pos;
                int64_t row;
                bool ok = true;
                if (!paged) {
                    row = (int64_t)b * kc.seq_stride + s;
                } else {
                    const int pg = ptab[s / ps - first_page];
                    row = (int64_t)pg * ps + s % ps;
                    ok = pg >= 0 && row < kc.num_rows;
                    row = ok ? row : 0;
                }
                const uint8_t* src = (const uint8_t*)kc.data + row * kIdxDim + 64 * g;
                kf[j][0] = *(const i32x8*)(src);
                kf[j][1] = *(const i32x8*)(src + 32);
                ks[j] = kc.scale ? kc.scale[row] : 1.0f;
                okm = ok ? (okm | (1u << j)) : (okm & ~(1u << j));
            };
#pragma unroll
            for (int j = 0; j < PF; j++) issue(j, j);
            for (int i0 = 0; i0 < nmy; i0 += PF) {
#pragma unroll
                for (int j = 0; j < PF; j++) {
                    const int pos = 32 * (wave + kTkWaves * (i0 + j)) + c;
                    // an invalid page reads as an all-zero row (score exactly 0)
                    const bool ok = (okm >> j) & 1u;
                    const i32x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
                    const i32x8 k0 = ok ? kf[j][0] : zero, k1 = ok ? kf[j][1] : zero;
                    const float ksj = ok ? ks[j] : 0.0f;
                    // With two queries the weights' LDS address passes through an empty asm at every
                    // subtile, so that the compiler does not hoist the weight reads out of the loop:
                    // held, they took 32 registers per query and the two-query kernel spilled (the
                    // values, and so the scores, are the same either way).  One query keeps them held.
                    uint32_t wbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&wsh[0][0];
                    if constexpr (QG > 1) asm volatile("" : "+v"(wbase));
#pragma unroll
                    for (int u = 0; u < QG; u++) {
                        const float sum = fp8_head_sum<NHS>(
                            qf[u], k0, k1,
                            [&](int i) {
                                if constexpr (QG == 1) return *(const f32x4*)&wsh[u][i];
                                typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
                                return *(lds_f32x4*)(uintptr_t)(wbase + 4u * (uint32_t)(u * H + i));
                            },
                            g);
                        if (g == 0 && i0 + j < nmy && pos < nrow[u]) {
                            const uint32_t key = order_key(fp8_score(scale, ksj, sum));
                            lds[u * slen + pos] = key;
                            lo[u] = min(lo[u], key);
                            hi[u] = max(hi[u], key);
                        }
                    }
                    issue(j, i0 + j + PF);
                }
            }
        }
        __syncthreads();   // every key of the slice is in LDS
#pragma unroll 1
        for (int u = 0; u < nq; u++) {   // one copy of the selection code, run once per row
            if (u > 0) __syncthreads();   // the previous row's selection is done with sh
            const uint32_t l = (QG > 1 && u > 0) ? lo[QG - 1] : lo[0];
            const uint32_t h = (QG > 1 && u > 0) ? hi[QG - 1] : hi[0];
            topk_row<PASS, true>(lds + u * slen, sh, t0 + u, slice, nullptr, 0, bv, k, nullptr, 0, k, idx, sl, l, h);
        }
    }
}

// Rows of at most 32768 / qg positions take one slice (the whole row, no merge), or, when that leaves
// CUs idle, slices of at least kFuSplitMin positions.  Longer rows: the fewest slices (at most 8, as
// the merge allows, each at most 32768 / qg keys so that its keys fit LDS) that give about one
// workgroup per CU over the batch's sequences.
bool plan_slices(const BatchView& bv, int k, int qg, int& ns, int& slen) {
    if (k <= 0 || bv.T <= 0 || bv.max_len <= k) return false;
    if ((int64_t)bv.max_len * qg <= kCap) {
        // the row fits one slice; when one workgroup per sequence would leave CUs idle, it is split
        // into slices of at least kFuSplitMin positions (measured: 64 x 32768 as four slices of 8192,
        // indexer + top-k 81 us against 87 unfused and 150 as one slice; slices of 4096 lost to the
        // unfused pair, their merge outweighing the extra workgroups)
        const int ns_fill = (256 + bv.B - 1) / bv.B;
        const int nsp = min(min(ns_fill, min(kTkWaves, kCandCap / k)), bv.max_len / kFuSplitMin);
        ns = nsp >= 2 ? nsp : 1;
        slen = ((bv.max_len + ns - 1) / ns + 3) & ~3;
        return true;
    }
    if (bv.max_len <= kTwoPassMin) return false;
    const int cap = kCap / qg;
    const int ns_lds = (bv.max_len + cap - 1) / cap;
    const int ns_max = min(kTkWaves, kCandCap / k);
    const int ns_fill = (256 + bv.B - 1) / bv.B;
    ns = min(max(max(2, ns_lds), ns_fill), ns_max);
    if (ns < max(2, ns_lds)) return false;
    slen = ((bv.max_len + ns - 1) / ns + 3) & ~3;
    return slen * qg <= kCap;
}

}  // namespace

bool indexer_topk_plan(int dtype, int H, const CacheView& kc, const BatchView& bv, int k, int* nslices,
                       int* slice_len, size_t* ws_bytes) {
    if (dtype != DSA_FP8_E4M3 || (H != 32 && H != 64) || bv.max_q > 2) return false;
    if (kc.page_table != nullptr && kc.page_size < kFuMinPage) return false;
    int ns = 0, slen = 0;
    if (!plan_slices(bv, k, bv.max_q, ns, slen)) return false;
    *nslices = ns;
    *slice_len = slen;
    *ws_bytes = ns > 1 ? slices_bytes(bv.T, ns, k) : 0;
    return true;
}

bool indexer_topk_rows_exceed_slice(const BatchView& bv) { return (int64_t)bv.max_len * bv.max_q > kCap; }

size_t indexer_topk_workspace_bound(const BatchView& bv, int k) {
    if (k <= 0 || bv.T <= 0) return 0;
    if ((int64_t)bv.max_len * bv.max_q <= kCap && bv.max_len < 2 * kFuSplitMin) return 0;   // one slice: no candidates
    return slices_bytes(bv.T, min(kTkWaves, kCandCap / max(k, 1)), k);
}

hipError_t launch_indexer_topk(const uint8_t* q, const float* q_scale, const float* w, int H, const CacheView& kc,
                               const BatchView& bv, float scale, int k, int32_t* idx, void* ws, hipStream_t st) {
    int ns = 0, slen = 0;
    size_t bytes = 0;
    if (!indexer_topk_plan(DSA_FP8_E4M3, H, kc, bv, k, &ns, &slen, &bytes)) return hipErrorInvalidValue;
    const TkSlices sl = ns > 1 ? slices_in(ws, bv.T, ns, k, slen) : TkSlices{nullptr, nullptr, nullptr, 1, slen};
    const int qg = bv.max_q;
    const int npages = kc.page_table ? (slen + kc.page_size - 1) / kc.page_size + 1 : 0;
    const size_t shm = ((size_t)qg * slen + npages) * sizeof(uint32_t);
    const dim3 grid(ns, bv.B);
    hipError_t e = hipSuccess;
    auto go = [&](auto kern) {
        e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        if (e == hipSuccess) {
            kern<<<grid, kTkBlock, shm, st>>>(q, q_scale, w, kc, bv, scale, k, sl, idx);
            e = hipGetLastError();
        }
    };
    if (ns == 1) {   // the whole row in one workgroup: the selection is final
        if (qg == 1) {
            if (H == 32) go(indexer_topk_kernel<1, 1, 0>);
            else go(indexer_topk_kernel<2, 1, 0>);
        } else {
            if (H == 32) go(indexer_topk_kernel<1, 2, 0>);
            else go(indexer_topk_kernel<2, 2, 0>);
        }
        return e;
    }
    if (qg == 1) {
        if (H == 32) go(indexer_topk_kernel<1, 1, 1>);
        else go(indexer_topk_kernel<2, 1, 1>);
    } else {
        if (H == 32) go(indexer_topk_kernel<1, 2, 1>);
        else go(indexer_topk_kernel<2, 2, 1>);
    }
    if (e != hipSuccess) return e;
    return launch_topk_merge(bv, k, ws, ns, slen, idx, st);
}

}  // namespace dsa
