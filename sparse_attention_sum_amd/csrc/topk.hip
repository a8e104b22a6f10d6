// topk.hip -- the top-k kernels and their launch: one workgroup per row (or per slice of a long
// row, then one per row for the merge); the selection itself is topk_row in topk_core.h.
#include "topk_core.h"

namespace dsa {
namespace {

template <int PASS>
__global__ __launch_bounds__(kTkBlock) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                        BatchView bv, int k, const int32_t* __restrict__ kq,
                                                        int window, int width, int32_t* __restrict__ out,
                                                        TkSlices sl) {
    extern __shared__ __align__(16) uint32_t lds[];
    __shared__ TkShared sh;
    topk_row<PASS, false>(lds, sh, blockIdx.x, PASS == 1 ? (int)blockIdx.y : 0, scores, ld, bv, k, kq, window, width,
                          out, sl, 0u, 0u);
}

}  // namespace

// Two passes when a workspace is given and the rows are long: up to 8 slices per row (the merge
// keeps nslices * k candidates in LDS), each slice short enough to be cached in LDS.
static bool topk_two_pass(const BatchView& bv, int k, int& nslices, int& slice_len) {
    if (bv.max_len <= kTwoPassMin || k <= 0) return false;
    // as few slices as the LDS key cache allows (a slice workgroup holds up to kCap keys, one per
    // CU): more slices mean more rounds of workgroups and a longer merge
    nslices = min(min(kTkWaves, kCandCap / k), max(2, (bv.max_len + kCap - 1) / kCap));
    if (nslices < 2) return false;
    slice_len = ((bv.max_len + nslices - 1) / nslices + 3) & ~3;
    return slice_len <= kCap;
}

size_t topk_workspace_bytes(const BatchView& bv, int k) {
    int ns = 0, len = 0;
    if (bv.T <= 0 || !topk_two_pass(bv, k, ns, len)) return 0;
    return slices_bytes(bv.T, ns, k);
}

hipError_t launch_topk_merge(const BatchView& bv, int k, void* ws, int nslices, int slice_len, int32_t* idx,
                             hipStream_t st) {
    const TkSlices sl = slices_in(ws, bv.T, nslices, k, slice_len);
    const size_t shm = (size_t)kLdsWords * sizeof(uint32_t);
    hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)shm);
    if (e != hipSuccess) return e;
    topk_kernel<2><<<bv.T, kTkBlock, shm, st>>>(nullptr, 0, bv, k, nullptr, 0, k, idx, sl);
    return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int64_t ld, const BatchView& bv, int k, const int32_t* kq, int window,
                       int32_t* idx, void* ws, size_t ws_bytes, hipStream_t st) {
    if (bv.T == 0) return hipSuccess;
    int ns = 0, len = 0;
    const size_t need = topk_workspace_bytes(bv, k);
    if (ws != nullptr && need > 0 && ws_bytes >= need && topk_two_pass(bv, k, ns, len)) {
        const TkSlices sl = slices_in(ws, bv.T, ns, k, len);
        const size_t shm1 = (size_t)min(len, kCap) * sizeof(uint32_t);
        const size_t shm2 = (size_t)kLdsWords * sizeof(uint32_t);
        hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shm1);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void*)topk_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm2);
        if (e != hipSuccess) return e;
        topk_kernel<1><<<dim3(bv.T, ns), kTkBlock, shm1, st>>>(scores, ld, bv, k, kq, window, k + window, idx, sl);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        topk_kernel<2><<<bv.T, kTkBlock, shm2, st>>>(scores, ld, bv, k, kq, window, k + window, idx, sl);
        return hipGetLastError();
    }
    // LDS for the longest row: its keys (rounded up so whole 16-byte reads stay inside), or the
    // candidate area when rows may exceed the key cache
    // (with a per-query k any query may select, so the key cache is sized for every row)
    size_t words = 0;
    if (bv.max_len > (kq != nullptr ? 0 : k))
        words = bv.max_len > kCap ? (size_t)kLdsWords : (size_t)((bv.max_len + 3) & ~3);
    const size_t shm = words * sizeof(uint32_t);
    if (shm > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shm);
        if (e != hipSuccess) return e;
    }
    TkSlices none{};
    topk_kernel<0><<<bv.T, kTkBlock, shm, st>>>(scores, ld, bv, k, kq, window, k + window, idx, none);
    return hipGetLastError();
}

}  // namespace dsa
