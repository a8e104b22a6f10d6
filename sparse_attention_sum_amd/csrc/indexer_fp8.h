// indexer_fp8.h -- device pieces of the fp8 lightning indexer shared by the decode indexer
// (indexer.hip) and the fused indexer -> top-k kernel (indexer_topk.hip), so that both compute every
// score with the same instructions in the same order (bit-identical scores).
//
// Score of query t against visible token s (page "一文讀懂DeepSeek-V3.2核心技術DSA", section
// "DSA 的四步工作流程", indexer-scoring step; page "DeepSeek 稀疏注意力路线（V3 / V3.2 / V4）",
// section "两阶段流程", item 1):  S[t,s] = scale * k_scale[s] * sum_j w'[t,j] * max(0, q[t,j,:] . k[s,:]).
#pragma once

#include "kernels.h"

namespace dsa {
namespace {

// max(0, x) as a signed-integer max of the bits: non-negative floats order like their bit patterns,
// and every negative float (sign bit set) is a negative integer, which becomes +0.  One VALU
// instruction; fmaxf would add a canonicalising max in IEEE mode.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, f32x16 c) {
    // format 0 = e4m3 for both operands; block scales 127 = 2^0.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Operand layout of v_mfma_f32_32x32x64_f8f6f4 (lane l, half g = l/32, column c = l%32): lane l holds
// row/column c and the 32 k-values 32g..32g+31 of each MFMA; in k-step ks, half g carries dims
// 64g + 32ks + [0,32), so a lane reads 64 contiguous bytes of one key row (k0, k1) and of one query
// head row (qf[hs][0..1]).  Accumulator: lane l, register i holds key c and head 8(i/4) + 4g + i%4.
//
// The weighted head sum sum_j w'[j] max(0, q_j . k_c) of this lane's key c for one query: NHS slices
// of 32 heads, w'[i .. i+3] from wv4(i) (four heads' weights, read from LDS by the caller); the two
// 32-lane halves hold the two 16-head halves of every slice, and one cross-half add completes the
// sum in every lane.
template <int NHS, typename WV4>
__device__ __forceinline__ float fp8_head_sum(const i32x8 (&qf)[NHS][2], const i32x8& k0, const i32x8& k1,
                                              WV4&& wv4, int g) {
    float sum = 0.0f;
#pragma unroll
    for (int hs = 0; hs < NHS; hs++) {
        f32x16 acc = {};
        acc = mfma_fp8(qf[hs][0], k0, acc);
        acc = mfma_fp8(qf[hs][1], k1, acc);
#pragma unroll
        for (int blk = 0; blk < 4; blk++) {
            // heads 32 hs + 8 blk + 4 g + [0, 4) of accumulator registers 4 blk + [0, 4)
            const f32x4 wv = wv4(32 * hs + 8 * blk + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; e++) sum = fmaf(wv[e], relu_bits(acc[4 * blk + e]), sum);
        }
    }
    sum += __shfl_xor(sum, 32, 64);
    return sum;
}

// The score from the head sum: scale * k_scale * sum (an invalid key row has k_scale 0).
__device__ __forceinline__ float fp8_score(float scale, float kscale, float sum) { return scale * kscale * sum; }

}  // namespace
}  // namespace dsa
