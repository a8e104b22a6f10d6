// indexer.hip -- lightning-indexer kernels for gfx950.
//
// Score of query t against visible token s (page "一文讀懂DeepSeek-V3.2核心技術DSA", section
// "DSA 的四步工作流程", indexer-scoring step; page "DeepSeek 稀疏注意力路线（V3 / V3.2 / V4）",
// section "两阶段流程", item 1):
//     S[t,s] = scale * k_scale[s] * sum_j w'[t,j] * max(0, q[t,j,:] . k[s,:]),   w' = w * q_scale.
// Folding q_scale into w' and applying k_scale after the head sum is exact because both scales are
// non-negative and max(0, a x) = a max(0, x) for a >= 0.
//
// Three kernels:
//   * fp8 decode:  one wave streams 256 keys of a sequence straight from HBM into MFMA operands
//                  (v_mfma_f32_32x32x64_f8f6f4), several 32-key subtiles in flight; the 1-2 query
//                  tokens of a pass share every key fetch.  HBM-bound: 132 bytes per key (128 fp8 + 4 scale).
//   * bf16 prefill: four query tokens per workgroup (one per wave, 64 heads = two 32-row MFMA
//                  tiles); 64-key tiles are staged once in LDS and shared by the four waves
//                  (v_mfma_f32_32x32x16_bf16).  MFMA-bound.
//   * fp8 prefill: the same streamed structure with the fp8 MFMA, for fp8 batches with more than
//                  eight queries per sequence.
//   * up to 32 heads, any dtype: (token, head) pairs as the 32 MFMA rows (f32, bf16 or fp8 MFMA);
//                  f32 inputs, and bf16 / fp8 shapes the kernels above do not take.
//   * generic:     any dtype / head count, one thread per (query, key); used for the shapes the
//                  MFMA kernels do not cover (more than 32 heads that are not 32 or 64).
// The ReLU-weight-sum epilogue runs on the MFMA accumulators in registers: the 32x32 accumulator
// layout gives every lane 16 head rows of one key column, so the head sum is 16 in-register FMAs
// per tile plus one cross-half shuffle.
#include "indexer_fp8.h"

namespace dsa {
namespace {


// The masked entries of a score row: -inf over positions [lo, hi), written by nthr threads (thread
// index tid).  A call owns the rows (or the part of a row) it masks, so these stores never meet a
// score store.
__device__ __forceinline__ void write_masked(float* row, int64_t lo, int64_t hi, int tid, int nthr) {
    for (int64_t s = lo + tid; s < hi; s += nthr) row[s] = -INFINITY;
}

// Rows of a batch whose queries see no position (max_len == 0): every entry of [0, ld) is masked.
__global__ __launch_bounds__(256) void mask_rows_kernel(float* __restrict__ scores, int64_t ld) {
    write_masked(scores + (int64_t)blockIdx.x * ld, 0, ld, threadIdx.x, 256);
}

// ---------------------------------------------------------------------------------------------
// generic path

constexpr int kGenBlock = 256;

__global__ __launch_bounds__(kGenBlock) void indexer_generic_kernel(
    const void* __restrict__ q, int dtype, const float* __restrict__ q_scale, const float* __restrict__ w,
    int H, CacheView kc, BatchView bv, float scale, float* __restrict__ scores, int64_t ld, int skip_le,
    int mask) {
    extern __shared__ float gsm[];
    float* qs = gsm;                 // [H][128], q * q_scale
    float* wsh = gsm + H * kIdxDim;  // [H]
    const int t = blockIdx.x;
    const int b = bv.q_seq[t];
    if (b < 0 || b >= bv.B) return;
    const int n = min(bv.q_len[t], bv.max_len);
    const int s0 = blockIdx.y * kGenBlock;
    if (mask) {   // this block's positions past n (the last block also takes [grid end, ld))
        const int64_t hi = blockIdx.y + 1 == gridDim.y ? ld : min(ld, (int64_t)s0 + kGenBlock);
        write_masked(scores + (int64_t)t * ld, max((int64_t)s0, (int64_t)max(n, 0)), hi, threadIdx.x, kGenBlock);
    }
    if (n <= skip_le) return;
    if (s0 >= n) return;
    for (int i = threadIdx.x; i < H * kIdxDim; i += kGenBlock) {
        const int j = i / kIdxDim;
        const float sc = q_scale ? q_scale[(int64_t)t * H + j] : 1.0f;
        qs[i] = load_elem(q, dtype, (int64_t)t * H * kIdxDim + i) * sc;
    }
    for (int j = threadIdx.x; j < H; j += kGenBlock) wsh[j] = w[(int64_t)t * H + j];
    __syncthreads();
    const int s = s0 + threadIdx.x;
    if (s >= n) return;
    const int64_t row = cache_row(kc, b, s);
    float kv[kIdxDim];
    float ks = 0.0f;
    if (row >= 0) {
        if (dtype == DSA_F32) {   // 16-byte loads (a row is 512 bytes)
            const f32x4* kr = (const f32x4*)((const float*)kc.data + row * kIdxDim);
#pragma unroll
            for (int i = 0; i < kIdxDim / 4; i++) {
                const f32x4 v = kr[i];
                kv[4 * i] = v[0];
                kv[4 * i + 1] = v[1];
                kv[4 * i + 2] = v[2];
                kv[4 * i + 3] = v[3];
            }
        } else {
            for (int i = 0; i < kIdxDim; i++) kv[i] = load_elem(kc.data, dtype, row * kIdxDim + i);
        }
        ks = kc.scale ? kc.scale[row] : 1.0f;
    } else {
        for (int i = 0; i < kIdxDim; i++) kv[i] = 0.0f;
    }
    float total = 0.0f;
    for (int j = 0; j < H; j++) {
        float dot = 0.0f;
#pragma unroll
        for (int i = 0; i < kIdxDim; i += 4) {   // the query row in 16-byte LDS reads, same order of FMAs
            const f32x4 qv = *(const f32x4*)&qs[j * kIdxDim + i];
            dot = fmaf(qv[0], kv[i], dot);
            dot = fmaf(qv[1], kv[i + 1], dot);
            dot = fmaf(qv[2], kv[i + 2], dot);
            dot = fmaf(qv[3], kv[i + 3], dot);
        }
        total = fmaf(wsh[j], relu_bits(dot), total);
    }
    scores[(int64_t)t * ld + s] = scale * ks * total;
}

// ---------------------------------------------------------------------------------------------
// Up to 32 heads (H dividing 32), any dtype: (token, head) pairs as the MFMA rows.
//
// A 32-row MFMA block holds 32 / H consecutive query tokens of one sequence times their H heads:
// row r is (token r / H, head r % H), so the block's query rows are 32 consecutive rows of q
// ([T, H, 128] flattened).  The 32 columns are keys.  Lane (g, c) holds dims [64g, 64g + 64) of
// query row c and of key c, read with 16-byte loads, and the k-slots of each MFMA step map onto
// those dims the same way for both operands:
//   f32  v_mfma_f32_32x32x2_f32, 64 steps: step s carries dims s and 64 + s;
//   bf16 v_mfma_f32_32x32x16_bf16, 8 steps: half g carries dims 64g + 8s + [0, 8);
//   fp8  v_mfma_scale_f32_32x32x64_f8f6f4, 2 steps: half g carries dims 64g + 32s + [0, 32).
// Accumulator register i of lane (g, c) is row 8(i/4) + 4g + i%4 against key c: for H <= 4 all rows
// of a token lie in one lane, for H >= 8 they are split over lanes c and c + 32 (one cross-half add).
// A workgroup takes one row block and 256 consecutive keys (two 32-key tiles per wave, both loaded
// before the first MFMA).  Used for f32 inputs and for bf16 / fp8 batches the specialised kernels
// above do not take (fewer than 32 heads, fp8 caches without key scales or with pages of fewer
// than 64 tokens).
constexpr int kRowWaves = 4;
constexpr int kRowTiles = 2;                           // 32-key tiles per wave
constexpr int kRowChunk = kRowWaves * kRowTiles * 32;  // keys per workgroup

// One lane's 64 dims of a query or key row in the operand form of dtype DT.
template <int DT> struct RowOperand;
template <> struct RowOperand<DSA_F32> {
    float v[64];
    __device__ __forceinline__ void load(const void* base, int64_t row, int g, bool ok) {
        const f32x4* src = (const f32x4*)((const float*)base + row * kIdxDim + 64 * g);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const f32x4 x = src[i];
#pragma unroll
            for (int e = 0; e < 4; e++) v[4 * i + e] = ok ? x[e] : 0.0f;
        }
    }
};
template <> struct RowOperand<DSA_BF16> {
    bf16x8 v[8];
    __device__ __forceinline__ void load(const void* base, int64_t row, int g, bool ok) {
        const bf16x8* src = (const bf16x8*)((const uint16_t*)base + row * kIdxDim + 64 * g);
        const bf16x8 zero = {};
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = ok ? src[i] : zero;
    }
};
template <> struct RowOperand<DSA_FP8_E4M3> {
    i32x8 v[2];
    __device__ __forceinline__ void load(const void* base, int64_t row, int g, bool ok) {
        const i32x8* src = (const i32x8*)((const uint8_t*)base + row * kIdxDim + 64 * g);
        const i32x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
        v[0] = ok ? src[0] : zero;
        v[1] = ok ? src[1] : zero;
    }
};

template <int DT>
__device__ __forceinline__ f32x16 row_dots(const RowOperand<DT>& qo, const RowOperand<DT>& ko) {
    f32x16 acc = {};
    if constexpr (DT == DSA_F32) {
#pragma unroll
        for (int st = 0; st < 64; st++) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qo.v[st], ko.v[st], acc, 0, 0, 0);
    } else if constexpr (DT == DSA_BF16) {
#pragma unroll
        for (int st = 0; st < 8; st++) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qo.v[st], ko.v[st], acc, 0, 0, 0);
    } else {
        acc = mfma_fp8(qo.v[0], ko.v[0], acc);
        acc = mfma_fp8(qo.v[1], ko.v[1], acc);
    }
    return acc;
}

template <int H, int DT>
__global__ __launch_bounds__(kRowWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void indexer_rows_mfma_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    CacheView kc, BatchView bv, float scale, float* __restrict__ scores, int64_t ld, int skip_le, int mask) {
    static_assert(H >= 1 && H <= 32 && 32 % H == 0, "heads must divide 32");
    constexpr int QR = 32 / H;   // tokens per row block
    __shared__ __attribute__((aligned(16))) float wsh[32];   // w' = w * q_scale of the block's 32 rows
    __shared__ int nsh[QR];                                  // visible positions of the block's tokens
    const int b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    int qb = bv.cu_q[b], qe = bv.cu_q[b + 1];
    qb = max(0, min(qb, bv.T));
    qe = max(qb, min(qe, bv.T));
    const int t0 = qb + QR * blockIdx.x;
    if (t0 >= qe) return;
    const int nq = min(QR, qe - t0);
    if (tid < 32) {
        const int tl = tid / H;
        const int64_t r = (int64_t)min(t0 + tl, qe - 1) * H + tid % H;
        const float ws = q_scale ? q_scale[r] : 1.0f;
        wsh[tid] = tl < nq ? w[r] * ws : 0.0f;
    }
    if (tid < QR) {
        int n = tid < nq ? min(bv.q_len[t0 + tid], bv.max_len) : 0;
        if (n <= skip_le) n = 0;
        nsh[tid] = max(n, 0);
    }
    __syncthreads();
    const int64_t s_lo = (int64_t)blockIdx.y * kRowChunk;
    if (mask) {   // this block's positions past n (the last block also takes [grid end, ld))
        const int64_t s_hi = blockIdx.y + 1 == gridDim.y ? ld : min(ld, s_lo + kRowChunk);
        for (int u = 0; u < nq; u++)
            write_masked(scores + (int64_t)(t0 + u) * ld, max(s_lo, (int64_t)nsh[u]), s_hi, tid, kRowWaves * 64);
    }
    int nmax = 0;
    for (int u = 0; u < nq; u++) nmax = max(nmax, nsh[u]);
    const int64_t key0 = s_lo + (int64_t)wave * kRowTiles * 32;
    if (key0 >= nmax) return;

    // query rows: row c of the block; rows of tokens past the batch read a valid row and are never stored
    RowOperand<DT> qo;
    qo.load(q, min((int64_t)t0 * H + c, (int64_t)qe * H - 1), g, true);
    // keys of both tiles (positions past the context read its last key; an invalid page is a zero row)
    RowOperand<DT> ko[kRowTiles];
    float ks[kRowTiles];
#pragma unroll
    for (int tt = 0; tt < kRowTiles; tt++) {
        const int64_t s = min(key0 + 32 * tt + c, (int64_t)nmax - 1);
        const int64_t row = cache_row(kc, b, s);
        const bool ok = row >= 0;
        ko[tt].load(kc.data, ok ? row : 0, g, ok);
        ks[tt] = ok ? (kc.scale ? kc.scale[row] : 1.0f) : 0.0f;
    }
#pragma unroll
    for (int tt = 0; tt < kRowTiles; tt++) {
        const f32x16 acc = row_dots<DT>(qo, ko[tt]);
        // weighted ReLU head sums: dense index du of the lane's tokens
        constexpr int NU = H <= 4 ? 16 / H : 32 / H;   // tokens per lane
        float tot[NU];
#pragma unroll
        for (int u = 0; u < NU; u++) tot[u] = 0.0f;
#pragma unroll
        for (int a = 0; a < 4; a++) {
            const f32x4 wv = *(const f32x4*)&wsh[8 * a + 4 * g];   // rows 8a + 4g + [0, 4)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int du = H <= 4 ? a * (4 / H) + e / H : (8 * a) / H;
                tot[du] = fmaf(wv[e], relu_bits(acc[4 * a + e]), tot[du]);
            }
        }
        if constexpr (H >= 8) {
#pragma unroll
            for (int u = 0; u < NU; u++) tot[u] += __shfl_xor(tot[u], 32, 64);
        }
        const int64_t s = key0 + 32 * tt + c;
#pragma unroll
        for (int u = 0; u < NU; u++) {
            // token of dense index u: H <= 4: row 8a + 4g + e with u = a (4/H) + e/H; H >= 8: 8a/H = u
            const int tl = H <= 4 ? (8 * (u / (4 / H))) / H + (4 * g) / H + (u % (4 / H)) : u;
            if ((H <= 4 || g == 0) && tl < nq && s < nsh[tl])
                scores[(int64_t)(t0 + tl) * ld + s] = scale * ks[tt] * tot[u];
        }
    }
}

// ---------------------------------------------------------------------------------------------
// fp8 decode path: v_mfma_f32_32x32x64_f8f6f4.
//
// Operand layout (lane l, half g = l/32, column c = l%32): lane l holds row/column c and the 32
// k-values 32g..32g+31 of the MFMA.  Both operands use the same dim assignment, so the contraction
// is over the right pairs whatever order the hardware sums in: in k-step ks, half g carries dims
// 64g + 32ks + [0,32).  A lane therefore reads 64 contiguous bytes of one key row.
// Accumulator: lane l, register i holds column c (the key) and row 8(i/4) + 4g + i%4 (the head).

constexpr int kDecKeysPerWave = 256;
constexpr int kDecWaves = 4;


// QG query tokens of one sequence share each key fetch (1 for plain decode, 2 for two-token
// speculative decode).  A wave keeps PF = 3 key subtiles (32 keys each) in flight: the loads of subtile
// i + PF are issued as soon as subtile i has been consumed.  The storage rows of all of the wave's
// subtiles are looked up first (one batch of page-table loads), so a key load never waits for its
// page lookup.  The head weights of a pass live in a per-wave LDS area (read 4 at a time where
// they are used), which keeps registers for the key ring.  Loads past the end of the context are
// clamped to its last token (in bounds; their scores are not stored).
template <int NHS, int QG>
__global__ __launch_bounds__(kDecWaves * 64) void indexer_fp8_decode_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    CacheView kc, BatchView bv, float scale, float* __restrict__ scores, int64_t ld, int skip_le, int mask) {
    constexpr int H = 32 * NHS;
    // three subtiles in flight, for one query or two (one query: 21.0 against 21.4-21.7 us with four at
    // decode 64 x 8192, 61.4-61.8 against 62.8 at 64 x 32768; two queries: 82 against 86-87 us with two)
    constexpr int PF = 3;
    constexpr int kSub = kDecKeysPerWave / 32;
    __shared__ __attribute__((aligned(16))) float wsh[kDecWaves][QG][H];   // w * q_scale, per wave
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, c = lane & 31;
    int qb = bv.cu_q[b], qe = bv.cu_q[b + 1];
    qb = max(0, min(qb, bv.T));
    qe = max(qb, min(qe, bv.T));
    const int64_t key0 = (int64_t)blockIdx.x * (kDecWaves * kDecKeysPerWave) + wave * kDecKeysPerWave;

    for (int t0 = qb; t0 < qe; t0 += QG) {
        const int nq = min(QG, qe - t0);
        int n[QG];
#pragma unroll
        for (int u = 0; u < QG; u++) {
            n[u] = u < nq ? min(bv.q_len[t0 + u], bv.max_len) : 0;
            if (n[u] <= skip_le) n[u] = 0;
        }
        int nmax = n[0];
#pragma unroll
        for (int u = 1; u < QG; u++) nmax = max(nmax, n[u]);
        if (mask) {   // this block's positions past n (the last block also takes [grid end, ld))
            const int64_t blo = (int64_t)blockIdx.x * (kDecWaves * kDecKeysPerWave);
            const int64_t bhi = blockIdx.x + 1 == gridDim.x ? ld : min(ld, blo + kDecWaves * kDecKeysPerWave);
            for (int u = 0; u < nq; u++)
                write_masked(scores + (int64_t)(t0 + u) * ld, max(blo, (int64_t)max(n[u], 0)), bhi, threadIdx.x,
                             kDecWaves * 64);
        }
        if (key0 >= nmax) continue;

        // storage rows of the wave's subtiles: lane (g, c) reads key key0 + 32*sub + c
        uint32_t rowv[kSub];
        uint32_t okm = 0;                  // bit sub: the key's page is valid
        if (kc.page_table == nullptr) {
#pragma unroll
            for (int sub = 0; sub < kSub; sub++) {
                const int64_t s = key0 + 32 * sub + c < nmax ? key0 + 32 * sub + c : (int64_t)nmax - 1;
                rowv[sub] = (uint32_t)((int64_t)b * kc.seq_stride + s);
                okm |= 1u << sub;
            }
        } else {
            // all page-table reads first, then the row arithmetic: the reads are in flight together
            // (positions and page numbers fit 32 bits: one 32-bit division per key, its quotient reused)
            int32_t pg[kSub], off[kSub];
            const int32_t* pt = kc.page_table + (int64_t)b * kc.pt_stride;
            const int ps = kc.page_size;
#pragma unroll
            for (int sub = 0; sub < kSub; sub++) {
                const int s = min((int)key0 + 32 * sub + c, nmax - 1);
                const int pi = s / ps;
                off[sub] = s - pi * ps;
                pg[sub] = pt[pi];
            }
#pragma unroll
            for (int sub = 0; sub < kSub; sub++) {
                const int64_t row = (int64_t)pg[sub] * ps + off[sub];
                const bool ok = pg[sub] >= 0 && row < kc.num_rows;
                rowv[sub] = ok ? (uint32_t)row : 0u;
                okm |= ok ? (1u << sub) : 0u;
            }
        }
        // Memory order: this pass's head weights first (a lane loads at most H/64 of them), then the
        // first PF key subtiles, then the query block; the weights go to LDS after all of that is
        // issued, so that store waits for the weight loads only, not for the key stream behind them.
        float wv_raw[QG][(H + 63) / 64], sv_raw[QG][(H + 63) / 64];
#pragma unroll
        for (int u = 0; u < QG; u++) {
            const int t = t0 + (u < nq ? u : 0);
#pragma unroll
            for (int j = 0; j < (H + 63) / 64; j++) {
                const int r = min(lane + 64 * j, H - 1);
                wv_raw[u][j] = w[(int64_t)t * H + r];
                sv_raw[u][j] = q_scale ? q_scale[(int64_t)t * H + r] : 1.0f;
            }
        }
        i32x8 kf[PF][2];
        float ks[PF];
        auto load_keys = [&](int j, int sub) {
            const uint8_t* src = (const uint8_t*)kc.data + (int64_t)rowv[sub] * kIdxDim + 64 * g;
            kf[j][0] = *(const i32x8*)(src);
            kf[j][1] = *(const i32x8*)(src + 32);
            ks[j] = kc.scale ? kc.scale[rowv[sub]] : 1.0f;
        };
#pragma unroll
        for (int j = 0; j < PF; j++) load_keys(j, j);

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
        // this pass's weights into the wave's own LDS area (no other wave reads it)
#pragma unroll
        for (int u = 0; u < QG; u++)
#pragma unroll
            for (int j = 0; j < (H + 63) / 64; j++) {
                const int r = lane + 64 * j;
                if (r < H) wsh[wave][u][r] = u < nq ? wv_raw[u][j] * sv_raw[u][j] : 0.0f;
            }

#pragma unroll
        for (int sub = 0; sub < kSub; sub++) {
            const int j = sub % PF;
            const int64_t s = key0 + 32 * sub + c;
            // an invalid page reads as an all-zero row
            const bool ok = (okm >> sub) & 1u;
            const i32x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
            const i32x8 k0 = ok ? kf[j][0] : zero, k1 = ok ? kf[j][1] : zero;
            const float ksj = ok ? ks[j] : 0.0f;
#pragma unroll
            for (int u = 0; u < QG; u++) {
                const float sum = fp8_head_sum<NHS>(
                    qf[u], k0, k1, [&](int i) { return *(const f32x4*)&wsh[wave][u][i]; }, g);
                if (g == 0 && s < n[u]) scores[(int64_t)(t0 + u) * ld + s] = fp8_score(scale, ksj, sum);
            }
            if (sub + PF < kSub) load_keys(j, sub + PF);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// bf16 prefill path: v_mfma_f32_32x32x16_bf16, keys staged in LDS.
//
// Operand layout: lane l (half g, column c) holds row/column c and k-values 8g..8g+7.  In k-step
// ks (0..7) half g carries dims 64g + 8ks + [0,8), so a lane reads 128 contiguous bytes of a key row.

constexpr int kPreWaves = 4;
constexpr int kPreTile = 64;      // keys per LDS tile
constexpr int kPreRowB = 272;     // LDS row stride: 256 data bytes + 16 pad (bank spread)

__device__ __forceinline__ f32x16 mfma_bf16_32(const bf16x8& a, const bf16x8& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int NHS>
__global__ __launch_bounds__(kPreWaves * 64) void indexer_bf16_prefill_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    CacheView kc, BatchView bv, float scale, float* __restrict__ scores, int64_t ld, int skip_le, int mask) {
    constexpr int H = 32 * NHS;
    constexpr int kChunksPerThread = kPreTile * 16 / (kPreWaves * 64);   // 16-byte chunks
    __shared__ __attribute__((aligned(16))) uint8_t tile_lds[2][kPreTile * kPreRowB];
    __shared__ int nmax_sh;

    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, c = lane & 31;
    int qb = bv.cu_q[b], qe = bv.cu_q[b + 1];
    qb = max(0, min(qb, bv.T));
    qe = max(qb, min(qe, bv.T));
    const int tq0 = qb + kPreWaves * (gridDim.x - 1 - blockIdx.x);   // longest groups first
    if (tq0 >= qe) return;
    const int t = tq0 + wave;
    const bool has_q = t < qe;
    int n = has_q ? min(bv.q_len[t], bv.max_len) : 0;
    if (n <= skip_le) n = 0;
    if (threadIdx.x == 0) nmax_sh = 0;
    __syncthreads();
    if (lane == 0) atomicMax(&nmax_sh, n);
    __syncthreads();
    const int nmax = nmax_sh;
    // the wave's own row past n (written after the scores, or now when no query of the block has any)
    auto mask_row = [&]() {
        if (mask && has_q) write_masked(scores + (int64_t)t * ld, max(n, 0), ld, lane, 64);
    };
    if (nmax == 0) {
        mask_row();
        return;
    }

    bf16x8 qf[NHS][8];
    float wr[NHS][16];
#pragma unroll
    for (int hs = 0; hs < NHS; hs++) {
        const uint16_t* src = q + ((int64_t)(has_q ? t : tq0) * H + 32 * hs + c) * kIdxDim + 64 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ks++) qf[hs][ks] = *(const bf16x8*)(src + 8 * ks);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int r = 32 * hs + 8 * (i / 4) + 4 * g + (i % 4);
            const int tt = has_q ? t : tq0;
            const float sc = q_scale ? q_scale[(int64_t)tt * H + r] : 1.0f;
            wr[hs][i] = w[(int64_t)tt * H + r] * sc;
        }
    }

    const int ntiles = (nmax + kPreTile - 1) / kPreTile;
    i32x4 stage[kChunksPerThread];
    auto load_tile = [&](int tile) {
#pragma unroll
        for (int r = 0; r < kChunksPerThread; r++) {
            const int ci = threadIdx.x + kPreWaves * 64 * r;
            const int rr = ci >> 4, cc = ci & 15;
            const int64_t s = (int64_t)tile * kPreTile + rr;
            const int64_t row = s < nmax ? cache_row(kc, b, s) : -1;
            stage[r] = row >= 0 ? *(const i32x4*)((const uint8_t*)kc.data + row * (kIdxDim * 2) + cc * 16)
                                : i32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int r = 0; r < kChunksPerThread; r++) {
            const int ci = threadIdx.x + kPreWaves * 64 * r;
            const int rr = ci >> 4, cc = ci & 15;
            *(i32x4*)(&tile_lds[buf][rr * kPreRowB + cc * 16]) = stage[r];
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int tile = 0; tile < ntiles; tile++) {
        const int buf = tile & 1;
        if (tile + 1 < ntiles) load_tile(tile + 1);
#pragma unroll
        for (int sub = 0; sub < kPreTile / 32; sub++) {
            const int sb = tile * kPreTile + sub * 32;
            if (sb < n) {
                bf16x8 kf[8];
                const uint8_t* rowp = &tile_lds[buf][(sub * 32 + c) * kPreRowB + g * 128];
#pragma unroll
                for (int ks = 0; ks < 8; ks++) kf[ks] = *(const bf16x8*)(rowp + 16 * ks);
                float sum = 0.0f;
#pragma unroll
                for (int hs = 0; hs < NHS; hs++) {
                    f32x16 acc = {};
#pragma unroll
                    for (int ks = 0; ks < 8; ks++) acc = mfma_bf16_32(qf[hs][ks], kf[ks], acc);
#pragma unroll
                    for (int i = 0; i < 16; i++) sum = fmaf(wr[hs][i], relu_bits(acc[i]), sum);
                }
                sum += __shfl_xor(sum, 32, 64);
                const int s = sb + c;
                if (g == 0 && s < n) {
                    float ks = 1.0f;
                    if (kc.scale) {
                        const int64_t row = cache_row(kc, b, s);
                        ks = row >= 0 ? kc.scale[row] : 0.0f;
                    }
                    scores[(int64_t)t * ld + s] = scale * ks * sum;
                }
            }
        }
        if (tile + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }
    mask_row();
}

// ---------------------------------------------------------------------------------------------
// bf16 prefill path, streamed through LDS by DMA: eight query tokens per workgroup (one per wave,
// all heads), 64-key tiles fetched with global_load_lds_dwordx4 into a three-deep ring, so the keys
// pass through no registers and the loop carries almost no per-key address work.
//
// Tile layout: DMA instruction r of wave w fills bytes [1024 (2w + r), +1024) of a tile buffer, so
// lane L writes 16 bytes to key row kr = 4 (2w + r) + L/16, slot L%16.  Slot p of row kr holds the
// row's 16-byte chunk p ^ (kr & 15): the MFMA-operand reads below (16 lanes reading the same chunk
// of 16 consecutive rows) then touch 16 distinct 16-byte bank groups.
// Keys past the longest query of the workgroup, and rows of out-of-range pages, are fetched from an
// all-zero row, which scores 0 exactly (ReLU(0) = 0).
//
// Inside a tile each wave runs 2 * NHS MFMA chains (subtile x head slice, eight MFMAs each); the
// ReLU-weight epilogue of chain c (32 VALU instructions) is interleaved with the MFMAs of chain c + 1,
// which keeps the VALU work in the shadow of the matrix unit.
// With 32 heads (NHS = 1) the chains stream their key operands from LDS a few steps ahead instead of
// holding a whole subtile's, which keeps the wave within 128 registers: two workgroups then share a
// CU (four waves per SIMD), and each one's tile barrier and boundary work run under the other's
// MFMAs.  At 64 heads a wave needs more than 128 registers for its query block alone plus the
// chains, and splitting a query's heads over two waves doubles the LDS operand reads and the tile
// DMAs per MFMA (measured slower), so that instance stays at two waves per SIMD.

constexpr int kPfWaves = 8;
constexpr int kPfTile = 64;                              // keys per tile
constexpr int kPfTileBytes = kPfTile * kIdxDim * 2;      // 16 KiB
constexpr int kPfTabMax = 4096;                          // tiles per sequence, paged layout (LDS table)

__device__ const uint8_t kZeroKeyRow[kIdxDim * 2] __attribute__((aligned(256))) = {};

template <typename T>
__device__ __forceinline__ uint32_t lds_off(T* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)p;
}

// global_load_lds_dwordx4: 16 bytes per lane from src into LDS at m0 + 16 * lane.  Written as asm so
// that the compiler does not track the LDS write: its alias bookkeeping would otherwise drain every
// DMA in flight (vmcnt(0)) before each read of a tile buffer.  Arrival is awaited explicitly.  The
// s_nop covers the hazard of m0 written right before a DMA that reads it.
__device__ __forceinline__ void pf_dma(const uint8_t* src, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// Waits for this wave's own LDS operations only, then the workgroup barrier (no vmcnt drain: tile
// DMAs stay in flight across it; their arrival is awaited explicitly).
__device__ __forceinline__ void pf_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// acc = q_slice . k_subtile^T (32 heads x 32 keys), eight MFMAs; meanwhile the epilogue of the
// previous chain folds 16 head rows of `prev` into `sum` (w * max(0, x), two VALU per element), and
// pre(ks) may issue an operand read for a later chain.  Each MFMA is issued before the VALU of its
// step, so the new accumulator and `prev` are live together and never share registers (shared
// registers made the next chain's first MFMA wait for the previous chain to drain).
template <bool EPI, typename Pre>
__device__ __forceinline__ f32x16 pf_chain(const bf16x8 (&qs)[8], const bf16x8 (&kf)[8], const f32x16& prev,
                                           const float (&wp)[16], float& sum, Pre&& pre) {
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ks++) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qs[ks], kf[ks], acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        pre(ks);
        if (EPI) {
            sum = fmaf(wp[2 * ks], relu_bits(prev[2 * ks]), sum);
            sum = fmaf(wp[2 * ks + 1], relu_bits(prev[2 * ks + 1]), sum);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the MFMA / VALU interleave as written
    }
    return acc;
}

// The same chain with its key operands read from the subtile in LDS kPfAhead steps ahead (a few
// registers instead of a subtile's 32).
constexpr int kPfAhead = 3;
template <bool EPI>
__device__ __forceinline__ f32x16 pf_chain_lds(const bf16x8 (&qs)[8], const uint8_t* sub, const uint32_t (&roff)[8],
                                               const f32x16& prev, const float (&wp)[16], float& sum) {
    bf16x8 kb[kPfAhead];
#pragma unroll
    for (int u = 0; u < kPfAhead; u++) kb[u] = *(const bf16x8*)(sub + roff[u]);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ks++) {
        const bf16x8 k = kb[ks % kPfAhead];
        if (ks + kPfAhead < 8) kb[ks % kPfAhead] = *(const bf16x8*)(sub + roff[ks + kPfAhead]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qs[ks], k, acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (EPI) {
            sum = fmaf(wp[2 * ks], relu_bits(prev[2 * ks]), sum);
            sum = fmaf(wp[2 * ks + 1], relu_bits(prev[2 * ks + 1]), sum);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
}

__device__ __forceinline__ float pf_epilogue(const f32x16& a, const float (&wp)[16], float sum) {
#pragma unroll
    for (int i = 0; i < 16; i++) sum = fmaf(wp[i], relu_bits(a[i]), sum);
    return sum;
}

template <int NHS>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(4 / NHS, 4 / NHS)))
void indexer_bf16_stream_kernel(const uint16_t* __restrict__ q, const float* __restrict__ q_scale,
                                const float* __restrict__ w, CacheView kc, BatchView bv, float scale,
                                float* __restrict__ scores, int64_t ld, int skip_le, int mask) {
    constexpr int H = 32 * NHS;
    __shared__ __attribute__((aligned(1024))) uint8_t tile_a[kPfTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t tile_b[kPfTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t tile_c[kPfTileBytes];
    __shared__ int32_t tab[kPfTabMax];      // paged layout: first storage row of each tile, -1 if none
    __shared__ int nmax_sh;

    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, c = lane & 31;
    int qb = bv.cu_q[b], qe = bv.cu_q[b + 1];
    qb = max(0, min(qb, bv.T));
    qe = max(qb, min(qe, bv.T));
    const int tq0 = qb + kPfWaves * (gridDim.x - 1 - blockIdx.x);   // longest groups first
    if (tq0 >= qe) return;
    const int t = tq0 + wave;
    const bool has_q = t < qe;
    int n = has_q ? min(bv.q_len[t], bv.max_len) : 0;
    if (n <= skip_le) n = 0;
    n = max(n, 0);
    if (threadIdx.x == 0) nmax_sh = 0;
    __syncthreads();
    if (lane == 0) atomicMax(&nmax_sh, n);
    __syncthreads();
    const int nmax = nmax_sh;
    // the wave's own row past n: written after the loop (its stores then never sit between the tile
    // DMAs and the explicit waits for them), or now when no query of the block has a position
    auto mask_row = [&]() {
        if (mask && has_q) write_masked(scores + (int64_t)t * ld, n, ld, lane, 64);
    };
    if (nmax == 0) {
        mask_row();
        return;
    }
    const int ntiles = (nmax + kPfTile - 1) / kPfTile;
    const bool paged = kc.page_table != nullptr;
    if (paged) {
        for (int j = threadIdx.x; j < ntiles; j += kPfWaves * 64) {
            const int64_t s0 = (int64_t)j * kPfTile;
            const int64_t page = kc.page_table[(int64_t)b * kc.pt_stride + s0 / kc.page_size];
            const int64_t row0 = page * kc.page_size + s0 % kc.page_size;
            tab[j] = (page >= 0 && row0 < kc.num_rows) ? (int32_t)row0 : -1;
        }
    }

    // operands of this wave's query: head 32 hs + c, dims 64 g + 8 ks .. +8
    bf16x8 qf[NHS][8];
    float wr[NHS][16];
    const int tq = has_q ? t : tq0;
#pragma unroll
    for (int hs = 0; hs < NHS; hs++) {
        const uint16_t* src = q + ((int64_t)tq * H + 32 * hs + c) * kIdxDim + 64 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ks++) qf[hs][ks] = *(const bf16x8*)(src + 8 * ks);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int r = 32 * hs + 8 * (i / 4) + 4 * g + (i % 4);
            const float sc = q_scale ? q_scale[(int64_t)tq * H + r] : 1.0f;
            wr[hs][i] = w[(int64_t)tq * H + r] * sc;
        }
    }
    if (paged) __syncthreads();   // the page table above
    // scalar loads still outstanding in the loop would force every LDS wait there to wait for all
    // (scalar loads return out of order): have the ones the loop uses land before this wait
    asm volatile("" ::"s"(scale), "s"(ld), "s"(scores));
    __builtin_amdgcn_s_waitcnt(0);   // operands in registers before any tile DMA is counted

    // DMA of tile j into buf: two instructions per wave, 4 key rows each
    const int kr_base = 8 * wave + (lane >> 4);
    auto issue = [&](int j, uint8_t* buf) {
#pragma unroll
        for (int r = 0; r < 2; r++) {
            const int kr = kr_base + 4 * r;
            const int64_t s = (int64_t)j * kPfTile + kr;
            const uint8_t* src = kZeroKeyRow;
            if (s < nmax) {
                int64_t row;
                if (paged) {
                    const int r0 = tab[j];
                    row = (r0 >= 0 && (int64_t)r0 + kr < kc.num_rows) ? (int64_t)r0 + kr : -1;
                } else {
                    row = (int64_t)b * kc.seq_stride + s;
                }
                if (row >= 0) src = (const uint8_t*)kc.data + row * (kIdxDim * 2);
            }
            src += 16 * ((lane & 15) ^ (kr & 15));
            pf_dma(src, lds_off(buf) + (2 * wave + r) * 1024);
        }
    };

    // MFMA-operand read offsets: lane (g, c) takes chunk 8 g + ks of row c of a 32-key subtile
    uint32_t roff[8];
#pragma unroll
    for (int ks = 0; ks < 8; ks++) roff[ks] = 256 * c + 16 * ((8 * g + ks) ^ (c & 15));

    float pend[2] = {0.0f, 0.0f};
    int pend_s0 = -1;
    float* srow = scores + (int64_t)t * ld;
    auto flush = [&]() {
        if (pend_s0 >= 0 && g == 0) {
#pragma unroll
            for (int sub = 0; sub < 2; sub++) {
                const int s = pend_s0 + 32 * sub + c;
                if (s < n) srow[s] = pend[sub];
            }
        }
        pend_s0 = -1;
    };

    auto compute = [&](const uint8_t* buf, int j) {
        const int s0 = j * kPfTile;
        if (s0 >= n) return;
        const bool two = s0 + 32 < n;
        if constexpr (NHS == 1) {   // operands streamed from LDS (see above)
            float sum0 = 0.0f, sum1 = 0.0f;
            const f32x16 none = {};
            f32x16 x = pf_chain_lds<false>(qf[0], buf, roff, none, wr[0], sum0);
            if (two) {
                x = pf_chain_lds<true>(qf[0], buf + 8192, roff, x, wr[0], sum0);
                sum1 = pf_epilogue(x, wr[0], sum1);
            } else {
                sum0 = pf_epilogue(x, wr[0], sum0);
            }
            const auto h0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum0), __float_as_uint(sum0), false, false);
            const auto h1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum1), __float_as_uint(sum1), false, false);
            pend[0] = scale * (sum0 + __uint_as_float(h0[1]));
            pend[1] = scale * (sum1 + __uint_as_float(h1[1]));
            pend_s0 = s0;
            return;
        }
        bf16x8 kf0[8], kf1[8];
#pragma unroll
        for (int ks = 0; ks < 8; ks++) kf0[ks] = *(const bf16x8*)(buf + roff[ks]);
        __builtin_amdgcn_sched_barrier(0);
        // the subtile-1 operands are read one per MFMA of the first chain: at most 8 LDS reads are
        // outstanding, so each MFMA waits for its own operand only (lgkmcnt counts to 15)
        auto rd1 = [&](int ks) { kf1[ks] = *(const bf16x8*)(buf + 8192 + roff[ks]); };
        auto none_pre = [](int) {};
        float sum0 = 0.0f, sum1 = 0.0f;
        const f32x16 none = {};
        f32x16 x = pf_chain<false>(qf[0], kf0, none, wr[0], sum0, rd1);
        if constexpr (NHS == 2) x = pf_chain<true>(qf[1], kf0, x, wr[0], sum0, none_pre);
        if (two) {
            x = pf_chain<true>(qf[0], kf1, x, wr[NHS - 1], sum0, none_pre);
            if constexpr (NHS == 2) x = pf_chain<true>(qf[1], kf1, x, wr[0], sum1, none_pre);
            sum1 = pf_epilogue(x, wr[NHS - 1], sum1);
        } else {
            sum0 = pf_epilogue(x, wr[NHS - 1], sum0);
        }
        // the two 32-lane halves hold the two 16-head halves of every 32-head slice
        const auto h0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum0), __float_as_uint(sum0), false, false);
        const auto h1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum1), __float_as_uint(sum1), false, false);
        pend[0] = scale * (sum0 + __uint_as_float(h0[1]));
        pend[1] = scale * (sum1 + __uint_as_float(h1[1]));
        pend_s0 = s0;
    };

    // tile j sits in buffer j % 3; the DMA of tile j + 2 goes to the buffer tile j - 1 used
    auto step = [&](int j, const uint8_t* cur, uint8_t* ahead) {
        if (j + 1 < ntiles)
            asm volatile("s_waitcnt vmcnt(2)" ::: "memory");   // this wave's part of tile j is in LDS
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        pf_barrier();                                           // everyone's part; tile j - 1 is free
        if (j + 2 < ntiles) issue(j + 2, ahead);
        flush();
        compute(cur, j);
    };

    issue(0, tile_a);
    if (ntiles > 1) issue(1, tile_b);
    for (int j = 0; j < ntiles; j += 3) {
        step(j, tile_a, tile_c);
        if (j + 1 < ntiles) step(j + 1, tile_b, tile_a);
        if (j + 2 < ntiles) step(j + 2, tile_c, tile_b);
    }
    flush();
    mask_row();
}

// ---------------------------------------------------------------------------------------------
// fp8 prefill path, streamed through LDS by DMA: the bf16 streamed kernel's structure (eight query
// tokens per workgroup, one per wave, all heads; 64-key tiles by global_load_lds_dwordx4 into a
// three-deep ring) with the fp8 MFMA v_mfma_f32_32x32x64_f8f6f4 (two k-steps per 128-dim key row)
// and the per-key scale.
//
// Tile layout: a key row is 128 bytes = 8 chunks; DMA instruction of wave w fills bytes
// [1024 w, +1024) of a buffer, lane L writing 16 bytes to key row kr = 8 w + L/8, slot L%8.  Slot p of
// row r holds chunk p ^ ((r >> 1) & 7): the operand reads below (16 lanes reading one chunk of 16
// consecutive rows) then fall in 16 distinct 16-byte bank groups (rows r and r + 8 are an even
// number of 128-byte rows apart, so the XOR key differs between them).
// Operand layout as in the decode kernel: in k-step ks, half g of the wave carries dims
// 64 g + 32 ks + [0, 32) of its row (key c or head c), 32 bytes per lane per step.
// Each tile's key scales (two per lane: keys c and 32 + c) are loaded when its DMA is issued, so a
// tile's wait covers three vector-memory operations per lane.

constexpr int kF8Tile = 64;
constexpr int kF8TileBytes = kF8Tile * kIdxDim;   // 8 KiB

template <int NHS>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void indexer_fp8_stream_kernel(const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
                               const float* __restrict__ w, CacheView kc, BatchView bv, float scale,
                               float* __restrict__ scores, int64_t ld, int skip_le, int mask) {
    constexpr int H = 32 * NHS;
    __shared__ __attribute__((aligned(1024))) uint8_t tile_a[kF8TileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t tile_b[kF8TileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t tile_c[kF8TileBytes];
    __shared__ int32_t tab[kPfTabMax];      // paged layout: first storage row of each tile, -1 if none
    __shared__ int nmax_sh;

    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, c = lane & 31;
    int qb = bv.cu_q[b], qe = bv.cu_q[b + 1];
    qb = max(0, min(qb, bv.T));
    qe = max(qb, min(qe, bv.T));
    const int tq0 = qb + kPfWaves * (gridDim.x - 1 - blockIdx.x);   // longest groups first
    if (tq0 >= qe) return;
    const int t = tq0 + wave;
    const bool has_q = t < qe;
    int n = has_q ? min(bv.q_len[t], bv.max_len) : 0;
    if (n <= skip_le) n = 0;
    n = max(n, 0);
    if (threadIdx.x == 0) nmax_sh = 0;
    __syncthreads();
    if (lane == 0) atomicMax(&nmax_sh, n);
    __syncthreads();
    const int nmax = nmax_sh;
    // the wave's own row past n, written after the loop (or now when no query of the block has any)
    auto mask_row = [&]() {
        if (mask && has_q) write_masked(scores + (int64_t)t * ld, n, ld, lane, 64);
    };
    if (nmax == 0) {
        mask_row();
        return;
    }
    const int ntiles = (nmax + kF8Tile - 1) / kF8Tile;
    const bool paged = kc.page_table != nullptr;
    if (paged) {
        for (int j = threadIdx.x; j < ntiles; j += kPfWaves * 64) {
            const int64_t s0 = (int64_t)j * kF8Tile;
            const int64_t page = kc.page_table[(int64_t)b * kc.pt_stride + s0 / kc.page_size];
            const int64_t row0 = page * kc.page_size + s0 % kc.page_size;
            tab[j] = (page >= 0 && row0 < kc.num_rows) ? (int32_t)row0 : -1;
        }
    }

    // operands of this wave's query: head 32 hs + c, dims 64 g + [0, 64)
    i32x8 qf[NHS][2];
    float wr[NHS][16];
    const int tq = has_q ? t : tq0;
#pragma unroll
    for (int hs = 0; hs < NHS; hs++) {
        const uint8_t* src = q + ((int64_t)tq * H + 32 * hs + c) * kIdxDim + 64 * g;
        qf[hs][0] = *(const i32x8*)(src);
        qf[hs][1] = *(const i32x8*)(src + 32);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int r = 32 * hs + 8 * (i / 4) + 4 * g + (i % 4);
            const float sc = q_scale ? q_scale[(int64_t)tq * H + r] : 1.0f;
            wr[hs][i] = w[(int64_t)tq * H + r] * sc;
        }
    }
    if (paged) __syncthreads();   // the page table above
    // scalar loads still outstanding in the loop would make every LDS wait there wait for all
    asm volatile("" ::"s"(scale), "s"(ld), "s"(scores));
    __builtin_amdgcn_s_waitcnt(0);   // operands in registers before any tile DMA is counted

    // storage row of position s of tile j (-1: not a valid row)
    auto row_of = [&](int j, int64_t s) -> int64_t {
        if (s >= nmax) return -1;
        if (paged) {
            const int r0 = tab[j];
            const int64_t row = (int64_t)r0 + (s - (int64_t)j * kF8Tile);
            return (r0 >= 0 && row < kc.num_rows) ? row : -1;
        }
        return (int64_t)b * kc.seq_stride + s;
    };
    // DMA of tile j into buf (one instruction per wave, 8 key rows) and the tile's key scales
    // (keys c and 32 + c of the tile, for the flush of its scores)
    const int kr = 8 * wave + (lane >> 3);
    float ksa[2], ksb[2], ksc[2];
    auto issue = [&](int j, uint8_t* buf, float (&ks)[2]) {
        const int64_t s = (int64_t)j * kF8Tile + kr;
        const int64_t row = row_of(j, s);
        const uint8_t* src = row >= 0 ? (const uint8_t*)kc.data + row * kIdxDim : kZeroKeyRow;
        src += 16 * ((lane & 7) ^ ((kr >> 1) & 7));
        pf_dma(src, lds_off(buf) + wave * 1024);
#pragma unroll
        for (int sub = 0; sub < 2; sub++) {
            const int64_t rs = row_of(j, (int64_t)j * kF8Tile + 32 * sub + c);
            const float v = kc.scale[rs >= 0 ? rs : 0];
            ks[sub] = rs >= 0 ? v : 0.0f;
        }
    };

    // operand read offsets: lane (g, c) takes chunks 4 g + [0, 4) of row c of a 32-key subtile
    uint32_t roff[4];
#pragma unroll
    for (int i = 0; i < 4; i++) roff[i] = 128 * c + 16 * ((4 * g + i) ^ ((c >> 1) & 7));

    float pend[2] = {0.0f, 0.0f};
    int pend_s0 = -1;
    float* srow = scores + (int64_t)t * ld;
    auto flush = [&]() {
        if (pend_s0 >= 0 && g == 0) {
#pragma unroll
            for (int sub = 0; sub < 2; sub++) {
                const int s = pend_s0 + 32 * sub + c;
                if (s < n) srow[s] = pend[sub];
            }
        }
        pend_s0 = -1;
    };

    auto compute = [&](const uint8_t* buf, int j, const float (&ks)[2]) {
        const int s0 = j * kF8Tile;
        if (s0 >= n) return;
        float sum[2] = {0.0f, 0.0f};
#pragma unroll
        for (int sub = 0; sub < 2; sub++) {
            if (sub == 1 && s0 + 32 >= n) break;
            i32x8 kf[2];
#pragma unroll
            for (int st = 0; st < 2; st++) {
                const i32x4 lo = *(const i32x4*)(buf + 4096 * sub + roff[2 * st]);
                const i32x4 hi = *(const i32x4*)(buf + 4096 * sub + roff[2 * st + 1]);
                kf[st] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int hs = 0; hs < NHS; hs++) {
                f32x16 acc = {};
                acc = mfma_fp8(qf[hs][0], kf[0], acc);
                acc = mfma_fp8(qf[hs][1], kf[1], acc);
#pragma unroll
                for (int i = 0; i < 16; i++) sum[sub] = fmaf(wr[hs][i], relu_bits(acc[i]), sum[sub]);
            }
        }
        // the two 32-lane halves hold the two 16-head halves of every 32-head slice
#pragma unroll
        for (int sub = 0; sub < 2; sub++) {
            const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum[sub]), __float_as_uint(sum[sub]),
                                                            false, false);
            pend[sub] = scale * ks[sub] * (sum[sub] + __uint_as_float(h[1]));
        }
        pend_s0 = s0;
    };

    // tile j sits in buffer j % 3; the DMA of tile j + 2 goes to the buffer tile j - 1 used
    auto step = [&](int j, const uint8_t* cur, const float (&kcur)[2], uint8_t* ahead, float (&kahead)[2]) {
        if (j + 1 < ntiles)
            asm volatile("s_waitcnt vmcnt(3)" ::: "memory");   // this wave's part of tile j, and its scales
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        pf_barrier();                                           // everyone's part; tile j - 1 is free
        if (j + 2 < ntiles) issue(j + 2, ahead, kahead);
        flush();
        compute(cur, j, kcur);
    };

    issue(0, tile_a, ksa);
    if (ntiles > 1) issue(1, tile_b, ksb);
    for (int j = 0; j < ntiles; j += 3) {
        step(j, tile_a, ksa, tile_c, ksc);
        if (j + 1 < ntiles) step(j + 1, tile_b, ksb, tile_a, ksa);
        if (j + 2 < ntiles) step(j + 2, tile_c, ksc, tile_b, ksb);
    }
    flush();
    mask_row();
}

}  // namespace

hipError_t launch_indexer(const void* q, int dtype, const float* q_scale, const float* w, int H,
                          const CacheView& kc, const BatchView& bv, float scale, float* scores,
                          int64_t ld, int skip_le, int mask, hipStream_t st) {
    if (bv.T == 0) return hipSuccess;
    if (mask) skip_le = 0;   // every row is written whole
    if (bv.max_len == 0) {
        if (!mask || ld == 0) return hipSuccess;
        mask_rows_kernel<<<bv.T, 256, 0, st>>>(scores, ld);
        return hipGetLastError();
    }
    if (bv.max_len <= skip_le) return hipSuccess;
    const int nhs = (H % 32 == 0) ? H / 32 : 0;
    if (dtype == DSA_FP8_E4M3 && (nhs == 1 || nhs == 2) && bv.max_q <= 8) {
        dim3 grid((bv.max_len + kDecWaves * kDecKeysPerWave - 1) / (kDecWaves * kDecKeysPerWave), bv.B);
        const uint8_t* q8 = (const uint8_t*)q;
        const int block = kDecWaves * 64;
        if (bv.max_q == 1) {
            if (nhs == 1)
                indexer_fp8_decode_kernel<1, 1><<<grid, block, 0, st>>>(q8, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
            else
                indexer_fp8_decode_kernel<2, 1><<<grid, block, 0, st>>>(q8, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
        } else {
            if (nhs == 1)
                indexer_fp8_decode_kernel<1, 2><<<grid, block, 0, st>>>(q8, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
            else
                indexer_fp8_decode_kernel<2, 2><<<grid, block, 0, st>>>(q8, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
        }
        return hipGetLastError();
    }
    const bool stream_layout = kc.page_table == nullptr ||
                               (kc.page_size % kPfTile == 0 && (int64_t)bv.max_len <= (int64_t)kPfTabMax * kPfTile);
    if (dtype == DSA_FP8_E4M3 && (nhs == 1 || nhs == 2) && kc.scale != nullptr && stream_layout) {
        // fp8 with more than 8 queries per sequence: the streamed prefill kernel
        dim3 grid((bv.max_q + kPfWaves - 1) / kPfWaves, bv.B);
        if (nhs == 1)
            indexer_fp8_stream_kernel<1><<<grid, kPfWaves * 64, 0, st>>>(
                (const uint8_t*)q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
        else
            indexer_fp8_stream_kernel<2><<<grid, kPfWaves * 64, 0, st>>>(
                (const uint8_t*)q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
        return hipGetLastError();
    }
    if (dtype == DSA_BF16 && (nhs == 1 || nhs == 2) && kc.scale == nullptr && stream_layout) {
        dim3 grid((bv.max_q + kPfWaves - 1) / kPfWaves, bv.B);
        if (nhs == 1)
            indexer_bf16_stream_kernel<1><<<grid, kPfWaves * 64, 0, st>>>(
                (const uint16_t*)q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
        else
            indexer_bf16_stream_kernel<2><<<grid, kPfWaves * 64, 0, st>>>(
                (const uint16_t*)q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
        return hipGetLastError();
    }
    if (dtype == DSA_BF16 && (nhs == 1 || nhs == 2)) {
        dim3 grid((bv.max_q + kPreWaves - 1) / kPreWaves, bv.B);
        if (nhs == 1)
            indexer_bf16_prefill_kernel<1><<<grid, kPreWaves * 64, 0, st>>>(
                (const uint16_t*)q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
        else
            indexer_bf16_prefill_kernel<2><<<grid, kPreWaves * 64, 0, st>>>(
                (const uint16_t*)q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask);
        return hipGetLastError();
    }
    if ((dtype == DSA_F32 || dtype == DSA_BF16 || dtype == DSA_FP8_E4M3) && H >= 1 && H <= 32 && 32 % H == 0) {
        const int qr = 32 / H;
        dim3 grid((bv.max_q + qr - 1) / qr, (bv.max_len + kRowChunk - 1) / kRowChunk, bv.B);
        auto go = [&](auto dt) {
            constexpr int DT = decltype(dt)::value;
            switch (H) {
                case 1: indexer_rows_mfma_kernel<1, DT><<<grid, kRowWaves * 64, 0, st>>>(q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask); break;
                case 2: indexer_rows_mfma_kernel<2, DT><<<grid, kRowWaves * 64, 0, st>>>(q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask); break;
                case 4: indexer_rows_mfma_kernel<4, DT><<<grid, kRowWaves * 64, 0, st>>>(q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask); break;
                case 8: indexer_rows_mfma_kernel<8, DT><<<grid, kRowWaves * 64, 0, st>>>(q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask); break;
                case 16: indexer_rows_mfma_kernel<16, DT><<<grid, kRowWaves * 64, 0, st>>>(q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask); break;
                default: indexer_rows_mfma_kernel<32, DT><<<grid, kRowWaves * 64, 0, st>>>(q, q_scale, w, kc, bv, scale, scores, ld, skip_le, mask); break;
            }
        };
        if (dtype == DSA_F32) go(std::integral_constant<int, DSA_F32>{});
        else if (dtype == DSA_BF16) go(std::integral_constant<int, DSA_BF16>{});
        else go(std::integral_constant<int, DSA_FP8_E4M3>{});
        return hipGetLastError();
    }
    const size_t shm = (size_t)H * (kIdxDim + 1) * sizeof(float);
    if (shm > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)indexer_generic_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        if (e != hipSuccess) return e;
    }
    dim3 grid(bv.T, (bv.max_len + kGenBlock - 1) / kGenBlock);
    indexer_generic_kernel<<<grid, kGenBlock, shm, st>>>(q, dtype, q_scale, w, H, kc, bv, scale, scores, ld,
                                                         skip_le, mask);
    return hipGetLastError();
}

}  // namespace dsa
