// sparse_mla.hip -- sparse MLA in MQA form for gfx950.
//
// For query t, head h and the selected positions I of t (page "一文讀懂DeepSeek-V3.2核心技術DSA",
// section "DSA 的四步工作流程", sparse-MLA step; page "DeepSeek-V3.2加速技术详解", section 3.1
// "MHA版MLA VS MQA版MLA": every head attends over the same shared latent rows and the value
// up-projection comes afterwards):
//     z_j = softmax_scale * q[t,h,:576] . c[I_j,:576],   out[t,h,:] = sum_j softmax(z)_j c[I_j,:512].
//
// Workgroup = (query, split of the index slots), 8 waves, 16 heads per wave (up to 128 heads).
//   1. The split's valid indices are compacted (order kept) into an LDS list of storage rows.
//   2. Tiles of 32 selected rows (32 x 1152 B) are gathered straight into LDS with gfx950's
//      global_load_lds_dwordx4 (no staging registers), double-buffered: the next tile's loads are
//      in flight while the current one is consumed.  One fetch of a row serves all heads -- the
//      MQA form is what makes the sparse gather cheap.
//   3. Logits S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys as rows, the wave's 16 heads as
//      columns); the query block stays in registers for the whole split.
//   4. Online softmax in base 2: each lane owns 8 keys of one head; the head's running max needs
//      two cross-lane steps.
//   5. O += P V with v_mfma_f32_16x16x32_bf16.  P is already in operand layout (no shuffle): its
//      8 keys per lane define the k-slot order, and V is read in the matching order with the
//      gfx950 LDS transpose load ds_read_b64_tr_b16.
// A split writes normalised partial outputs and their log-sum-exp; a combine kernel merges splits
// by log-sum-exp weights in a fixed order, so results are deterministic.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kMlaWaves = 8;
constexpr int kMlaThreads = kMlaWaves * 64;
constexpr int kTile = 32;                       // selected rows per LDS tile
constexpr int kRowChunks = kDqk * 2 / 16;       // 72 16-byte chunks per latent row
constexpr int kRowSlots = kRowChunks + 1;       // LDS row = 72 chunks + 1 pad chunk (bank spread)
constexpr int kRowB = kRowSlots * 16;           // 1168 bytes
constexpr int kTileSlots = kTile * kRowSlots;   // 2336 16-byte LDS slots per tile
constexpr int kLoadsPerWave = (kTileSlots + kMlaThreads - 1) / kMlaThreads;
constexpr int kMaxList = 4096;                  // index slots per split
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kMlaThreads) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, int H, CacheView lat, BatchView bv, const int32_t* __restrict__ idx,
    int k, int per_split, int splits, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
    extern __shared__ __attribute__((aligned(16))) uint8_t msm[];
    uint8_t* tiles = msm;                                         // [2][kTile][kRowB]
    int32_t* rows = (int32_t*)(msm + 2 * kTile * kRowB);          // [per_split]
    __shared__ int wcount[kMlaWaves];

    const int t = blockIdx.x / splits, split = blockIdx.x % splits;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int b = bv.q_seq[t];
    const bool seq_ok = b >= 0 && b < bv.B;
    const int n = seq_ok ? min(bv.q_len[t], bv.max_len) : 0;
    const int j0 = split * per_split, j1 = min(k, j0 + per_split);
    const uint64_t lt_mask = (1ull << lane) - 1ull;

    // 1. compact the valid selected positions of this split into storage rows
    int cnt = 0;
    for (int base = j0; base < j1; base += kMlaThreads) {
        const int slot = base + tid;
        const int s = slot < j1 ? idx[(int64_t)t * k + slot] : -1;
        const int64_t row = (s >= 0 && s < n) ? cache_row(lat, b, s) : -1;
        const bool valid = row >= 0;
        const uint64_t bal = __ballot(valid);
        if (lane == 0) wcount[wave] = __popcll(bal);
        __syncthreads();
        int off = cnt, tot = 0;
        for (int w = 0; w < kMlaWaves; w++) {
            if (w < wave) off += wcount[w];
            tot += wcount[w];
        }
        if (valid) rows[off + __popcll(bal & lt_mask)] = (int32_t)row;
        cnt += tot;
        __syncthreads();
    }

    // query block of this wave: lane (g, j) holds head 16*wave + j, dims 32*kk + 8*g + [0, 8)
    const int hq = 16 * wave + j;
    const bool wave_on = 16 * wave < H;
    bf16x8 qf[kDqk / 32];
    const bf16x8 zero8 = {};
#pragma unroll
    for (int kk = 0; kk < kDqk / 32; kk++)
        qf[kk] = (wave_on && hq < H) ? *(const bf16x8*)(q + ((int64_t)t * H + hq) * kDqk + 32 * kk + 8 * g) : zero8;

    f32x4 oacc[kDv / 16];
#pragma unroll
    for (int nd = 0; nd < kDv / 16; nd++) oacc[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    const int ntiles = (cnt + kTile - 1) / kTile;
    // 2. gather a tile straight into LDS (global_load_lds_dwordx4): wave instruction r of wave w
    //    fills LDS slots [64 (8 r + w), +64); slot p holds chunk p % 73 of tile row p / 73 (the 73rd
    //    slot of a row is padding and is not loaded).  Rows past the end of the list repeat the
    //    last selected row, so every LDS value stays finite; their logits are masked to -inf.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto load_tile = [&](int tile, int buf) {
        uint8_t* tb = tiles + buf * kTile * kRowB;
#pragma unroll
        for (int r = 0; r < kLoadsPerWave; r++) {
            const int p0 = (r * kMlaWaves + wave_u) * 64;
            const int p = p0 + lane;
            if (p < kTileSlots) {
                const int rr = p / kRowSlots, cc = p - rr * kRowSlots;
                if (cc < kRowChunks) {
                    const int row = rows[min(tile * kTile + rr, cnt - 1)];
                    const uint8_t* src = (const uint8_t*)lat.data + (int64_t)row * (kDqk * 2) + cc * 16;
                    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                                     (__attribute__((address_space(3))) void*)(tb + p0 * 16), 16, 0, 0);
                }
            }
        }
    };

    if (ntiles > 0) load_tile(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int tile = 0; tile < ntiles; tile++) {
        const int buf = tile & 1;
        if (tile + 1 < ntiles) load_tile(tile + 1, buf ^ 1);
        if (wave_on) {
            const uint8_t* tb = tiles + buf * kTile * kRowB;
            // 3. logits for keys 16*nt + 4*g + i (rows) x heads j (columns)
            f32x4 sacc[2];
#pragma unroll
            for (int nt = 0; nt < 2; nt++) {
                sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                const uint8_t* rp = tb + (16 * nt + j) * kRowB + 16 * g;
#pragma unroll
                for (int kk = 0; kk < kDqk / 32; kk++) sacc[nt] = mfma16(*(const bf16x8*)(rp + 64 * kk), qf[kk], sacc[nt]);
            }
            // 4. online softmax; slot r of this lane is key 16*(r/4) + 4*g + r%4 of the tile
            float z[8];
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const int key = tile * kTile + 16 * (r / 4) + 4 * g + (r % 4);
                z[r] = key < cnt ? sacc[r / 4][r % 4] * scale_log2 : -INFINITY;
            }
            float mt = z[0];
#pragma unroll
            for (int r = 1; r < 8; r++) mt = fmaxf(mt, z[r]);
            mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float m_new = fmaxf(m_run, mt);
            const float mbase = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = exp2f(m_run - mbase);
            float psum = 0.0f;
            bf16x8 pf;
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const float p = exp2f(z[r] - mbase);
                psum += p;
                pf[r] = (__bf16)p;
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            float ao[4];
#pragma unroll
            for (int i = 0; i < 4; i++) ao[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
            for (int nd = 0; nd < kDv / 16; nd++)
#pragma unroll
                for (int i = 0; i < 4; i++) oacc[nd][i] *= ao[i];
            // 5. O[heads 4g+i][dims 16nd + j] += P V; V rows come transposed from LDS so that lane
            //    (g, j) receives dim 16nd + j of keys 4g + [0,4) (first read) and 16 + 4g + [0,4).
            const uint8_t* vp = tb + (4 * g + (j >> 2)) * kRowB + 8 * (j & 3);
#pragma unroll
            for (int nd = 0; nd < kDv / 16; nd++) {
                const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 32 * nd));
                const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 16 * kRowB + 32 * nd));
                const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[nd] = mfma16(pf, vf, oacc[nd]);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    if (!wave_on) return;
    float l = l_run + __shfl_xor(l_run, 16, 64);
    l += __shfl_xor(l, 32, 64);                              // softmax denominator of head hq
    const float lse_h = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float li = __shfl(l, 4 * g + i, 64);
        inv[i] = li > 0.0f ? 1.0f / li : 0.0f;
    }
    if (splits == 1) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int head = 16 * wave + 4 * g + i;
            if (head < H) {
                uint16_t* op = out + ((int64_t)t * H + head) * kDv + j;
#pragma unroll
                for (int nd = 0; nd < kDv / 16; nd++) op[16 * nd] = f32_to_bf16_bits(oacc[nd][i] * inv[i]);
            }
        }
        if (lse && g == 0 && hq < H) lse[(int64_t)t * H + hq] = lse_h;
    } else {
        float* po = part_o + ((int64_t)t * splits + split) * H * kDv;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int head = 16 * wave + 4 * g + i;
            if (head < H) {
#pragma unroll
                for (int nd = 0; nd < kDv / 16; nd++) po[(int64_t)head * kDv + 16 * nd + j] = oacc[nd][i] * inv[i];
            }
        }
        if (g == 0 && hq < H) part_lse[((int64_t)t * splits + split) * H + hq] = lse_h;
    }
}

// Merge the splits of each (query, head): weights exp(lse_s - max), fixed order over s.
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse, int splits, int H,
                                                          int T, uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= T * H) return;
    const int lane = threadIdx.x & 63;
    const int t = wid / H, h = wid % H;
    float m = -INFINITY;
    for (int s = 0; s < splits; s++) m = fmaxf(m, part_lse[((int64_t)t * splits + s) * H + h]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.0f;
    if (m != -INFINITY) {
        for (int s = 0; s < splits; s++) {
            const float wgt = expf(part_lse[((int64_t)t * splits + s) * H + h] - m);
            wsum += wgt;
            const f32x4* po = (const f32x4*)(part_o + (((int64_t)t * splits + s) * H + h) * kDv + lane * 8);
            const f32x4 a = po[0], c = po[1];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                acc[e] = fmaf(wgt, a[e], acc[e]);
                acc[4 + e] = fmaf(wgt, c[e], acc[4 + e]);
            }
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    uint16_t* op = out + ((int64_t)t * H + h) * kDv + lane * 8;
    uint32_t packed[4];
#pragma unroll
    for (int e = 0; e < 4; e++)
        packed[e] = (uint32_t)f32_to_bf16_bits(acc[2 * e] * inv) | ((uint32_t)f32_to_bf16_bits(acc[2 * e + 1] * inv) << 16);
    *(i32x4*)op = i32x4{(int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]};
    if (lse && lane == 0) lse[(int64_t)t * H + h] = wsum > 0.0f ? m + logf(wsum) : -INFINITY;
}

}  // namespace

int mla_splits(int T, int k) {
    if (T <= 0 || k <= 0) return 1;
    int s = (256 + T - 1) / T;                 // aim at one 8-wave workgroup per CU
    s = min(s, max(1, k / 64));                // at least 64 index slots per split
    s = max(s, (k + kMaxList - 1) / kMaxList); // the LDS index list holds kMaxList slots
    return max(1, s);
}

size_t mla_workspace_bytes(int T, int k, int H) {
    const int s = mla_splits(T, k);
    if (s == 1) return 0;
    const size_t po = (size_t)T * s * H * kDv * sizeof(float);
    const size_t pl = (size_t)T * s * H * sizeof(float);
    return ((po + 255) & ~(size_t)255) + pl;
}

hipError_t launch_sparse_mla(const uint16_t* q, int H, const CacheView& lat, const BatchView& bv,
                             const int32_t* idx, int k, float softmax_scale, uint16_t* out, float* lse,
                             void* ws, hipStream_t st) {
    if (bv.T == 0) return hipSuccess;
    const int splits = mla_splits(bv.T, k);
    const int per_split = (k + splits - 1) / splits;
    const size_t shm = (size_t)2 * kTile * kRowB + (size_t)per_split * sizeof(int32_t);
    hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)shm);
    if (e != hipSuccess) return e;
    float* part_o = nullptr;
    float* part_lse = nullptr;
    if (splits > 1) {
        part_o = (float*)ws;
        const size_t po = (size_t)bv.T * splits * H * kDv * sizeof(float);
        part_lse = (float*)((uint8_t*)ws + ((po + 255) & ~(size_t)255));
    }
    const float scale_log2 = softmax_scale * 1.44269504088896340736f;
    sparse_mla_kernel<<<bv.T * splits, kMlaThreads, shm, st>>>(q, H, lat, bv, idx, k, per_split, splits, scale_log2,
                                                              out, lse, part_o, part_lse);
    e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int blocks = (bv.T * H + 3) / 4;
    mla_combine_kernel<<<blocks, 256, 0, st>>>(part_o, part_lse, splits, H, bv.T, out, lse);
    return hipGetLastError();
}

}  // namespace dsa
