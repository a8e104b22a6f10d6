// value_restore.hip -- the value up-projection after sparse MLA in MQA form, for gfx950.
//
// Page "DeepSeek-V3.2加速技术详解", section 3.1 "MHA版MLA VS MQA版MLA": attention runs on the shared
// latent vectors, and the value of each head is restored only afterwards.  For token t and head h:
//     out[t, h, n] = sum_{k < 512} o[t, h, k] * W[h, n, k],      n < d_h
// with o the sparse-MLA output in latent space and W[h] the head's value up-projection, stored
// [d_h][512] (each output dim's 512 weights contiguous).  A batched GEMM per head on the matrix
// cores: v_mfma_f32_32x32x16_bf16, fp32 accumulation, bf16 output (round to nearest even).
//
// Workgroup = (head, tile of 128 tokens, tile of 128 output dims), 4 waves of 64 x 64; K = 512 in
// chunks of 64, double-buffered in LDS with two more chunks in flight in registers (at this size
// the GEMM is bound by HBM: about 100 flop per byte, under the bf16 ridge, so what matters is bytes in
// flight; chunks of 64 rather than 32 cut the time by 6% at 16384 tokens and 16% at 64).  Both
// operands are K-contiguous, so each lane's MFMA fragment (8 consecutive k) is one 16-byte read; LDS
// rows are padded by 16 bytes (144-byte rows) to spread consecutive rows over the banks.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kVrThreads = 256;
constexpr int kVrM = 128;              // tokens per workgroup tile
constexpr int kVrN = 128;              // output dims per workgroup tile
constexpr int kVrK = 64;               // k per LDS chunk
constexpr int kVrRow = kVrK + 8;       // padded LDS row (elements): 144 bytes
constexpr int kVrCb = kVrK / 8;        // 16-byte pieces per row
constexpr int kLatent = 512;
constexpr int kVrChunks = kLatent / kVrK;   // 8
constexpr int kVrPieces = kVrM * kVrK / 8 / kVrThreads;   // 16-byte pieces per operand per thread: 4

typedef __attribute__((ext_vector_type(8))) __bf16 vr_bf16x8;

__global__ __launch_bounds__(kVrThreads) void value_restore_kernel(const uint16_t* o,
                                                                   const uint16_t* w, int T, int H,
                                                                   int dh, uint16_t* __restrict__ out,
                                                                   int heads_first) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kVrM * kVrRow];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kVrN * kVrRow];
    const int m0 = (heads_first ? blockIdx.y : blockIdx.x) * kVrM, h = heads_first ? blockIdx.x : blockIdx.y;
    const int n0 = blockIdx.z * kVrN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;     // the wave's 64 x 64 sub-tile
    const int c32 = lane & 31, g = lane >> 5;

    // global -> registers -> LDS: a chunk is 128 rows x 64 k of each operand = 1024 16-byte pieces
    // each; thread tid moves pieces tid + 256 j (row = piece / 8, 8-element column block = piece % 8).
    // Two chunks are in flight in registers while a third is consumed from LDS.
    // (register sets of native vectors: arrays of HIP's uint4 struct ended up in scratch memory)
    auto load_chunk = [&](int c, i32x4 (&ra)[kVrPieces], i32x4 (&rb)[kVrPieces]) {
#pragma unroll
        for (int j = 0; j < kVrPieces; j++) {
            const int piece = tid + kVrThreads * j, row = piece / kVrCb, cb = piece % kVrCb;
            const int t = min(m0 + row, T - 1);                   // rows past T repeat the last row
            ra[j] = *(const i32x4*)(o + ((int64_t)t * H + h) * kLatent + c * kVrK + 8 * cb);
            rb[j] = *(const i32x4*)(w + ((int64_t)h * dh + n0 + row) * kLatent + c * kVrK + 8 * cb);
        }
    };
    auto store_chunk = [&](int buf, const i32x4 (&ra)[kVrPieces], const i32x4 (&rb)[kVrPieces]) {
#pragma unroll
        for (int j = 0; j < kVrPieces; j++) {
            const int piece = tid + kVrThreads * j, row = piece / kVrCb, cb = piece % kVrCb;
            *(i32x4*)(&As[buf][row * kVrRow + 8 * cb]) = ra[j];
            *(i32x4*)(&Bs[buf][row * kVrRow + 8 * cb]) = rb[j];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = f32x16{};

    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < kVrK; ks += 16) {
            vr_bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                a[i] = *(const vr_bf16x8*)(&As[buf][(wm + 32 * i + c32) * kVrRow + ks + 8 * g]);
                b[i] = *(const vr_bf16x8*)(&Bs[buf][(wn + 32 * i + c32) * kVrRow + ks + 8 * g]);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
        }
    };

    i32x4 a0[kVrPieces], b0[kVrPieces], a1[kVrPieces], b1[kVrPieces];
    load_chunk(0, a0, b0);
    load_chunk(1, a1, b1);
    store_chunk(0, a0, b0);
    load_chunk(2, a0, b0);
    __syncthreads();
    // chunk c is in LDS buffer c & 1; chunk c + 1 in the register set (c + 1) & 1, chunk c + 2 in flight
#pragma unroll
    for (int c = 0; c < kVrChunks; c += 2) {
        compute(0);
        store_chunk(1, a1, b1);                       // chunk c + 1 (buffer 1 was last read before the barrier)
        __syncthreads();
        if (c + 3 < kVrChunks) load_chunk(c + 3, a1, b1);
        compute(1);
        if (c + 2 < kVrChunks) {
            store_chunk(0, a0, b0);                   // chunk c + 2
            __syncthreads();
            if (c + 4 < kVrChunks) load_chunk(c + 4, a0, b0);
        }
    }
    // acc[i][j]: register e holds output dim wn + 32 j + 8 (e / 4) + 4 g + e % 4 of token
    // wm + 32 i + c32 (the B fragment supplies the rows of the 32 x 32 block)
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int t = m0 + wm + 32 * i + c32;
        if (t >= T) continue;
        uint16_t* orow = out + ((int64_t)t * H + h) * dh + n0 + wn;
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int n = 32 * j + 8 * q + 4 * g;
                uint2 v;
                v.x = (uint32_t)f32_to_bf16_bits(acc[i][j][4 * q]) | ((uint32_t)f32_to_bf16_bits(acc[i][j][4 * q + 1]) << 16);
                v.y = (uint32_t)f32_to_bf16_bits(acc[i][j][4 * q + 2]) | ((uint32_t)f32_to_bf16_bits(acc[i][j][4 * q + 3]) << 16);
                *(uint2*)(orow + n) = v;
            }
    }
}

}  // namespace

hipError_t launch_value_restore(const uint16_t* o, const uint16_t* w, int T, int H, int dh, uint16_t* out,
                                hipStream_t st) {
    if (T == 0) return hipSuccess;
    // heads vary fastest: the workgroups that run together cover every head of a few token tiles and
    // read whole token rows o[t][0 .. H) (H KiB, contiguous) instead of 1 KiB rows 128 KiB apart;
    // 698 -> 613-650 us at 16384 tokens x 128 heads, although the head weights are then fetched again
    // from past the L2 (FETCH_SIZE x1.07 -> x1.56 of the algorithmic bytes).  Ordering eight heads per
    // XCD over consecutive token tiles, which keeps each XCD's weights in its L2, measured 775-782 us.
    // (More token tiles than a grid's second dimension holds: tokens first.)
    const int tiles = (T + kVrM - 1) / kVrM;
    const int heads_first = tiles <= 65535 ? 1 : 0;
    const dim3 grid(heads_first ? H : tiles, heads_first ? tiles : H, dh / kVrN);
    value_restore_kernel<<<grid, kVrThreads, 0, st>>>(o, w, T, H, dh, out, heads_first);
    return hipGetLastError();
}

}  // namespace dsa
