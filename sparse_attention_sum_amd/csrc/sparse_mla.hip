// sparse_mla.hip -- sparse MLA in MQA form for gfx950.
//
// For query t, head h and the selected positions I of t (page "一文讀懂DeepSeek-V3.2核心技術DSA",
// section "DSA 的四步工作流程", sparse-MLA step; page "DeepSeek-V3.2加速技术详解", section 3.1
// "MHA版MLA VS MQA版MLA": every head attends over the same shared latent rows and the value
// up-projection comes afterwards):
//     z_j = softmax_scale * q[t,h,:576] . c[I_j,:576],   out[t,h,:] = sum_j softmax(z)_j c[I_j,:512].
//
// Workgroup = (query, split of the index slots), 8 waves = 4 head groups of 32 heads x 2 halves;
// two waves per SIMD.  The two waves of a head group split the work so that each holds only half
// of the query block and half of the output block (under 256 registers, which is what allows two
// waves per SIMD):
//   * logits: wave half h contracts query dims [288h, 288h + 288) against the tile, the partial
//     logits are exchanged through LDS and both waves add them in the same order;
//   * output: wave half h accumulates value dims [256h, 256h + 256).
// Per tile:
//   1. Tiles of 32 selected rows (32 x 1152 B) are gathered straight into LDS with gfx950's
//      global_load_lds_dwordx4 (no staging registers), triple-buffered in three distinct LDS arrays
//      so two tiles' loads overlap the current tile's math.  One fetch of a row serves all heads
//      -- the MQA form is what makes the sparse gather cheap.
//   2. Partial logits S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (32 keys as rows, the group's 32
//      heads as columns).
//   3. Softmax in base 2 against a fixed per-head reference (the head's max over the first tile):
//      a lane holds 16 of the 32 keys of one head, the other 16 are in the lane 32 away.  The output
//      block is never rescaled in the loop; a split whose logits climb more than 2^64 above the
//      reference is redone in two passes (exact max, then accumulation).
//   4. O += P V with v_mfma_f32_32x32x16_bf16.  P is already in operand layout (no shuffle): the 16
//      keys a lane owns define the k-slot order of the two K=16 steps, and V is read in the matching
//      order with the gfx950 LDS transpose load ds_read_b64_tr_b16.
// A split writes its normalised partial output (bf16) and log-sum-exp; a combine kernel merges
// splits by log-sum-exp weights in a fixed order, so results are deterministic.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kMlaWaves = 8;
constexpr int kMlaThreads = kMlaWaves * 64;
constexpr int kHeadsPerGroup = 32;
constexpr int kQkHalf = kDqk / 2;               // 288 query dims per wave half
constexpr int kVHalf = kDv / 2;                 // 256 value dims per wave half
constexpr int kTile = 32;                       // selected rows per LDS tile
constexpr int kRowChunks = kDqk * 2 / 16;       // 72 16-byte chunks per latent row
constexpr int kRowSlots = kRowChunks + 1;       // LDS row = 72 chunks + 1 pad chunk (bank spread)
constexpr int kRowB = kRowSlots * 16;           // 1168 bytes
constexpr int kTileSlots = kTile * kRowSlots;   // 2336 16-byte LDS slots per tile
constexpr int kTileB = kTileSlots * 16;
constexpr int kLoadsPerWave = (kTileSlots + kMlaThreads - 1) / kMlaThreads;
constexpr int kMaxList = 2048;                  // index slots per split
constexpr int kAhead = 2;                       // logit operand reads in flight
constexpr int kAheadV = 2;                      // value operand steps in flight
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kHeadroom = 64.0f;              // log2 margin above a head's reference max

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier for the main loop: waits for this wave's own LDS operations only.
// __syncthreads() also carries a release fence, which makes the compiler drain every outstanding
// vector-memory operation (vmcnt(0)) -- including the global->LDS tile loads kept in flight on
// purpose.  Tile completion is handled explicitly (s_waitcnt vmcnt(N) before the barrier), so the
// loop needs only the LDS ordering.  The "memory" clobber keeps the compiler from moving memory
// accesses across it.
// Byte offset of an LDS object, as ds_* instructions address it.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)p;
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 tr_pair(const uint8_t* p0, const uint8_t* p1) {
    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}

__global__ __launch_bounds__(kMlaThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, int H, CacheView lat, BatchView bv, const int32_t* __restrict__ idx,
    int k, int per_split, int splits, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
    // Three distinct LDS tiles: with fixed roles per (unrolled) iteration the compiler can tell that
    // reads of one tile do not depend on the in-flight global->LDS loads into the others.
    __shared__ __attribute__((aligned(16))) uint8_t tile_a[kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t tile_b[kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t tile_c[kTileB];
    __shared__ __attribute__((aligned(16))) f32x4 sx[kMlaWaves][4][64];   // partial-logit exchange
    __shared__ int32_t rows[kMaxList];
    __shared__ int wcount[kMlaWaves];
    __shared__ int xflag[kMlaWaves];   // per wave: number of partial-logit blocks published in sx
    __shared__ bf16x8 qlast[kMlaWaves][64];   // the last query fragment of each lane (see below)

    // XCD-aware order: consecutive workgroups go to different XCDs (round robin over 8), so the
    // splits of one query take block ids 8 apart and share that XCD's L2 for the query block.
    const int nb = gridDim.x;
    const int bid = blockIdx.x;
    const int lid = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
    const int t = lid / splits, split = lid % splits;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hg = wave >> 1, half = wave & 1;      // head group, half of the dims
    const int c32 = lane & 31, g = lane >> 5;       // 32x32 operand layout: column / row c32, k-half g
    const int b = bv.q_seq[t];
    const bool seq_ok = b >= 0 && b < bv.B;
    const int n = seq_ok ? min(bv.q_len[t], bv.max_len) : 0;
    const int j0 = split * per_split, j1 = min(k, j0 + per_split);
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    if (lane == 0) xflag[wave] = 0;

    const int hq = kHeadsPerGroup * hg + c32;
    const bool wave_on = kHeadsPerGroup * hg < H;

    // Memory order of the prologue: the first pass of index reads, then the query half-block, then
    // (after the compaction) the first tile's gathers; the second tile's follow the first barrier,
    // so that they do not join the prologue's burst of reads from every workgroup at once.  The compaction synchronises through LDS
    // only, so the query loads -- 18 per lane, each spanning 32 head rows -- stay in flight while
    // it runs.
    // The first 512 index entries go straight into LDS (tile_c is unused until the loop) with a
    // global_load_lds_dword issued in asm; the asm also takes the query pointer, so the compiler
    // keeps the query loads after it, and exactly kQf of them follow -- the explicit vmcnt below
    // relies on that count.  Every load here is unconditional, from a clamped in-range address,
    // with the value selected afterwards.
    constexpr int kQf = kQkHalf / 16;
    const uint16_t* qrow = q + ((int64_t)t * H + (kHeadsPerGroup * hg + c32 < H ? hq : 0)) * kDqk + kQkHalf * half + 8 * g;
    {
        const int32_t* src = idx + (int64_t)t * k + min(j0 + tid, k - 1);
        asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off"
                     ::"v"(src), "{m0}"(lds_addr(tile_c) + 256 * __builtin_amdgcn_readfirstlane(wave)), "v"(qrow)
                     : "memory");
    }
    // query half-block: lane (g, c32) holds head 32*hg + c32, dims 288*half + 16*kk + 8*g + [0, 8).
    // The last of the 18 fragments is parked in LDS (read back once per tile): with all 18 in
    // VGPRs the loop needs one register more than the 256 it has at two waves per SIMD, and a
    // scratch reload would wait for the tile loads in flight.
    bf16x8 qf[kQf - 1];
    const bf16x8 zero8 = {};
    const bool q_on = wave_on && hq < H;
#pragma unroll
    for (int kk = 0; kk < kQf - 1; kk++) {
        const bf16x8 v = *(const bf16x8*)(qrow + 16 * kk);
        qf[kk] = q_on ? v : zero8;
    }
    const bf16x8 q_last_raw = *(const bf16x8*)(qrow + 16 * (kQf - 1));
    const bf16x8 q_last = q_on ? q_last_raw : zero8;
    // the index DMA has landed once at most the kQf query loads issued after it are outstanding
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kQf), "v"(qrow) : "memory");
    const int raw_first = ((const int32_t*)tile_c)[tid];
    const int s_first = j0 + tid < j1 ? raw_first : -1;

    // 0. compact the valid selected positions of this split into storage rows
    int cnt = 0;
    for (int base = j0; base < j1; base += kMlaThreads) {
        const int slot = base + tid;
        const int s = base == j0 ? s_first : slot < j1 ? idx[(int64_t)t * k + slot] : -1;
        const int64_t row = (s >= 0 && s < n) ? cache_row(lat, b, s) : -1;
        const bool valid = row >= 0;
        const uint64_t bal = __ballot(valid);
        if (lane == 0) wcount[wave] = __popcll(bal);
        lds_barrier();
        int off = cnt, tot = 0;
        for (int w = 0; w < kMlaWaves; w++) {
            if (w < wave) off += wcount[w];
            tot += wcount[w];
        }
        if (valid) rows[off + __popcll(bal & lt_mask)] = (int32_t)row;
        cnt += tot;
        lds_barrier();
    }

    const int ntiles = (cnt + kTile - 1) / kTile;
    // 1. gather a tile straight into LDS: wave instruction r of wave w fills LDS slots
    //    [64 (8 r + w), +64) of the layout above (padding slots are not loaded).  Rows past the end
    //    of the list repeat the last selected row, so every LDS value stays finite; their logits
    //    are masked to -inf.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int my_loads = (kTileSlots - wave_u * 64 + kMlaThreads - 1) / kMlaThreads;   // instructions per tile
    auto load_tile = [&](int tile, uint8_t* tb) {
        // the lane and wave numbers pass through an empty asm so that the slot arithmetic below is
        // redone at each call instead of being hoisted into registers that stay live all loop long
        // (held, the wave-uniform offsets alone took some twenty scalar registers)
        int lane_o = lane, wave_o = wave_u;
        asm volatile("" : "+v"(lane_o), "+s"(wave_o));
        const int rbase = tile * kTile, last = cnt - 1;
#pragma unroll
        for (int r = 0; r < kLoadsPerWave; r++) {
            const int p0 = (r * kMlaWaves + wave_o) * 64;
            const int rr0 = p0 / kRowSlots, cc0 = p0 - rr0 * kRowSlots;
            const int c = cc0 + lane_o;
            const bool wrap = c >= kRowSlots;
            const int cc = wrap ? c - kRowSlots : c;
            const int rr = rr0 + (wrap ? 1 : 0);
            if (p0 + lane_o < kTileSlots) {
                if (cc < kRowChunks) {
                    const int row = rows[min(rbase + rr, last)];
                    const uint8_t* src = (const uint8_t*)lat.data + (int64_t)row * (kDqk * 2) + cc * 16;
                    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                                     (__attribute__((address_space(3))) void*)(tb + p0 * 16), 16, 0, 0);
                }
            }
        }
    };
    // wait until the next tile to consume has landed; the newest tile's loads may stay in flight
    auto wait_ahead = [&](bool next_exists, bool newest_in_flight) {
        if (next_exists && newest_in_flight) {
            if (my_loads == kLoadsPerWave)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerWave) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerWave - 1) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    };
    if (ntiles > 0) load_tile(0, tile_a);
    qlast[wave][lane] = q_last;   // waits for the query loads only; the gathers stay in flight
    const uint32_t qlast_addr = lds_addr(&qlast[wave][lane]);

    f32x16 oacc[kVHalf / 32];
#pragma unroll
    for (int nd = 0; nd < kVHalf / 32; nd++) oacc[nd] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;

    // V transpose-read address of this lane: 16-lane group G = lane/16 takes k-half g = G/2 and
    // dims 16*(G%2) of each 32-dim block; lane jj of the group points at row 4g + jj/4 (+16m + 8h
    // per step) and dims 4*(jj%4).
    const int G = lane >> 4, jj = lane & 15;
    const int v_off = kRowB * (4 * g + (jj >> 2)) + 32 * (G & 1) + 8 * (jj & 3) + 2 * kVHalf * half;

    // 2. partial logits over this wave's half of the query dims; register i holds key
    //    8*(i/4) + 4*g + i%4 of the tile for head c32
    auto qk_tile = [&](const uint8_t* tb) -> f32x16 {
        f32x16 sacc = {};
        // the parked query fragment; read in asm, with its wait, so the compiler does not hold the
        // read back for the tile loads in flight
        bf16x8 ql;
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(ql) : "v"(qlast_addr) : "memory");
        // the lane number passes through an empty asm: the row offset is recomputed here (a few
        // VALU per tile) rather than held in a register across the loop
        const uint8_t* rp = tb + c32 * kRowB + 16 * g + 2 * kQkHalf * half;
        bf16x8 kb[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; u++) kb[u] = *(const bf16x8*)(rp + 32 * u);
#pragma unroll
        for (int kk = 0; kk < kQkHalf / 16; kk++) {
            const bf16x8 a = kb[kk % kAhead];
            if (kk + kAhead < kQkHalf / 16) kb[kk % kAhead] = *(const bf16x8*)(rp + 32 * (kk + kAhead));
            sacc = mfma32(a, kk < kQf - 1 ? qf[kk] : ql, sacc);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int kk = 0; kk < kQkHalf / 16 - kAhead; kk++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
        return sacc;
    };
    // the two halves' partial logits -> full (unscaled) logits; IEEE addition is commutative, so
    // both waves of the pair get bit-identical sums.  Keys past the end of the list (last tile
    // only) are masked to -inf.
    // Only the two waves of a pair meet here: each publishes its partial block in sx and then bumps
    // its own counter in xflag; the partner waits for that count.  (A workgroup barrier here would
    // lock all eight waves into the same phase.)  The end-of-tile barrier orders the next write of
    // sx after the partner's read of this one.  The writes are one asm block: written in C++, the
    // compiler may make them wait for every tile load in flight (it cannot always tell that `sx` is
    // not their destination); the flag is read in asm for the same reason.
    const uint32_t sx_mine = lds_addr(&sx[wave][0][lane]);
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform: scalar addresses
    const uint32_t flag_mine = lds_addr(&xflag[wave_s]), flag_other = lds_addr(&xflag[wave_s ^ 1]);
    int xepoch = 0;
    auto publish = [&](const f32x16& z) {
        // z comes straight from the MFMA chain; the hazard padding the compiler adds before its own
        // reads of an MFMA result is not applied to inline asm, so the block starts with 20 wait
        // states itself (more than any MFMA result needs before an LDS instruction reads it).
        asm volatile(
            "s_nop 15\n\t"
            "s_nop 3\n\t"
            "ds_write_b128 %0, %1\n\t"
            "ds_write_b128 %0, %2 offset:1024\n\t"
            "ds_write_b128 %0, %3 offset:2048\n\t"
            "ds_write_b128 %0, %4 offset:3072\n\t"
            "s_waitcnt lgkmcnt(0)\n\t"
            "ds_write_b32 %5, %6\n\t"
            "s_waitcnt lgkmcnt(0)" ::"v"(sx_mine), "v"(f32x4{z[0], z[1], z[2], z[3]}), "v"(f32x4{z[4], z[5], z[6], z[7]}),
            "v"(f32x4{z[8], z[9], z[10], z[11]}), "v"(f32x4{z[12], z[13], z[14], z[15]}), "v"(flag_mine),
            "v"(xepoch + 1) : "memory");
        xepoch++;
    };
    auto logits = [&](int tile, f32x16& z) -> float {   // z: this wave's partial logits in, full logits out
        // bounded wait for the partner (both waves of a pair run the same sequence of exchanges,
        // so the count always arrives; the bound only keeps a broken invariant from hanging)
        for (int spin = 0; spin < (1 << 22); spin++) {
            int f;
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(f) : "v"(flag_other) : "memory");
            if (__builtin_amdgcn_readfirstlane(f) >= xepoch) break;
            __builtin_amdgcn_s_sleep(1);
        }
        const f32x4* other = &sx[wave ^ 1][0][lane];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const f32x4 o = other[64 * u];
#pragma unroll
            for (int e = 0; e < 4; e++) z[4 * u + e] += o[e];
            // half the partner's values at a time: fewer live registers at this point keeps the
            // query block out of scratch (a reload would wait for the tile loads in flight)
            if (u == 1) __builtin_amdgcn_sched_barrier(0);
        }
        if ((tile + 1) * kTile > cnt) {
#pragma unroll
            for (int i = 0; i < 16; i++)
                if (tile * kTile + 8 * (i / 4) + 4 * g + (i % 4) >= cnt) z[i] = -INFINITY;
        }
        float mt = z[0];
#pragma unroll
        for (int i = 1; i < 16; i++) mt = fmaxf(mt, z[i]);
        return fmaxf(mt, __shfl_xor(mt, 32, 64)) * scale_log2;   // scaled max over the 32 keys
    };
    // 4. O[heads 8(i/4) + 4g + i%4][dims 256*half + 32nd + c32] += P V.  Step m covers keys
    //    16m + 8(r/4) + 4g + r%4 in k-slot r; the two transpose reads fetch rows 16m + 4g + [0,4)
    //    and 16m + 8 + 4g + [0,4).
    auto pv_tile = [&](f32x16 (&acc)[kVHalf / 32], const uint8_t* tb, const f32x16& z, float mref) {
        bf16x8 pf[2];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            // p = 2^(scale*log2e*z - mref); the raw v_exp_f32 is enough: its argument is at most
            // kHeadroom and anything below 2^-126 may flush to zero
            const float p = __builtin_amdgcn_exp2f(fmaf(z[i], scale_log2, -mref));
            l_run += p;
            pf[i / 8][i % 8] = (__bf16)p;
        }
        const uint8_t* vp = tb + v_off;
        constexpr int kSteps = 2 * (kVHalf / 32);
        bf16x8 vb[kAheadV];
#pragma unroll
        for (int u = 0; u < kAheadV; u++) {
            const uint8_t* p0 = vp + (16 * (u % 2)) * kRowB + 64 * (u / 2);
            vb[u] = tr_pair(p0, p0 + 8 * kRowB);
        }
#pragma unroll
        for (int st = 0; st < kSteps; st++) {
            const bf16x8 v = vb[st % kAheadV];
            if (st + kAheadV < kSteps) {
                const int nx = st + kAheadV;
                const uint8_t* p0 = vp + (16 * (nx % 2)) * kRowB + 64 * (nx / 2);
                vb[st % kAheadV] = tr_pair(p0, p0 + 8 * kRowB);
            }
            acc[st / 2] = mfma32(pf[st % 2], v, acc[st / 2]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAheadV, 0);
#pragma unroll
        for (int st = 0; st < kSteps - kAheadV; st++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAheadV, 0);
    };

    // 3. softmax reference: each head keeps the max of its first tile as a fixed reference, so the
    //    output block is never rescaled inside the loop.  That is exact while no later logit
    //    exceeds the reference by more than kHeadroom (log2 units): p <= 2^kHeadroom cannot
    //    overflow and whatever underflows is below 2^-126 of the largest term.  Past that margin
    //    the workgroup redoes the split in two passes with a fresh accumulator (exact max first).
    //    Every wave takes part in the exchange barrier, also waves without heads.
    bool over = false;
    auto fast_tile = [&](int tile, const uint8_t* tb, uint8_t* nb) {
        // every wave runs the QK step (a wave without heads holds a zero query block); the fences
        // keep the scheduler from stretching register lifetimes across it.  Tile i + 2 is gathered
        // into the buffer that tile i - 1 freed once this wave's QK step is issued: waves reach this
        // point at different times, so the workgroup's gathers do not all queue at the barrier.
        // The partial logits are published before those gathers are issued, so the partner finds
        // them when it is done with its own (about 1 us less per launch than publishing after).
        __builtin_amdgcn_sched_barrier(0);
        f32x16 z = qk_tile(tb);
        __builtin_amdgcn_sched_barrier(0);
        publish(z);
        __builtin_amdgcn_sched_barrier(0);
        if (tile + 2 < ntiles) load_tile(tile + 2, nb);
        __builtin_amdgcn_sched_barrier(0);
        const float mt = logits(tile, z);
        if (!wave_on) return;
        if (tile == 0) m_run = mt;
        over |= mt > m_run + kHeadroom;
        pv_tile(oacc, tb, z, m_run);
    };

    wait_ahead(true, false);
    lds_barrier();
    if (ntiles > 1) load_tile(1, tile_b);   // under tile 0's work rather than in the prologue's burst
    for (int tile = 0; tile < ntiles; tile += 3) {
        // tile i is consumed while tiles i+1 (issued earlier) and i+2 (issued during tile i) are
        // in flight
        fast_tile(tile, tile_a, tile_c);
        wait_ahead(tile + 1 < ntiles, tile + 2 < ntiles);
        lds_barrier();
        if (tile + 1 >= ntiles) break;
        fast_tile(tile + 1, tile_b, tile_a);
        wait_ahead(tile + 2 < ntiles, tile + 3 < ntiles);
        lds_barrier();
        if (tile + 2 >= ntiles) break;
        fast_tile(tile + 2, tile_c, tile_b);
        wait_ahead(tile + 3 < ntiles, tile + 4 < ntiles);
        lds_barrier();
    }

    // 5. normalise and store (bf16 output when the split is the whole selection, else bf16 partials)
    const int hp = (H + kHeadsPerGroup - 1) / kHeadsPerGroup * kHeadsPerGroup;   // padded heads
    auto finish = [&](const f32x16 (&acc)[kVHalf / 32], float lsum, float mref) {
        if (!wave_on) return;
        const float l = lsum + __shfl_xor(lsum, 32, 64);        // softmax denominator of head hq
        const float lse_h = l > 0.0f ? (mref + log2f(l)) * kLn2 : -INFINITY;
        float inv[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float li = __shfl(l, 8 * (i / 4) + 4 * g + (i % 4), 64);
            inv[i] = li > 0.0f ? 1.0f / li : 0.0f;
        }
        if (splits == 1) {
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int head = kHeadsPerGroup * hg + 8 * (i / 4) + 4 * g + (i % 4);
                if (head < H) {
                    uint16_t* op = out + ((int64_t)t * H + head) * kDv + kVHalf * half + c32;
#pragma unroll
                    for (int nd = 0; nd < kVHalf / 32; nd++) op[32 * nd] = f32_to_bf16_bits(acc[nd][i] * inv[i]);
                }
            }
            if (lse && half == 0 && g == 0 && hq < H) lse[(int64_t)t * H + hq] = lse_h;
        } else {
            // bf16 partials in the accumulator's own lane order, 8 bytes per lane per store:
            // [t][split][wave][nd][i/4][lane][i%4]; element (wave, nd, i, lane) is head
            // 32*(wave/2) + 8*(i/4) + 4*(lane/32) + i%4, dim 256*(wave%2) + 32*nd + lane%32.
            i32x2* po = (i32x2*)(part_o + ((int64_t)t * splits + split) * hp * kDv + (int64_t)wave * kHeadsPerGroup * kVHalf);
#pragma unroll
            for (int nd = 0; nd < kVHalf / 32; nd++)
#pragma unroll
                for (int ig = 0; ig < 4; ig++) {
                    const uint32_t lo = (uint32_t)f32_to_bf16_bits(acc[nd][4 * ig] * inv[4 * ig]) |
                                        ((uint32_t)f32_to_bf16_bits(acc[nd][4 * ig + 1] * inv[4 * ig + 1]) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16_bits(acc[nd][4 * ig + 2] * inv[4 * ig + 2]) |
                                        ((uint32_t)f32_to_bf16_bits(acc[nd][4 * ig + 3] * inv[4 * ig + 3]) << 16);
                    po[(nd * 4 + ig) * 64 + lane] = i32x2{(int)lo, (int)hi};
                }
            if (half == 0 && g == 0) part_lse[((int64_t)t * splits + split) * hp + hq] = lse_h;
        }
    };

    if (!__syncthreads_or(over)) {
        finish(oacc, l_run, m_run);
        return;
    }
    // rare: logits spread too far for a fixed reference -- exact max, then accumulate afresh
    float m_exact = -INFINITY;
    for (int tile = 0; tile < ntiles; tile++) {
        __syncthreads();
        load_tile(tile, tile_a);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f32x16 z = wave_on ? qk_tile(tile_a) : f32x16{};
        publish(z);
        m_exact = fmaxf(m_exact, logits(tile, z));
    }
    f32x16 acc2[kVHalf / 32];
#pragma unroll
    for (int nd = 0; nd < kVHalf / 32; nd++) acc2[nd] = f32x16{};
    l_run = 0.0f;
    for (int tile = 0; tile < ntiles; tile++) {
        __syncthreads();
        load_tile(tile, tile_a);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f32x16 z = wave_on ? qk_tile(tile_a) : f32x16{};
        publish(z);
        logits(tile, z);
        if (wave_on) pv_tile(acc2, tile_a, z, m_exact);
    }
    finish(acc2, l_run, m_exact);
}

// Merge the splits of each (query, head) with weights exp(lse_s - lse), in a fixed order over s.
// One workgroup per (query, head group of 32, part of the group's partial block); a thread merges
// one 16-byte chunk.  S (the split count) is a template argument for the common counts, so a
// thread issues all S loads before it uses the first; the weights of the group's heads are
// computed into LDS by each workgroup (32 x S small loads).
constexpr int kCombThreads = 256;
constexpr int kMaxSplitsComb = 64;
constexpr int kCombChunks = kHeadsPerGroup * kDv / 8;         // 16-byte chunks per head group
constexpr int kCombParts = kCombChunks / kCombThreads;        // workgroups per (query, group)
static_assert(kCombParts * 64 == kDv, "a combine workgroup covers 64 value dims of its 32 heads");

template <int S>   // S > 0: compile-time split count; S == 0: runtime count `splits`
__global__ __launch_bounds__(kCombThreads) void mla_combine_kernel(const uint16_t* __restrict__ part_o,
                                                                   const float* __restrict__ part_lse, int splits,
                                                                   int H, int T, uint16_t* __restrict__ out,
                                                                   float* __restrict__ lse) {
    __shared__ float wts[kMaxSplitsComb][kHeadsPerGroup];
    __shared__ float lsv[kMaxSplitsComb][kHeadsPerGroup];
    const int ns = S > 0 ? S : splits;
    const int hp = (H + kHeadsPerGroup - 1) / kHeadsPerGroup * kHeadsPerGroup;   // padded heads
    const int ngroups = hp / kHeadsPerGroup;
    const int part = blockIdx.x % kCombParts;
    const int t = blockIdx.x / kCombParts / ngroups, hg = blockIdx.x / kCombParts % ngroups;
    const int tid = threadIdx.x;
    // chunk c (16 bytes = 8 bf16) of the group: row rho = c/32 (nd = rho/4, ig = rho%4), partial
    // lanes L = 2*(c%32) and L+1, each with 4 consecutive heads 8*ig + 4*(L/32) + e at dims
    // 32*nd + L%32 (+1)
    const int c = part * kCombThreads + tid;
    const uint16_t* src = part_o + (int64_t)t * ns * hp * kDv + (int64_t)hg * kHeadsPerGroup * kDv + 8 * c;
    const int64_t sstride = (int64_t)hp * kDv;
    i32x4 raw[S > 0 ? S : 1];
    if constexpr (S > 0) {
#pragma unroll
        for (int s = 0; s < S; s++) raw[s] = *(const i32x4*)(src + s * sstride);
    }
    // the group's split log-sum-exps, loaded once by the whole workgroup (not split by split)
    for (int q = tid; q < ns * kHeadsPerGroup; q += kCombThreads)
        lsv[q / kHeadsPerGroup][q % kHeadsPerGroup] =
            part_lse[((int64_t)t * ns + q / kHeadsPerGroup) * hp + kHeadsPerGroup * hg + q % kHeadsPerGroup];
    __syncthreads();
    if (tid < kHeadsPerGroup) {
        const int head = kHeadsPerGroup * hg + tid;
        float m = -INFINITY;
        for (int s = 0; s < ns; s++) m = fmaxf(m, lsv[s][tid]);
        float wsum = 0.0f;
        for (int s = 0; s < ns; s++) wsum += m == -INFINITY ? 0.0f : expf(lsv[s][tid] - m);
        const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
        for (int s = 0; s < ns; s++) wts[s][tid] = m == -INFINITY ? 0.0f : expf(lsv[s][tid] - m) * inv;
        if (lse && part == 0 && head < H) lse[(int64_t)t * H + head] = wsum > 0.0f ? m + logf(wsum) : -INFINITY;
    }
    __syncthreads();
    const int rho = c >> 5, nd = rho >> 2, ig = rho & 3, L = 2 * (c & 31);
    const int hl0 = 8 * ig + 4 * (L >> 5);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto fold = [&](const i32x4& r, int s) {
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const uint32_t wd = (uint32_t)r[e / 2];
            const float v = bf16_bits_to_f32((uint16_t)(e % 2 ? wd >> 16 : wd & 0xffff));
            acc[e] = fmaf(wts[s][hl0 + (e % 4)], v, acc[e]);
        }
    };
    if constexpr (S > 0) {
#pragma unroll
        for (int s = 0; s < S; s++) fold(raw[s], s);
    } else {
        // batches of 8 loads in flight (clamped to the last split; the surplus is not folded)
        constexpr int kB = 8;
        for (int s0 = 0; s0 < ns; s0 += kB) {
            i32x4 r[kB];
#pragma unroll
            for (int u = 0; u < kB; u++) r[u] = *(const i32x4*)(src + min(s0 + u, ns - 1) * sstride);
#pragma unroll
            for (int u = 0; u < kB; u++)
                if (s0 + u < ns) fold(r[u], s0 + u);
        }
    }
    // the workgroup's output block (32 heads x 64 dims) goes through LDS so that each thread stores
    // 16 contiguous bytes of one head row (rather than four 4-byte pieces of four rows: about 1 us
    // less per decode launch)
    __shared__ uint32_t ot[kHeadsPerGroup][32 + 1];
    const int dl = 32 * nd + (L & 31) - 64 * part;
#pragma unroll
    for (int e = 0; e < 4; e++)
        ot[hl0 + e][dl >> 1] = (uint32_t)f32_to_bf16_bits(acc[e]) | ((uint32_t)f32_to_bf16_bits(acc[4 + e]) << 16);
    __syncthreads();
    {
        const int hh = tid >> 3, q4 = tid & 7;
        const int head = kHeadsPerGroup * hg + hh;
        if (head < H)
            *(i32x4*)(out + ((int64_t)t * H + head) * kDv + 64 * part + 8 * q4) =
                i32x4{(int)ot[hh][4 * q4], (int)ot[hh][4 * q4 + 1], (int)ot[hh][4 * q4 + 2], (int)ot[hh][4 * q4 + 3]};
    }
}

}  // namespace

int mla_splits(int T, int k) {
    if (T <= 0 || k <= 0) return 1;
    int s = (256 + T - 1) / T;                 // aim at one workgroup per CU
    s = min(s, max(1, k / 64));                // at least 64 index slots per split
    s = max(s, (k + kMaxList - 1) / kMaxList); // the LDS index list holds kMaxList slots
    return max(1, min(s, kMaxSplitsComb));
}

size_t mla_workspace_bytes(int T, int k, int H) {
    const int s = mla_splits(T, k);
    if (s == 1) return 0;
    const int hp = (H + kHeadsPerGroup - 1) / kHeadsPerGroup * kHeadsPerGroup;
    const size_t po = (size_t)T * s * hp * kDv * sizeof(uint16_t);
    const size_t pl = (size_t)T * s * hp * sizeof(float);
    return ((po + 255) & ~(size_t)255) + pl;
}

hipError_t launch_sparse_mla(const uint16_t* q, int H, const CacheView& lat, const BatchView& bv,
                             const int32_t* idx, int k, float softmax_scale, uint16_t* out, float* lse,
                             void* ws, hipStream_t st) {
    if (bv.T == 0) return hipSuccess;
    const int splits = mla_splits(bv.T, k);
    const int per_split = (k + splits - 1) / splits;
    uint16_t* part_o = nullptr;
    float* part_lse = nullptr;
    if (splits > 1) {
        part_o = (uint16_t*)ws;
        const int hp = (H + kHeadsPerGroup - 1) / kHeadsPerGroup * kHeadsPerGroup;
        const size_t po = (size_t)bv.T * splits * hp * kDv * sizeof(uint16_t);
        part_lse = (float*)((uint8_t*)ws + ((po + 255) & ~(size_t)255));
    }
    const float scale_log2 = softmax_scale * 1.44269504088896340736f;
    hipError_t e;
    sparse_mla_kernel<<<bv.T * splits, kMlaThreads, 0, st>>>(q, H, lat, bv, idx, k, per_split, splits, scale_log2,
                                                              out, lse, part_o, part_lse);
    e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int hp = (H + kHeadsPerGroup - 1) / kHeadsPerGroup * kHeadsPerGroup;
    const int blocks = bv.T * (hp / kHeadsPerGroup) * kCombParts;
    switch (splits) {
        case 2: mla_combine_kernel<2><<<blocks, kCombThreads, 0, st>>>(part_o, part_lse, splits, H, bv.T, out, lse); break;
        case 3: mla_combine_kernel<3><<<blocks, kCombThreads, 0, st>>>(part_o, part_lse, splits, H, bv.T, out, lse); break;
        case 4: mla_combine_kernel<4><<<blocks, kCombThreads, 0, st>>>(part_o, part_lse, splits, H, bv.T, out, lse); break;
        case 8: mla_combine_kernel<8><<<blocks, kCombThreads, 0, st>>>(part_o, part_lse, splits, H, bv.T, out, lse); break;
        case 16: mla_combine_kernel<16><<<blocks, kCombThreads, 0, st>>>(part_o, part_lse, splits, H, bv.T, out, lse); break;
        case 32: mla_combine_kernel<32><<<blocks, kCombThreads, 0, st>>>(part_o, part_lse, splits, H, bv.T, out, lse); break;
        default: mla_combine_kernel<0><<<blocks, kCombThreads, 0, st>>>(part_o, part_lse, splits, H, bv.T, out, lse); break;
    }
    return hipGetLastError();
}

}  // namespace dsa
