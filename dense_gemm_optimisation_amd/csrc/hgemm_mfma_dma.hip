// bf16 / fp16 GEMM on the CDNA4 matrix cores, fast path for aligned operands.
//
// Same block tile -> wave tile -> matrix instruction hierarchy as the general
// kernel ("GPU GEMM 优化完全拆解（三）", pinghaoyang.com.cn, section
// "从 kernel 到库"), with the data movement rebuilt around three gfx950
// features:
//
//   * direct global -> LDS loads (buffer_load_dwordx4 ... lds): every lane
//     moves 16 bytes into LDS at M0 + 16*lane without passing through
//     registers, so a wave fills 1 KiB of LDS per instruction.  This is the
//     role cp.async / TMA play on the pages' hardware (section 9.2 of
//     "CUDA GEMM 矩阵乘法优化指南", blog.zhenwei.site; section 3 of the hgemm
//     sm120 article, wingedge777.com).  The buffer's range check turns loads
//     outside the matrix into zeros, which handles ragged M, N and K tiles;
//   * LDS transpose reads (ds_read_b64_tr_b16): within each group of 16
//     lanes, lane j receives element j%4 of the 8-byte piece that lane
//     4e + j/4 addressed, as its element e.  If lane i of the group addresses
//     row i/4, columns 4(i%4)..4(i%4)+3 of a row-major 4 x 16 block, lane j
//     receives column j.  An operand stored contiguous along M or N (row-major
//     B, column-major A) is therefore copied into LDS unchanged and read in
//     the K-contiguous form the matrix instruction wants (the role ldmatrix
//     .trans plays in section "ldmatrix" of the pinghaoyang.com.cn page);
//   * v_mfma_f32_32x32x16_{bf16,f16} with the operands swapped (C^T blocks =
//     B^T A^T): each lane's accumulators then hold four consecutive columns
//     of one row of C, which the epilogue stores as one 8- or 16-byte vector.
//
// Pipeline: two LDS stages of BK = 64 (2 x 64 KiB).  While the matrix
// instructions of stage s run, stage s + 1 is landing in the other buffer;
// operand fragments are double-buffered in registers, so the reads for k-step
// kk + 1 are in flight during the matrix instructions of k-step kk, and the
// reads of the next stage's first k-step are issued before the current
// stage's last matrix instructions (the two buffering scopes, shared memory
// and registers, of section 3.3 of the hgemm sm120 article).  One barrier per
// stage separates the last reads of a buffer from the loads that refill it.
//
// The operand panels, their LDS layouts and the epilogue are in
// dma_tile.hpp, shared with the 8-bit kernel.
#include "dma_streamk.hpp"

namespace libgemm {
namespace {

using namespace dmatile;

struct BF16 {};
struct F16 {};

template <class T>
__device__ inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ inline f32x16 mfma32<BF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ inline f32x16 mfma32<F16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <class T, int OUT, bool A_KMAJOR, bool B_KMAJOR, int WAVES_M, int WAVES_N, int BK,
          int STAGES>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, 1) void hgemm_dma_kernel(DmaArgs p) {
    constexpr int WAVES = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int KK = BK / 16;  // matrix-instruction k steps per stage
    // LDS read instructions per k step: one per K-contiguous fragment, two
    // transpose reads per M/N-contiguous one
    constexpr int NREAD = FM * (A_KMAJOR ? 1 : 2) + FN * (B_KMAJOR ? 1 : 2);
    using OpA = Operand<A_KMAJOR, WAVES, BK>;
    using OpB = Operand<B_KMAJOR, WAVES, BK>;
    constexpr int PANEL = OpA::PANEL;
    constexpr int STAGE = 2 * PANEL;
    constexpr int PER_STAGE = OpA::PER_WAVE + OpB::PER_WAVE;  // direct loads per wave per stage
    static_assert(STAGES >= 2 && STAGES <= 5 && STAGES * STAGE <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

    TileCoord t = tile_of(p.grid, blockIdx.x);
    t.batch = uniform(t.batch);
    t.tm = uniform(t.tm);
    t.tn = uniform(t.tn);
    const int tid = threadIdx.x, lane = tid & 63;
    // The wave index is uniform across the wave; saying so keeps the LDS
    // destination of the direct loads (M0) in a scalar register.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Waves are dealt to the four SIMDs in turn, so consecutive waves share
    // a column block: the waves of one block column then sit on different
    // SIMDs, and when a tile hangs over the right edge of C (N = 128 in a
    // 256-wide tile, or one column of a last tile column) the waves left
    // with work are spread over all four matrix units.
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    // A wave whose WTM x WTN block lies wholly outside C only loads its share
    // of the panels and keeps the barriers.
    const bool live = m0 + wm * WTM < p.M && n0 + wn * WTN < p.N;

    OpA opa;
    OpB opb;
    opa.init(p.A + t.batch * p.sA, p.lda, p.M, m0, p.span_a, wave, lane);
    opb.init(p.B + t.batch * p.sB, p.ldb, p.N, n0, p.span_b, wave, lane);

    LDS char *lds = (LDS char *)smem;  // generic -> LDS address space
    const int64_t steps = (p.K + BK - 1) / BK;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Prologue: fill every stage buffer, then wait for the first.
#pragma unroll
    for (int st = 0; st < STAGES; ++st) {
        if (st < steps) {
            opa.issue(lds + st * STAGE, st, p.K, wave);
            opb.issue(lds + st * STAGE + PANEL, st, p.K, wave);
        }
    }
    wait_stages<PER_STAGE, STAGES>(int(steps - 1 < STAGES - 1 ? steps - 1 : STAGES - 1));
    __syncthreads();

    const int64_t main_steps = steps - 1;
    if (!live) {
        // the refills and barriers of the loop below, nothing else
        int b = 0;
        for (int64_t s = 0; s < main_steps; ++s) {
            const int64_t later = steps - 2 - s;
            wait_stages<PER_STAGE, STAGES>(int(later < STAGES - 2 ? later : STAGES - 2));
            __syncthreads();
            const int64_t refill = s + STAGES;
            if (refill < steps) {
                opa.issue(lds + b * STAGE, refill, p.K, wave);
                opb.issue(lds + b * STAGE + PANEL, refill, p.K, wave);
            }
            b = b + 1 == STAGES ? 0 : b + 1;
        }
        return;
    }

    u32x4 fa[2][FM], fb[2][FN];
    auto read = [&](int buf, int kk, int slot) {
        const LDS char *sa = lds + buf * STAGE;
        const LDS char *sb = sa + PANEL;
        // in the order the matrix instructions consume them: all of B's
        // fragments are used by the first row of instructions
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[slot][j] = opb.frag(sb, wn * WTN + j * 32, kk, lane);
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[slot][i] = opa.frag(sa, wm * WTM + i * 32, kk, lane);
    };
    read(0, 0, 0);

    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<T>(fb[slot][j], fa[slot][i], acc[i][j]);
    };

    // Every stage but the last.  Its first KK - 1 k16 steps read the next
    // step's fragments while computing.  Its last step waits for stage s + 1
    // (this wave's loads, then every wave's through the barrier, which also
    // says every wave is done reading this stage's buffer), reads stage
    // s + 1's first fragments, and runs its matrix instructions with the
    // refill of this buffer (stage s + STAGES) spread between them, so a load
    // that waits for the memory pipeline does not hold back the matrix core.
    // The last stage is peeled off so that no branch joins the code after the
    // barrier: the LDS counter waits stay exact there.
    int buf = 0;
    for (int64_t s = 0; s < main_steps; ++s) {
#pragma unroll
        for (int kk = 0; kk < KK - 1; ++kk) {
            read(buf, kk + 1, (kk & 1) ^ 1);
            mfmas(kk & 1);
            interleave_reads<NREAD, FM * FN>();
        }
        constexpr int LAST = (KK - 1) & 1;
        const int64_t later = steps - 2 - s;
        wait_stages<PER_STAGE, STAGES>(int(later < STAGES - 2 ? later : STAGES - 2));
        wait_lgkmcnt0();
        __syncthreads();
        const int nbuf = buf + 1 == STAGES ? 0 : buf + 1;
        read(nbuf, 0, LAST ^ 1);
        const int64_t refill = s + STAGES;
        const bool do_refill = refill < steps;
        const u32x4 ra = opa.rsrc(refill), rb = opb.rsrc(refill);
        const uint32_t la = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds + buf * STAGE));
        const uint32_t lb = la + PANEL;
        const int64_t kleft = p.K - refill * BK;
        // one direct load after each matrix instruction
        static_assert(PER_STAGE <= FM * FN, "loads per instruction");
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[i][j] = mfma32<T>(fb[LAST][j], fa[LAST][i], acc[i][j]);
                const int q = i * FN + j;
                if (do_refill) {
                    if (q < OpA::PER_WAVE) opa.load(ra, la, q, kleft, wave);
                    else if (q < PER_STAGE) opb.load(rb, lb, q - OpA::PER_WAVE, kleft, wave);
                }
            }
        buf = nbuf;
    }
    // The last stage.
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if (kk < KK - 1) read(buf, kk + 1, (kk & 1) ^ 1);
        mfmas(kk & 1);
        interleave_reads<NREAD, FM * FN>();
    }

    // C is staged in stage buffers the last stage does not use: every wave
    // finished reading them before the last barrier, and no load targets
    // them any more, so no further barrier is needed.  Staging takes NEED
    // consecutive buffers: the next one when one suffices, else the first
    // NEED or the NEED after them, whichever excludes the last stage's.
    constexpr int NEED = (WAVES * 32 * WTN * 4 + STAGE - 1) / STAGE;
    static_assert(NEED == 1 || 2 * NEED <= STAGES, "epilogue staging fits beside the last stage");
    const int free0 = NEED == 1 ? (buf + 1 == STAGES ? 0 : buf + 1) : (buf >= NEED ? 0 : NEED);
    LDS char *stage_free = lds + free0 * STAGE;
    store_tile_lds<OUT, FM, FN>(p, acc, t.batch, m0 + wm * WTM, n0 + wn * WTN, lane,
                                reinterpret_cast<LDS float *>(stage_free) + wave * 32 * WTN);
}

// The same steps and epilogue as functions, for the stream-K kernel (the
// one-tile kernel above keeps them inline, where they compile to slightly
// faster code).
// k steps [kb, ke) (BK each) of tile t into acc through the LDS ring at
// `lds`; returns the ring buffer the last step used (the epilogue stages C in
// the others).  On return every wave has passed the last barrier.
template <class T, bool A_KMAJOR, bool B_KMAJOR, int WAVES_M, int WAVES_N, int BK, int STAGES>
__device__ __forceinline__ int dma_tile_steps(const DmaArgs &p, LDS char *lds, const TileCoord &t,
                                              int64_t kb, int64_t ke,
                                              f32x16 (&acc)[BM / WAVES_M / 32][BN / WAVES_N / 32]) {
    constexpr int WAVES = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int KK = BK / 16;  // matrix-instruction k steps per stage
    // LDS read instructions per k step: one per K-contiguous fragment, two
    // transpose reads per M/N-contiguous one
    constexpr int NREAD = FM * (A_KMAJOR ? 1 : 2) + FN * (B_KMAJOR ? 1 : 2);
    using OpA = Operand<A_KMAJOR, WAVES, BK>;
    using OpB = Operand<B_KMAJOR, WAVES, BK>;
    constexpr int PANEL = OpA::PANEL;
    constexpr int STAGE = 2 * PANEL;
    constexpr int PER_STAGE = OpA::PER_WAVE + OpB::PER_WAVE;  // direct loads per wave per stage

    const int tid = threadIdx.x, lane = tid & 63;
    // The wave index is uniform across the wave; saying so keeps the LDS
    // destination of the direct loads (M0) in a scalar register.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;

    OpA opa;
    OpB opb;
    opa.init(p.A + t.batch * p.sA, p.lda, p.M, m0, p.span_a, wave, lane);
    opb.init(p.B + t.batch * p.sB, p.ldb, p.N, n0, p.span_b, wave, lane);

    const int64_t steps = ke - kb;

    // Prologue: fill every stage buffer, then wait for the first.
#pragma unroll
    for (int st = 0; st < STAGES; ++st) {
        if (st < steps) {
            opa.issue(lds + st * STAGE, kb + st, p.K, wave);
            opb.issue(lds + st * STAGE + PANEL, kb + st, p.K, wave);
        }
    }
    wait_stages<PER_STAGE, STAGES>(int(steps - 1 < STAGES - 1 ? steps - 1 : STAGES - 1));
    __syncthreads();

    u32x4 fa[2][FM], fb[2][FN];
    auto read = [&](int buf, int kk, int slot) {
        const LDS char *sa = lds + buf * STAGE;
        const LDS char *sb = sa + PANEL;
        // in the order the matrix instructions consume them: all of B's
        // fragments are used by the first row of instructions
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[slot][j] = opb.frag(sb, wn * WTN + j * 32, kk, lane);
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[slot][i] = opa.frag(sa, wm * WTM + i * 32, kk, lane);
    };
    read(0, 0, 0);

    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<T>(fb[slot][j], fa[slot][i], acc[i][j]);
    };

    // Every stage but the last.  Its first KK - 1 k16 steps read the next
    // step's fragments while computing.  Its last step waits for stage s + 1
    // (this wave's loads, then every wave's through the barrier, which also
    // says every wave is done reading this stage's buffer), reads stage
    // s + 1's first fragments, and runs its matrix instructions with the
    // refill of this buffer (stage s + STAGES) spread between them, so a load
    // that waits for the memory pipeline does not hold back the matrix core.
    // The last stage is peeled off so that no branch joins the code after the
    // barrier: the LDS counter waits stay exact there.
    int buf = 0;
    const int64_t main_steps = steps - 1;
    for (int64_t s = 0; s < main_steps; ++s) {
#pragma unroll
        for (int kk = 0; kk < KK - 1; ++kk) {
            read(buf, kk + 1, (kk & 1) ^ 1);
            mfmas(kk & 1);
            interleave_reads<NREAD, FM * FN>();
        }
        constexpr int LAST = (KK - 1) & 1;
        const int64_t later = steps - 2 - s;
        wait_stages<PER_STAGE, STAGES>(int(later < STAGES - 2 ? later : STAGES - 2));
        wait_lgkmcnt0();
        __syncthreads();
        const int nbuf = buf + 1 == STAGES ? 0 : buf + 1;
        read(nbuf, 0, LAST ^ 1);
        const int64_t refill = s + STAGES;
        const bool do_refill = refill < steps;
        const u32x4 ra = opa.rsrc(kb + refill), rb = opb.rsrc(kb + refill);
        const uint32_t la = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds + buf * STAGE));
        const uint32_t lb = la + PANEL;
        const int64_t kleft = p.K - (kb + refill) * BK;
        // one direct load after each matrix instruction
        static_assert(PER_STAGE <= FM * FN, "loads per instruction");
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[i][j] = mfma32<T>(fb[LAST][j], fa[LAST][i], acc[i][j]);
                const int q = i * FN + j;
                if (do_refill) {
                    if (q < OpA::PER_WAVE) opa.load(ra, la, q, kleft, wave);
                    else if (q < PER_STAGE) opb.load(rb, lb, q - OpA::PER_WAVE, kleft, wave);
                }
            }
        buf = nbuf;
    }
    // The last stage.
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if (kk < KK - 1) read(buf, kk + 1, (kk & 1) ^ 1);
        mfmas(kk & 1);
        interleave_reads<NREAD, FM * FN>();
    }
    return buf;
}

// C is staged in stage buffers the last stage does not use: every wave
// finished reading them before the last barrier, and no load targets them
// any more, so no further barrier is needed.  Staging takes NEED consecutive
// buffers: the next one when one suffices, else the first NEED or the NEED
// after them, whichever excludes the last stage's.
template <int OUT, int WAVES_M, int WAVES_N, int BK, int STAGES>
__device__ __forceinline__ void dma_tile_store(const DmaArgs &p, LDS char *lds, const TileCoord &t,
                                               int buf,
                                               const f32x16 (&acc)[BM / WAVES_M / 32][BN / WAVES_N / 32]) {
    constexpr int WAVES = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int STAGE = 2 * Operand<true, WAVES, BK>::PANEL;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    constexpr int NEED = (WAVES * 32 * WTN * 4 + STAGE - 1) / STAGE;
    static_assert(NEED == 1 || 2 * NEED <= STAGES, "epilogue staging fits beside the last stage");
    const int free0 = NEED == 1 ? (buf + 1 == STAGES ? 0 : buf + 1) : (buf >= NEED ? 0 : NEED);
    LDS char *stage_free = lds + free0 * STAGE;
    store_tile_lds<OUT, FM, FN>(p, acc, t.batch, t.tm * BM + wm * WTM, t.tn * BN + wn * WTN, lane,
                                reinterpret_cast<LDS float *>(stage_free) + wave * 32 * WTN);
}

// Stream-K schedule of the fast path (section 12.5 of "CUDA GEMM 矩阵乘法优化
// 指南", blog.zhenwei.site, persistent kernels and Stream-K), the same split
// as the general kernel's: one workgroup per compute unit (G); the tiles
// filling whole waves of G are computed whole, tile w + n*G by workgroup w;
// the (tile, k step) iterations of the other tiles are split evenly over
// Gs = min(G, iterations) workgroups; a piece covering a whole tile is stored
// through the epilogue, any other is written to the workgroup's slot 2w (the
// piece holding its last iteration) or 2w + 1 (its first), and
// dma_streamk_fixup (dma_streamk.hpp) adds the pieces of each cut tile in
// increasing workgroup order and applies the epilogue.
template <class T, int OUT, bool A_KMAJOR, bool B_KMAJOR, int WAVES_M, int WAVES_N, int BK,
          int STAGES>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, 1) void hgemm_dma_streamk_kernel(DmaArgs p,
                                                                                   DmaStreamK sk) {
    constexpr int FM = BM / WAVES_M / 32, FN = BN / WAVES_N / 32;
    constexpr int THREADS = WAVES_M * WAVES_N * 64;
    constexpr int STAGE = 2 * Operand<A_KMAJOR, WAVES_M * WAVES_N, BK>::PANEL;
    static_assert(STAGES * STAGE <= 160 * 1024, "LDS budget");
    static_assert(FM * FN * 4 * THREADS * 16 == SK_SLOT * 4, "a slot holds one tile");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
    LDS char *lds = (LDS char *)smem;

    // logical workgroup: the hardware id regrouped per XCD, so that the
    // workgroups of one die take consecutive tiles and ranges
    const int64_t G = gridDim.x, S = sk.steps;
    const int64_t w = uniform(xcd_remap(blockIdx.x, G, 8));
    const int64_t n_dp = uniform(sk_whole_tiles(sk, w, G));
    const int64_t begin = uniform(sk_begin(sk, w));
    const int64_t end = uniform(sk_end(sk, w));
    int64_t it = begin;
    for (int64_t item = 0;; ++item) {
        int64_t tile, kb, ke, local = 0;
        if (item < n_dp) {
            tile = w + item * G;
            kb = 0;
            ke = S;
        } else {
            if (it >= end) break;
            local = uniform(it / S);
            const StreamKPiece pc = sk_piece(sk, local, it, end);
            kb = pc.kb;
            ke = pc.ke;
            tile = sk.dp_tiles + local;
            it = local * S + ke;
        }
        TileCoord t = tile_of(p.grid, tile);
        t.batch = uniform(t.batch);
        t.tm = uniform(t.tm);
        t.tn = uniform(t.tn);
        // the previous piece's epilogue has read its staging buffers before
        // the ring is refilled
        if (item > 0) __syncthreads();
        f32x16 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        const int buf = dma_tile_steps<T, A_KMAJOR, B_KMAJOR, WAVES_M, WAVES_N, BK, STAGES>(
            p, lds, t, kb, ke, acc);
        if (kb == 0 && ke == S) {
            dma_tile_store<OUT, WAVES_M, WAVES_N, BK, STAGES>(p, lds, t, buf, acc);
        } else {
            store_partial<FM, FN, WAVES_M * WAVES_N * 64>(sk, sk_slot(sk, w, local, end), acc);
        }
    }
}

// Tile configuration of the fast path: 256 x 256 block tile, BK-deep
// stages, a ring of STAGES buffers, WAVES_M x WAVES_N waves.
#ifndef LIBGEMM_DMA_WM
#define LIBGEMM_DMA_WM 2
#endif
#ifndef LIBGEMM_DMA_WN
#define LIBGEMM_DMA_WN 4
#endif
#ifndef LIBGEMM_DMA_BK
#define LIBGEMM_DMA_BK 64
#endif
#ifndef LIBGEMM_DMA_STAGES
#define LIBGEMM_DMA_STAGES 2
#endif
#ifndef LIBGEMM_DMA_GROUP_M
#define LIBGEMM_DMA_GROUP_M 8
#endif

template <class T, int OUT, bool AK, bool BKM>
hipError_t launch(DmaArgs &a, hipStream_t stream) {
    constexpr int WM = LIBGEMM_DMA_WM, WN = LIBGEMM_DMA_WN;
    void *args[] = {&a};
    return hipLaunchKernel(
        reinterpret_cast<const void *>(
            &hgemm_dma_kernel<T, OUT, AK, BKM, WM, WN, LIBGEMM_DMA_BK, LIBGEMM_DMA_STAGES>),
        dim3(static_cast<unsigned>(a.grid.count())), dim3(WM * WN * 64), args, 0, stream);
}

template <class T, int OUT>
hipError_t launch_layout(const Problem &p, DmaArgs &a, hipStream_t stream) {
    if (p.a_kmajor)
        return p.b_kmajor ? launch<T, OUT, true, true>(a, stream)
                          : launch<T, OUT, true, false>(a, stream);
    return p.b_kmajor ? launch<T, OUT, false, true>(a, stream)
                      : launch<T, OUT, false, false>(a, stream);
}

template <class T, int OUT, bool AK, bool BKM>
hipError_t launch_sk(DmaArgs &a, DmaStreamK &sk, int64_t grid, hipStream_t stream) {
    constexpr int WM = LIBGEMM_DMA_WM, WN = LIBGEMM_DMA_WN;
    void *args[] = {&a, &sk};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void *>(&hgemm_dma_streamk_kernel<T, OUT, AK, BKM, WM, WN,
                                                                 LIBGEMM_DMA_BK, LIBGEMM_DMA_STAGES>),
        dim3(static_cast<unsigned>(grid)), dim3(WM * WN * 64), args, 0, stream);
    if (e != hipSuccess) return e;
    return launch_dma_streamk_fixup<OUT, WM, WN>(a, sk, a.grid.count(), stream);
}

template <class T, int OUT>
hipError_t launch_sk_layout(const Problem &p, DmaArgs &a, DmaStreamK &sk, int64_t grid,
                            hipStream_t stream) {
    if (p.a_kmajor)
        return p.b_kmajor ? launch_sk<T, OUT, true, true>(a, sk, grid, stream)
                          : launch_sk<T, OUT, true, false>(a, sk, grid, stream);
    return p.b_kmajor ? launch_sk<T, OUT, false, true>(a, sk, grid, stream)
                      : launch_sk<T, OUT, false, false>(a, sk, grid, stream);
}

}  // namespace

// The fast path needs every operand chunk either fully inside or fully
// outside its matrix (extents along the contiguous dimension, leading
// dimensions and batch strides multiples of 8 elements, 16-byte aligned
// bases) and slices whose byte extent fits the buffer range check.
bool hgemm_dma_eligible(const Problem &p) {
    if (p.in != Elem::BF16 && p.in != Elem::F16) return false;
    const int64_t sa = p.batch > 1 ? p.sA : 0, sb = p.batch > 1 ? p.sB : 0;
    if (!vec16_ok(p.A, p.lda, sa, 2) || !vec16_ok(p.B, p.ldb, sb, 2)) return false;
    if (!p.packed && ((p.a_kmajor ? p.K : p.M) % 8 || (p.b_kmajor ? p.K : p.N) % 8)) return false;
    const int64_t limit = int64_t(1) << 30;
    if (2 * operand_span_a(p) >= limit || 2 * operand_span_b(p) >= limit) return false;
    return true;
}

namespace {

DmaArgs make_dma_args(const Problem &p, int32_t xcds) {
    DmaArgs a{};
    a.M = p.M;
    a.N = p.N;
    a.K = p.K;
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.A = static_cast<const uint16_t *>(p.A);
    a.B = static_cast<const uint16_t *>(p.B);
    a.C = p.C;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.sA = p.batch > 1 ? p.sA : 0;
    a.sB = p.batch > 1 ? p.sB : 0;
    a.sC = p.batch > 1 ? p.sC : 0;
    a.grid = TileGrid{(p.M + BM - 1) / BM, (p.N + BN - 1) / BN, p.batch, LIBGEMM_DMA_GROUP_M, xcds};
    a.epi = p.epi;
    a.span_a = operand_span_a(p);
    a.span_b = operand_span_b(p);
    return a;
}

// Cost of the partial-tile exchange of the fast path's stream-K schedule, in
// k steps of one tile (1.8 us at 4096^3), measured on MI355X: about 0.14
// per partial tile written and read back (there are at most Gs + T_r), and 2
// for the fix-up launch.
constexpr double DMA_SK_STEPS_PER_PIECE = 0.14;
constexpr double DMA_SK_FIXED_STEPS = 2.0;

}  // namespace

hipError_t launch_hgemm_dma(const Problem &p, hipStream_t stream) {
    DmaArgs a = make_dma_args(p, 8);
    if (a.grid.count() > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool bf = p.in == Elem::BF16;
    if (elem_is_8bit(p.out))
        return bf ? launch_layout<BF16, OUT_F8>(p, a, stream)
                  : launch_layout<F16, OUT_F8>(p, a, stream);
    if (p.out == Elem::F32)
        return bf ? launch_layout<BF16, OUT_F32>(p, a, stream)
                  : launch_layout<F16, OUT_F32>(p, a, stream);
    return bf ? launch_layout<BF16, OUT_BF16>(p, a, stream)
              : launch_layout<F16, OUT_F16>(p, a, stream);
}

// Step time over partial-tile time for streamk_groups (1.8 us per k step of the direct-load kernel at 4096^3, 0.13 us per partial tile).
#ifndef LIBGEMM_DMA_SK_RATIO
#define LIBGEMM_DMA_SK_RATIO 14
#endif

// Worth it when the steps the cut last wave saves exceed the exchange: the
// last wave takes ceil(T_r * S / Gs) steps per workgroup instead of S, and
// the exchange grows with the pieces, about Gs + T_r partial tiles (G =
// HGEMM_STREAMK_MAX_GRID compute units, Gs from streamk_groups).
bool hgemm_dma_streamk_eligible(const Problem &p, bool force) {
    if (!hgemm_dma_eligible(p)) return false;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.batch;
    const int64_t steps = (p.K + LIBGEMM_DMA_BK - 1) / LIBGEMM_DMA_BK;
    const int64_t g = HGEMM_STREAMK_MAX_GRID;
    const int64_t cut = tiles % g;
    if (cut == 0 || tiles >= (int64_t(1) << 24) || steps >= (int64_t(1) << 24)) return false;
    if (force) return true;
    const int64_t gs = streamk_groups(g, cut, steps, LIBGEMM_DMA_SK_RATIO);
    const int64_t tail = (cut * steps + gs - 1) / gs;
    return double(steps - tail) > DMA_SK_STEPS_PER_PIECE * double(gs + cut) + DMA_SK_FIXED_STEPS;
}

namespace {

// The stream-K split of p: one workgroup per compute unit of MI355X (G =
// HGEMM_STREAMK_MAX_GRID; on a part with fewer units the schedule is still
// correct, the workgroups just do not all run at once).
StreamKSplit dma_streamk_split(const Problem &p) {
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.batch;
    return streamk_split(tiles, (p.K + LIBGEMM_DMA_BK - 1) / LIBGEMM_DMA_BK, HGEMM_STREAMK_MAX_GRID,
                         LIBGEMM_DMA_SK_RATIO);
}

}  // namespace

int64_t hgemm_dma_streamk_bytes(const Problem &p) {
    return 2 * dma_streamk_split(p).groups * int64_t(SK_SLOT) * 4;
}

hipError_t launch_hgemm_dma_streamk(const Problem &p, void *workspace, hipStream_t stream) {
    DmaArgs a = make_dma_args(p, 1);  // the work order itself spreads tiles over the dies
    DmaStreamK sk{};
    static_cast<StreamKSplit &>(sk) = dma_streamk_split(p);
    sk.partials = static_cast<float *>(workspace);
    const int64_t grid = streamk_grid(sk, HGEMM_STREAMK_MAX_GRID);
    if (grid == 0) return hipSuccess;
    const bool bf = p.in == Elem::BF16;
    if (p.out == Elem::F32)
        return bf ? launch_sk_layout<BF16, OUT_F32>(p, a, sk, grid, stream)
                  : launch_sk_layout<F16, OUT_F32>(p, a, sk, grid, stream);
    return bf ? launch_sk_layout<BF16, OUT_BF16>(p, a, sk, grid, stream)
              : launch_sk_layout<F16, OUT_F16>(p, a, sk, grid, stream);
}

}  // namespace libgemm
