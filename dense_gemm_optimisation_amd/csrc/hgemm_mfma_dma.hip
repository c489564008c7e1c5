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
#include "dma_tile.hpp"

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
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;

    OpA opa;
    OpB opb;
    const int64_t span_a = A_KMAJOR ? (p.M - 1) * p.lda + p.K : (p.K - 1) * p.lda + p.M;
    const int64_t span_b = B_KMAJOR ? (p.N - 1) * p.ldb + p.K : (p.K - 1) * p.ldb + p.N;
    opa.init(p.A + t.batch * p.sA, p.lda, p.M, m0, span_a, wave, lane);
    opb.init(p.B + t.batch * p.sB, p.ldb, p.N, n0, span_b, wave, lane);

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

int64_t span_of(int64_t rows, int64_t cols, bool row_contig, int64_t ld) {
    // rows x cols with `cols` contiguous when row_contig
    return row_contig ? (rows - 1) * ld + cols : (cols - 1) * ld + rows;
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
    if ((p.a_kmajor ? p.K : p.M) % 8 || (p.b_kmajor ? p.K : p.N) % 8) return false;
    const int64_t limit = int64_t(1) << 30;
    if (2 * span_of(p.M, p.K, p.a_kmajor, p.lda) >= limit) return false;
    if (2 * span_of(p.K, p.N, !p.b_kmajor, p.ldb) >= limit) return false;
    return true;
}

hipError_t launch_hgemm_dma(const Problem &p, hipStream_t stream) {
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
    a.grid = TileGrid{(p.M + BM - 1) / BM, (p.N + BN - 1) / BN, p.batch, LIBGEMM_DMA_GROUP_M, 8};
    if (a.grid.count() > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int esz = p.out == Elem::F32 ? 4 : 2;
    // 16-byte chunks of C rows (8 bf16/fp16 or 4 fp32 elements)
    const int cw = 16 / esz;
    a.vec_c = (reinterpret_cast<uintptr_t>(p.C) % 16) == 0 && p.ldc % cw == 0 && a.sC % cw == 0;
    a.epi = p.epi;
    const bool bf = p.in == Elem::BF16;
    if (p.out == Elem::F32)
        return bf ? launch_layout<BF16, OUT_F32>(p, a, stream)
                  : launch_layout<F16, OUT_F32>(p, a, stream);
    return bf ? launch_layout<BF16, OUT_BF16>(p, a, stream)
              : launch_layout<F16, OUT_F16>(p, a, stream);
}

}  // namespace libgemm
