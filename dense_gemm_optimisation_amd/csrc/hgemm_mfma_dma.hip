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
// LDS layouts (both XOR-swizzled in 16-byte chunks; the swizzle is applied by
// choosing which global chunk each lane fetches, because the direct loads
// place lanes linearly):
//   K-contiguous operand: [256 rows][64 k], 128 B per row, chunk c of row r
//     at c ^ ((r ^ (r >> 3)) & 7): 16 consecutive rows read at one logical
//     chunk hit distinct banks.
//   M/N-contiguous operand: [64 k][256 cols], 512 B per row, chunk c of row r
//     at c ^ 4*t(r), t(r) = (r & 7) ^ 4*((r >> 3) & 1): the eight rows one
//     transpose read touches fall in eight different 64-byte bank groups.
#include "gemm_problem.hpp"
#include "lds_dma.hpp"
#include "tile_schedule.hpp"

namespace libgemm {
namespace {

using dma::OOB;
using dma::direct_load16;
using dma::uniform;
using dma::wait_lgkmcnt0;
using dma::wait_vmcnt;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256;       // block tile (rows of A and columns of B)
constexpr int OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2;

struct DmaArgs {
    int64_t M, N, K;
    float alpha, beta;
    const uint16_t *A;
    const uint16_t *B;
    void *C;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;
    TileGrid grid;
    int vec_c;
    Epilogue epi;
};

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

// Swizzle of a K-contiguous panel row (CH 16-byte chunks per row): a
// permutation of [0, CH) chosen so that 16 consecutive rows read at one
// logical chunk fall on 16 distinct 16-byte bank groups of a 256-byte wide
// LDS (and 8 consecutive rows on 8 distinct groups of a 128-byte one).
template <int CH>
__device__ inline int swz_k(int row) {
    if (CH == 8) return (row ^ (row >> 3)) & 7;
    return ((row >> 1) ^ (row >> 2)) & 3;  // CH == 4
}
// Swizzle of an M/N-contiguous panel row (32 chunks of 16 bytes): XOR of
// chunk bits 2..4 with t(r) = (r & 7) ^ 4*((r >> 3) & 1), so the eight rows
// one transpose read touches use eight different 64-byte bank groups.
__device__ inline int swz_mn(int krow) { return ((krow & 7) ^ (((krow >> 3) & 1) << 2)) << 2; }

// One operand panel of the tile (256 rows of A or 256 columns of B, BK deep):
// where each lane fetches from, and how the wave reads fragments back.
template <bool KMAJOR, int WAVES, int BK>
struct Operand {
    static constexpr int PANEL = 256 * BK * 2;        // bytes
    static constexpr int BLOCKS = PANEL / 1024;       // 1 KiB direct loads per panel
    static constexpr int PER_WAVE = BLOCKS / WAVES;   // direct loads per wave per stage
    static constexpr int CH = BK / 8;                 // chunks per K-contiguous row
    static constexpr int ROWS_PER_BLOCK = 1024 / (2 * BK);
    static_assert(PER_WAVE >= 1 && BLOCKS % WAVES == 0, "panel split over waves");
    uint32_t voff[PER_WAVE];  // byte offset of this lane's chunk, stage 0
    int kl[PER_WAVE];         // k index (within a stage) of this lane's chunk
    const uint16_t *base;
    int64_t bytes;            // extent of the operand slice in bytes
    int64_t step;             // bytes the base advances per stage

    // X(r, k): KMAJOR -> X[r*ld + k], else X[k*ld + r]; rows [r0, r0+256) of R.
    __device__ void init(const uint16_t *x, int64_t ld, int64_t R, int64_t r0, int64_t span,
                         int wave, int lane) {
        base = x;
        bytes = span * 2;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int blk = wave * PER_WAVE + i;
            if (KMAJOR) {
                const int row = blk * ROWS_PER_BLOCK + lane / CH;
                const int c = (lane % CH) ^ swz_k<CH>(row);
                kl[i] = c * 8;
                const int64_t gr = r0 + row;
                voff[i] = gr < R ? uint32_t((gr * ld + c * 8) * 2) : OOB;
            } else {
                const int krow = blk * 2 + (lane >> 5);
                const int c = (lane & 31) ^ swz_mn(krow);
                kl[i] = krow;
                const int64_t gc = r0 + c * 8;
                voff[i] = gc < R ? uint32_t((krow * ld + gc) * 2) : OOB;
            }
        }
        step = KMAJOR ? int64_t(BK) * 2 : int64_t(BK) * ld * 2;
    }

    // Buffer descriptor of the slice that stage `stage` starts (raw buffer:
    // base, stride 0, size in bytes, 32-bit format); reads past its end
    // return zero.
    __device__ u32x4 rsrc(int64_t stage) const {
        const int64_t off = uniform(stage * step);
        return dma::raw_buffer(static_cast<uint64_t>(uniform(reinterpret_cast<int64_t>(base) + off)),
                               static_cast<uint32_t>(uniform(bytes - off)));
    }

    // Direct load i (of PER_WAVE) of this wave for the stage with descriptor
    // rs and kleft = K - stage*BK valid k values, into the panel at lds0.
    __device__ void load(u32x4 rs, uint32_t lds0, int i, int64_t kleft, int wave) const {
        const uint32_t v = (kleft < BK && kl[i] >= kleft) ? OOB : voff[i];
        direct_load16(rs, lds0 + (wave * PER_WAVE + i) * 1024, v);
    }

    // All direct loads of stage `stage` (k from stage*BK) into the panel at dst.
    __device__ void issue(LDS char *dst, int64_t stage, int64_t K, int wave) const {
        const u32x4 rs = rsrc(stage);
        const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) load(rs, lds0, i, K - stage * BK, wave);
    }

    // Fragment of 32 rows (from row `row0` of the panel) for k16 step kk.
    __device__ u32x4 frag(const LDS char *panel, int row0, int kk, int lane) const {
        if (KMAJOR) {
            const int row = row0 + (lane & 31);
            const int c = kk * 2 + (lane >> 5);
            return *reinterpret_cast<const LDS u32x4 *>(panel + row * (2 * BK) +
                                                        ((c ^ swz_k<CH>(row)) << 4));
        } else {
            const int g = lane >> 5, h = (lane >> 4) & 1, ii = lane & 15;
            const int col = row0 + h * 16 + 4 * (ii & 3);
            u32x4 out;
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const int krow = kk * 16 + g * 8 + e2 * 4 + (ii >> 2);
                const int c = (col >> 3) ^ swz_mn(krow);
                const LDS s16x4 *p = reinterpret_cast<const LDS s16x4 *>(
                    panel + krow * 512 + (c << 4) + ((col & 7) << 1));
                const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                              const_cast<LDS s16x4 *>(p)));
                out[2 * e2] = v[0];
                out[2 * e2 + 1] = v[1];
            }
            return out;
        }
    }
};

// Epilogue through LDS.  One wave's tile is FM x FN blocks of 32 x 32 (top
// left at (mw, nw)); block (i, j) holds C^T (the operands were swapped), so
// lane l has row mw + 32i + l % 32 and, in registers 4q .. 4q+3, columns
// nw + 32j + 8q + 4*(l / 32) + 0..3.  Each 32-row strip i is written to the
// wave's own LDS area as alpha*acc in fp32, row-major with its 16-byte
// chunks XOR-swizzled by row (chunk c of row r at c ^ (r mod 16), so the 32
// rows one write instruction touches spread over the banks), then read back so
// that every lane owns 16 contiguous bytes of one output row: a store
// instruction then writes whole rows of the strip (8 rows of 128 bytes for
// a 64-column bf16 strip) instead of 32 rows of 16 bytes, and C_old is read
// the same way when beta != 0.  Rows or columns outside C are skipped, and a
// chunk that crosses the right edge of C, or any chunk when C's rows are not
// 16-byte aligned, is stored element by element.
template <int OUT, int FM, int FN>
__device__ inline void store_tile_lds(const DmaArgs &p, const f32x16 (&acc)[FM][FN], int64_t batch,
                                      int64_t mw, int64_t nw, int lane, LDS float *scratch) {
    constexpr int W = FN * 32;          // strip width (columns)
    constexpr int PITCH = W;            // floats per staged row
    constexpr int SWZ = W / 4 - 1 < 15 ? W / 4 - 1 : 15;
    auto at = [&](int r, int col) {     // staged float (r, col), col a multiple of 4
        return scratch + r * PITCH + ((((col >> 2) ^ (r & SWZ))) << 2);
    };
    constexpr int CW = OUT == OUT_F32 ? 4 : 8;  // output elements per 16-byte chunk
    constexpr int CPR = W / CW;         // chunks per row
    constexpr int RPI = 64 / CPR;       // rows per store instruction
    char *Cb = static_cast<char *>(p.C) + batch * p.sC * (OUT == OUT_F32 ? 4 : 2);
    auto dec = [](uint16_t b) {
        return OUT == OUT_BF16 ? __builtin_bit_cast(float, uint32_t(b) << 16)
                               : static_cast<float>(__builtin_bit_cast(_Float16, b));
    };
    auto enc = [](float x) {
        return OUT == OUT_BF16 ? __builtin_bit_cast(uint16_t, static_cast<__bf16>(x))
                               : __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    };
    // Fused epilogue: the bias values this lane adds, loaded up front (its
    // columns are the same in every row it writes; its rows are known).
    const bool epi = p.epi.active();
    const int lcc = (lane % CPR) * CW;
    float bcol[CW], brow[FM][32 / RPI];
#pragma unroll
    for (int e = 0; e < CW; ++e) bcol[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) brow[i][it] = 0.0f;
    if (p.epi.bias != nullptr) {
        if (p.epi.per_row) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int it = 0; it < 32 / RPI; ++it)
                    brow[i][it] = epilogue_bias_or_zero(p.epi, batch,
                                                        mw + i * 32 + it * RPI + lane / CPR, p.M);
        } else {
#pragma unroll
            for (int e = 0; e < CW; ++e)
                bcol[e] = epilogue_bias_or_zero(p.epi, batch, nw + lcc + e, p.N);
        }
    }
    auto finish = [&](float v, int i, int it, int e) {
        return epilogue_act(p.epi.act, v + bcol[e] + brow[i][it]);
    };
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        // stage alpha*acc of strip i
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = p.alpha * acc[i][j][4 * q + e];
                *reinterpret_cast<LDS f32x4 *>(at(lane & 31, j * 32 + q * 8 + 4 * (lane >> 5))) = v;
            }
        // write it out row by row (the wave's own LDS reads follow its writes)
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
            const int r = it * RPI + lane / CPR, cc = (lane % CPR) * CW;
            const int64_t m = mw + i * 32 + r, n = nw + cc;
            float x[CW];
#pragma unroll
            for (int e4 = 0; e4 < CW / 4; ++e4) {
                const f32x4 v = *reinterpret_cast<const LDS f32x4 *>(at(r, cc + 4 * e4));
#pragma unroll
                for (int e = 0; e < 4; ++e) x[4 * e4 + e] = v[e];
            }
            if (m >= p.M || n >= p.N) continue;
            const int64_t off = m * p.ldc + n;
            if (p.vec_c && n + CW <= p.N) {
                if (OUT == OUT_F32) {
                    float *c = reinterpret_cast<float *>(Cb) + off;
                    f32x4 v = {x[0], x[1], x[2], x[3]};
                    if (p.beta != 0.0f) {
                        const f32x4 o = *reinterpret_cast<const f32x4 *>(c);
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(p.beta, o[e], v[e]);
                    }
                    if (epi)
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = finish(v[e], i, it, e);
                    *reinterpret_cast<f32x4 *>(c) = v;
                } else {
                    uint16_t *c = reinterpret_cast<uint16_t *>(Cb) + off;
                    if (p.beta != 0.0f) {
                        const u32x4 o = *reinterpret_cast<const u32x4 *>(c);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            x[e] = __builtin_fmaf(p.beta, dec(uint16_t(o[e / 2] >> (16 * (e % 2)))), x[e]);
                    }
                    if (epi)
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[e] = finish(x[e], i, it, e);
                    u32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = uint32_t(enc(x[2 * e])) | (uint32_t(enc(x[2 * e + 1])) << 16);
                    *reinterpret_cast<u32x4 *>(c) = w;
                }
            } else {
                const int nvalid = p.N - n < CW ? int(p.N - n) : CW;
                for (int e = 0; e < nvalid; ++e) {
                    if (OUT == OUT_F32) {
                        float *c = reinterpret_cast<float *>(Cb) + off + e;
                        float v = p.beta != 0.0f ? __builtin_fmaf(p.beta, *c, x[e]) : x[e];
                        if (epi) v = finish(v, i, it, e);
                        *c = v;
                    } else {
                        uint16_t *c = reinterpret_cast<uint16_t *>(Cb) + off + e;
                        float v = p.beta != 0.0f ? __builtin_fmaf(p.beta, dec(*c), x[e]) : x[e];
                        if (epi) v = finish(v, i, it, e);
                        *c = enc(v);
                    }
                }
            }
        }
    }
}

// Waits until at most `n` stages of direct loads (each `per` instructions)
// remain in flight; s_waitcnt takes an immediate, so the few possible
// counts are enumerated.
template <int PER, int STAGES>
__device__ inline void wait_stages(int n) {
    if (STAGES > 3 && n >= 3) { wait_vmcnt<(STAGES > 3 ? 3 : 0) * PER>(); return; }
    if (STAGES > 2 && n >= 2) { wait_vmcnt<(STAGES > 2 ? 2 : 0) * PER>(); return; }
    if (n >= 1) { wait_vmcnt<PER>(); return; }
    wait_vmcnt<0>();
}

// Scheduling hint for one k step: alternate one matrix instruction with one
// LDS read (the next step's fragments), then the remaining matrix
// instructions, so the reads' latency hides under the matrix work instead
// of being issued in a burst right before it is needed.
template <int NREAD, int NMFMA>
__device__ inline void interleave_reads() {
    // two reads after each of the first matrix instructions, so every read
    // is issued in the first half of the step
    constexpr int PAIRS = (NREAD + 1) / 2 < NMFMA ? (NREAD + 1) / 2 : NMFMA;
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
    }
    if (NMFMA > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - PAIRS, 0);
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
