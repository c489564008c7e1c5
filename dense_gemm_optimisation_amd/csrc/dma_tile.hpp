// Pieces of the direct-load matrix-core pipeline shared by the 16-bit and
// 8-bit fast-path kernels: the kernel arguments, the operand panels that
// direct global -> LDS loads fill and the fragments read back from them,
// the epilogue through LDS, and the wait / scheduling helpers.
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
#pragma once

#include "gemm_problem.hpp"
#include "lds_dma.hpp"
#include "tile_schedule.hpp"

namespace libgemm {
namespace dmatile {

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
// 16-byte chunks of C at element alignment only: a row of C starts wherever
// ldc puts it, and the memory system takes a 16-byte access at any
// element-aligned address (it splits one that straddles a cache line).
typedef float f32x4_ea __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4_ea __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x2_b1 __attribute__((ext_vector_type(2), aligned(1)));

constexpr int BM = 256, BN = 256;       // block tile (rows of A and columns of B)
constexpr int OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2;
constexpr int OUT_F8 = 3;  // E4M3 or E5M2 (Epilogue::out_e5m2), scaled and saturated

struct DmaArgs {
    int64_t M, N, K;
    float alpha, beta;
    const uint16_t *A;
    const uint16_t *B;
    void *C;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;
    TileGrid grid;
    Epilogue epi;
    int64_t span_a, span_b;  // elements of one slice of A and of B the loads may touch
};

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
// where each lane fetches from, and how the wave reads fragments back.  A
// K-contiguous panel's stage advances STEP 16-bit units along the rows
// (BK unless a stage uses only the first STEP of the BK it loads).
template <bool KMAJOR, int WAVES, int BK, int STEP = BK>
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
        step = KMAJOR ? int64_t(STEP) * 2 : int64_t(BK) * ld * 2;
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
    // rs and kleft = K - stage*STEP valid k values, into the panel at lds0.
    __device__ void load(u32x4 rs, uint32_t lds0, int i, int64_t kleft, int wave) const {
        const uint32_t v = (kleft < BK && kl[i] >= kleft) ? OOB : voff[i];
        direct_load16(rs, lds0 + (wave * PER_WAVE + i) * 1024, v);
    }

    // All direct loads of stage `stage` (k from stage*BK) into the panel at dst.
    __device__ void issue(LDS char *dst, int64_t stage, int64_t K, int wave) const {
        const u32x4 rs = rsrc(stage);
        const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) load(rs, lds0, i, K - stage * STEP, wave);
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
// the same way when beta != 0, at any element alignment of C's rows.  Rows
// or columns outside C are skipped, and the chunk that crosses the right
// edge of C is stored element by element.
template <int OUT, int FM, int FN>
__device__ inline void store_tile_lds(const DmaArgs &p, const f32x16 (&acc)[FM][FN], int64_t batch,
                                      int64_t mw, int64_t nw, int lane, LDS float *scratch) {
    constexpr int W = FN * 32;          // strip width (columns)
    constexpr int PITCH = W;            // floats per staged row
    constexpr int SWZ = W / 4 - 1 < 15 ? W / 4 - 1 : 15;
    auto at = [&](int r, int col) {     // staged float (r, col), col a multiple of 4
        return scratch + r * PITCH + ((((col >> 2) ^ (r & SWZ))) << 2);
    };
    constexpr int ESZ = OUT == OUT_F32 ? 4 : OUT == OUT_F8 ? 1 : 2;  // bytes per element of C
    // output elements per store: 16 bytes, or 8 for 8-bit outputs (whose
    // 16-element chunks need more registers than the accumulators leave)
    constexpr int CW = OUT == OUT_F8 ? 8 : 16 / ESZ;
    constexpr int CPR = W / CW;         // chunks per row
    constexpr int RPI = 64 / CPR;       // rows per store instruction
    static_assert(CPR >= 1 && 32 % RPI == 0, "strip shape");
    char *Cb = static_cast<char *>(p.C) + batch * p.sC * ESZ;
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
            if constexpr (OUT == OUT_F8) {
                // quantised: C is not read (beta is 0 for these outputs)
                uint8_t *c = reinterpret_cast<uint8_t *>(Cb) + off;
                u32x2_b1 w;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    w[h] = epilogue_f8x2(p.epi, finish(x[4 * h], i, it, 4 * h),
                                         finish(x[4 * h + 1], i, it, 4 * h + 1)) |
                           (epilogue_f8x2(p.epi, finish(x[4 * h + 2], i, it, 4 * h + 2),
                                          finish(x[4 * h + 3], i, it, 4 * h + 3)) << 16);
                if (n + CW <= p.N) {
                    *reinterpret_cast<u32x2_b1 *>(c) = w;
                } else {
                    const int nvalid = int(p.N - n);
#pragma unroll
                    for (int e = 0; e < CW; ++e)
                        if (e < nvalid) c[e] = uint8_t(w[e / 4] >> (8 * (e % 4)));
                }
            } else {
                if (n + CW <= p.N) {
                    if (OUT == OUT_F32) {
                        float *c = reinterpret_cast<float *>(Cb) + off;
                        f32x4 v = {x[0], x[1], x[2], x[3]};
                        if (p.beta != 0.0f) {
                            const f32x4 o = *reinterpret_cast<const f32x4_ea *>(c);
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(p.beta, o[e], v[e]);
                        }
                        if (epi)
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = finish(v[e], i, it, e);
                        *reinterpret_cast<f32x4_ea *>(c) = v;
                    } else {
                        uint16_t *c = reinterpret_cast<uint16_t *>(Cb) + off;
                        if (p.beta != 0.0f) {
                            const u32x4 o = *reinterpret_cast<const u32x4_ea *>(c);
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
                        *reinterpret_cast<u32x4_ea *>(c) = w;
                    }
                } else {
                    // element by element (a loop that keeps this rare path
                    // small: unrolled, it pushes the accumulators into scratch)
                    const int nvalid = int(p.N - n);
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

}  // namespace dmatile
}  // namespace libgemm
