// The direct-load GEMM of narrow floats on the CDNA4 matrix cores, for
// operands stored K-contiguous (row-major A, column-major B): 8-bit floats
// (E4M3, E5M2) with no scaling, and the block-scaled formats (MXFP8 with
// E4M3/E5M2 elements, MXFP6 with E2M3/E3M2, MXFP4 with E2M1), in which each
// 32 consecutive elements of a row share one E8M0 scale ("CUDA GEMM 矩阵乘法
// 优化指南", blog.zhenwei.site, section 13.2, FP8 and the block-scale
// quantisation of FP4/FP6).  Output in fp32, bf16 or fp16.
//
// Matrix instruction: v_mfma_scale_f32_32x32x64_f8f6f4, 64 k per instruction.
// A lane's fragment of a 32 x 64 block is 32 k of one row (row lane % 32):
// for 6- and 4-bit elements (24 or 16 bytes) the consecutive k of block
// lane / 32, for 8-bit ones 16 k of each block (see frag8); the lane's
// scale operand is the E8M0 byte of block lane / 32 (a constant 2^0 without
// scaling).  The
// operands are swapped (C^T = B^T A^T) as in the 16-bit kernels, so a lane's
// accumulators hold consecutive columns of C.
//
// The pipeline is the 16-bit direct-load one of dma_tile.hpp (256 x 256 block
// tile, 2 x 4 waves, a ring of LDS stages: two, or four for 4-bit elements)
// run on the bytes viewed as 16-bit pairs.  A stage is 128 k of every format:
// a K-contiguous panel row of 128 bytes for 8-bit elements, 64 bytes for
// 4-bit ones, and for 6-bit ones 128 bytes loaded of which the first 96 are
// that stage's (the stage advances 96 bytes along the row; the rest is
// loaded again as the next stage's start).  With scales, every stage's load
// group also carries one 4-byte direct load per lane that fetches 16 bytes
// (four stages' worth) of the scales of 16 panel rows into a ring of scale
// groups two groups ahead (f8_tile_steps).
#pragma once

#include <type_traits>

#include "dma_streamk.hpp"

namespace libgemm {
namespace {

using namespace dmatile;

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Operand format codes of the scaled matrix instruction.
constexpr int FMT_E4M3 = 0, FMT_E5M2 = 1, FMT_E2M3 = 2, FMT_E3M2 = 3, FMT_E2M1 = 4;

template <int F>
struct Fmt {
    static constexpr int WIDTH = F == FMT_E2M1 ? 4 : (F == FMT_E2M3 || F == FMT_E3M2) ? 6 : 8;
    static constexpr int ROWB = WIDTH == 4 ? 64 : 128;  // LDS bytes per panel row per stage
    static constexpr int STEPB = 128 * WIDTH / 8;       // bytes of a row per stage (128 k)
};

// Kernel arguments.  d carries C, the scalars, the epilogue, the tile grid,
// and the leading dimensions and batch strides of A and B in 16-bit units.
struct F8Args {
    DmaArgs d;
    int64_t K;                // k extent (elements); a multiple of 16 bytes per row
    int64_t ka, kb;           // row extents along K of A and B, in 16-bit units
    const uint8_t *sa, *sb;   // E8M0 scales: A(i, k) has sa[i*ldsa + k/32]; B(k, j) sb[j*ldsb + k/32]
    int64_t ldsa, ldsb;       // bytes, multiples of 4
    int64_t ssa, ssb;         // batch strides of the scales, bytes
};

// The 32-byte fragment of row row0 + lane % 32 for k step kk (64 k) of a
// K-contiguous panel with 8 chunks of 16 bytes per row, swizzled by
// swz_k<8>.  With 8-bit elements the instruction takes the low 16 bytes of
// every lane as k of the first 32-k block and the high 16 as k of the
// second (measured on gfx950: a one-hot A at each k under two block scales),
// so lane half h reads 16-k chunk 4kk + h (block 2kk) and chunk 4kk + 2 + h
// (block 2kk + 1), and its scale byte is that of block 2kk + h for the
// instruction's own pairing of lanes with blocks.  row0 is a multiple of
// 32, so the row's swizzle is that of lane % 32 with bit 2 flipped when bit
// 5 of row0 is set; written this way the per-lane part of every fragment
// address is one of eight values shared by all rows of both panels, and the
// row enters as a constant or wave-uniform offset.
__device__ inline i32x8 frag8(const LDS char *panel, int row0, int kk, int lane) {
    const int l = lane & 31;
    const int s = swz_k<8>(l) ^ ((row0 >> 3) & 7);
    const int c = kk * 4 + (lane >> 5);
    const LDS char *r = panel + row0 * 128 + l * 128;
    const u32x4 lo = *reinterpret_cast<const LDS u32x4 *>(r + ((c ^ s) << 4));
    const u32x4 hi = *reinterpret_cast<const LDS u32x4 *>(r + (((c + 2) ^ s) << 4));
    return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                 int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
}

// 6-bit elements: the lane's 24 bytes start at byte 24*(2kk + lane/32) of a
// 128-byte panel row; read as three 8-byte words, each inside one chunk.
__device__ inline i32x8 frag6(const LDS char *panel, int row0, int kk, int lane) {
    const int row = row0 + (lane & 31);
    const int s = swz_k<8>(row);
    const int o0 = 24 * (2 * kk + (lane >> 5));
    const LDS char *r = panel + row * 128;
    i32x8 out = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        const int o = o0 + 8 * w;
        const u32x2 v = *reinterpret_cast<const LDS u32x2 *>(r + (((o >> 4) ^ s) << 4) + (o & 8));
        out[2 * w] = int(v[0]);
        out[2 * w + 1] = int(v[1]);
    }
    return out;
}

// 4-bit elements: the lane's 16 bytes are chunk 2kk + lane/32 of a 64-byte
// panel row swizzled by swz_k<4>.
__device__ inline i32x8 frag4(const LDS char *panel, int row0, int kk, int lane) {
    const int row = row0 + (lane & 31);
    const int c = 2 * kk + (lane >> 5);
    const u32x4 v = *reinterpret_cast<const LDS u32x4 *>(panel + row * 64 + ((c ^ swz_k<4>(row)) << 4));
    return i32x8{int(v[0]), int(v[1]), int(v[2]), int(v[3]), 0, 0, 0, 0};
}

template <int F>
__device__ inline i32x8 frag(const LDS char *panel, int row0, int kk, int lane) {
    if (Fmt<F>::WIDTH == 8) return frag8(panel, row0, kk, lane);
    if (Fmt<F>::WIDTH == 6) return frag6(panel, row0, kk, lane);
    return frag4(panel, row0, kk, lane);
}

// acc + (B^T block) (A^T block) for k step KK of a stage: the first operand
// is B's fragment in B's format.  Scale operands: byte 2*KK of sb and sa
// (each lane's word holds the stage's block 2*kk + lane/32 in byte 2*kk).
template <int FA, int FB, int KK>
__device__ inline f32x16 mma8(i32x8 b, i32x8 a, f32x16 c, int sb, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FB, FA, 2 * KK, sb, 2 * KK, sa);
}

// 0x7F in every byte: E8M0 2^0 whichever byte the instruction selects.
constexpr int UNIT_SCALE = 0x7F7F7F7F;

// Schedule of one row of a wave tile: one matrix instruction, the NREAD LDS
// reads issued with it, the row's other instructions; then a scheduling
// barrier, so that the compiler keeps the rows in program order instead of
// hoisting every read of a stage to its top (which would need all the
// fragments live at once) and sinking the matrix instructions past the
// workgroup barrier.
template <int NREAD, int FN>
__device__ inline void hint_row() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, FN - 1, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// An empty volatile statement that takes x as an operand in the given
// register file: the instruction that produced x cannot move past it.
template <bool AGPR>
__device__ inline void pin(const f32x16 &x) {
    if (!AGPR) asm volatile("" ::"v"(x));
}

using dma::direct_load4;

#ifndef LIBGEMM_F8_WM
#define LIBGEMM_F8_WM 2
#endif
#ifndef LIBGEMM_F8_WN
#define LIBGEMM_F8_WN 4
#endif
#ifndef LIBGEMM_F8_STAGES
#define LIBGEMM_F8_STAGES 2
#endif
// 4-bit elements: a stage is 34 KiB (two 16 KiB panels and the scales), so
// four fit, and the epilogue stages C across two of them
#ifndef LIBGEMM_MX4_STAGES
#define LIBGEMM_MX4_STAGES 4
#endif
#ifndef LIBGEMM_F8_GROUP_M
#define LIBGEMM_F8_GROUP_M 16
#endif

constexpr int F8_BM = 256, F8_BN = 256;

// Stage buffers in the ring for formats FA, FB.
template <int FA, int FB>
constexpr int f8_stages() {
    return Fmt<FA>::WIDTH == 4 && Fmt<FB>::WIDTH == 4 ? LIBGEMM_MX4_STAGES : LIBGEMM_F8_STAGES;
}

// The sizes of the kernel's tiles, panels and stages for formats FA, FB.
template <int FA, int FB, int WAVES_M, int WAVES_N, bool MX>
struct F8Tile {
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int WTM = F8_BM / WAVES_M, WTN = F8_BN / WAVES_N;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    // Accumulators beyond 128 registers per lane live in the AGPRs (one
    // wave per SIMD); the statement that pins the instructions in place
    // must name the register file they are in.
    static constexpr bool ACC_AGPR = FM * FN * 16 > 128;
    using OpA = Operand<true, WAVES, Fmt<FA>::ROWB / 2, Fmt<FA>::STEPB / 2>;
    using OpB = Operand<true, WAVES, Fmt<FB>::ROWB / 2, Fmt<FB>::STEPB / 2>;
    static constexpr int PANEL_A = OpA::PANEL, PANEL_B = OpB::PANEL;
    static constexpr int DATA = PANEL_A + PANEL_B;
    // MX: a ring of three scale groups after the stage ring; a group holds
    // the scale words of four stages (16 bytes per panel row, A's 256 rows
    // then B's), so one 16-row x 16-byte load fetches four stages' worth of
    // 16 rows from 16 cache lines, where per-stage loads would touch a line
    // per row every stage
    static constexpr int SGROUP = 16 * (F8_BM + F8_BN);
    static constexpr int SRING = MX ? 3 * SGROUP : 0;
    static constexpr int EPI = WAVES * 32 * WTN * 4;              // epilogue staging
    // A stage buffer holds one stage's data; C is staged across the NEED
    // consecutive buffers the epilogue takes (f8_tile_store).
    static constexpr int STAGE = DATA;
    static constexpr int NEED = (EPI + STAGE - 1) / STAGE;
    static constexpr int PER_DATA = OpA::PER_WAVE + OpB::PER_WAVE;
    static constexpr int PER_STAGE = PER_DATA + (MX ? 1 : 0);  // direct loads per wave per stage
    static_assert(FM % 2 == 0, "A fragments alternate between two slots");
    static_assert(!MX || WAVES == 8, "scale loads: four waves per operand, 64 rows each");
    static_assert(PER_DATA % FN == 0, "refill split over the last row's instructions");
};

// 2 x 4 waves, each with a 128 x 64 wave tile (4 x 2 accumulator blocks,
// 128 registers); a stage is 128 k, two 64-k steps.  A lane's fragments are
// twice the size of the 16-bit kernel's, so double-buffering all of them
// would not fit beside the accumulators in the 256 registers a wave has at
// two waves per SIMD.  Instead B's two fragments are double-buffered by k
// step and A's four rotate through two slots: the instructions of row i (two
// of them) run while row i + 1's fragment is read, and the last row's run
// while the next k step's fragments are read.  At the end of a stage those
// reads target the next stage's buffer, so they follow the wait for that
// stage and the workgroup barrier; the refill of the stage just consumed is
// issued between the last two instructions, after the barrier has shown
// that every wave has read it.  With scales (MX), each lane reads its six
// fragments' scale words for the next stage from the scale ring right after
// the barrier, into registers that take over once the current stage's last
// row is done.
//
// f8_tile_steps runs stages [kb, ke) of one tile (128 k each, numbered from
// the start of K) into acc and returns the ring buffer that held the last
// one; the buffer after it is then free for the epilogue's staging.
template <int FA, int FB, int WAVES_M, int WAVES_N, int STAGES, bool MX>
__device__ __forceinline__ int f8_tile_steps(
    const F8Args &p, LDS char *lds, const TileCoord &t, int64_t kb, int64_t ke,
    f32x16 (&acc)[F8_BM / WAVES_M / 32][F8_BN / WAVES_N / 32]) {
    using L = F8Tile<FA, FB, WAVES_M, WAVES_N, MX>;
    constexpr int FM = L::FM, FN = L::FN, WTM = L::WTM, WTN = L::WTN;
    constexpr bool ACC_AGPR = L::ACC_AGPR;
    using OpA = typename L::OpA;
    using OpB = typename L::OpB;
    constexpr int PANEL_A = L::PANEL_A, PANEL_B = L::PANEL_B, STAGE = L::STAGE;
    constexpr int SGROUP = L::SGROUP;
    constexpr int PER_DATA = L::PER_DATA, PER_STAGE = L::PER_STAGE;

    const DmaArgs &d = p.d;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int64_t m0 = t.tm * F8_BM, n0 = t.tn * F8_BN;

    OpA opa;
    OpB opb;
    opa.init(d.A + t.batch * d.sA, d.lda, d.M, m0, (d.M - 1) * d.lda + p.ka, wave, lane);
    opb.init(d.B + t.batch * d.sB, d.ldb, d.N, n0, (d.N - 1) * d.ldb + p.kb, wave, lane);

    // MX: scale group g (stages 4g .. 4g+3, scale bytes 16g .. 16g+15 of a
    // row) sits in ring slot g % 3.  Load (g, part) is one 4-byte direct load
    // per lane by wave w of part 8*part + w of the group's 32: 16 panel rows
    // (A's when part < 2, else B's) of 16 bytes, lane l taking row l/4.  Word
    // v of panel row r holds the row's scale word v ^ ((r / 8) % 4), so that
    // the 32 rows one scale read touches fall in distinct banks.  Rows past
    // the matrix read zeros; words past a row's scales are read but used only
    // by stages past K.
    u32x4 srs_a = {0u, 0u, 0u, 0u}, srs_b = {0u, 0u, 0u, 0u};
    uint32_t sv[4] = {OOB, OOB, OOB, OOB};  // this lane's row offset for each part
    if (MX) {
        // panel row 128*(part & 1) + sl (plus 256 for B): (row / 8) % 4 is
        // (2*wave + lane/32) % 4
        const int sl = (lane >> 2) + 16 * wave, sd = 4 * ((lane & 3) ^ ((2 * wave + (lane >> 5)) & 3));
        srs_a = dma::raw_buffer(
            static_cast<uint64_t>(uniform(reinterpret_cast<int64_t>(p.sa + t.batch * p.ssa))),
            static_cast<uint32_t>(uniform(d.M * p.ldsa)));
        srs_b = dma::raw_buffer(
            static_cast<uint64_t>(uniform(reinterpret_cast<int64_t>(p.sb + t.batch * p.ssb))),
            static_cast<uint32_t>(uniform(d.N * p.ldsb)));
#pragma unroll
        for (int part = 0; part < 4; ++part) {
            const bool on_a = part < 2;
            const int64_t r = (on_a ? m0 : n0) + 128 * (part & 1) + sl;
            const int64_t R = on_a ? d.M : d.N;
            sv[part] = r < R ? static_cast<uint32_t>(r * (on_a ? p.ldsa : p.ldsb) + sd) : OOB;
        }
    }
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    const uint32_t sring = lds_base + STAGES * STAGE;
    auto load_scales = [&](int64_t g, int part) {
        if (!MX) return;
        const uint32_t dst =
            sring + static_cast<uint32_t>(g % 3) * SGROUP + static_cast<uint32_t>(8 * part + wave) * 256;
        direct_load4(part < 2 ? srs_a : srs_b, dst,
                     sv[part] == OOB ? OOB : sv[part] + static_cast<uint32_t>(16 * g));
    };
    const int64_t steps = ke - kb;

    // MX prologue: groups g0 and g0 + 1 whole, and the parts of g0 + 2 the
    // prologue stages do not carry (each stage's load group carries one
    // scale load, so the count per stage stays uniform); older than every
    // stage, so the first stage's wait covers them.
    const int64_t g0 = kb >> 2;
    if (MX) {
#pragma unroll
        for (int part = 0; part < 4; ++part) {
            load_scales(g0, part);
            load_scales(g0 + 1, part);
        }
#pragma unroll
        for (int part = STAGES; part < 4; ++part) load_scales(g0 + 2, part);
    }
#pragma unroll
    for (int st = 0; st < STAGES; ++st) {
        if (st < steps) {
            opa.issue(lds + st * STAGE, kb + st, p.ka, wave);
            opb.issue(lds + st * STAGE + PANEL_A, kb + st, p.kb, wave);
            if (st < 4) load_scales(g0 + 2, st);
        }
    }
    wait_stages<PER_STAGE, STAGES>(int(steps - 1 < STAGES - 1 ? steps - 1 : STAGES - 1));
    __syncthreads();

    i32x8 fb[2][FN], fa[2];
    auto read_b = [&](int buf, int kk, int slot) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[slot][j] = frag<FB>(lds + buf * STAGE + PANEL_A, wn * WTN + j * 32, kk, lane);
    };
    auto read_a = [&](int buf, int kk, int i) {
        fa[i & 1] = frag<FA>(lds + buf * STAGE, wm * WTM + i * 32, kk, lane);
    };
    // the scale words of the stage in `buf`: fragment rows' four bytes,
    // shifted so that k step kk's block (2kk + lane/32) sits in byte 2kk
    int sa[FM], sb[FN], nsa[FM], nsb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) sa[i] = nsa[i] = UNIT_SCALE;
#pragma unroll
    for (int j = 0; j < FN; ++j) sb[j] = nsb[j] = UNIT_SCALE;
    // the scale words of absolute stage a, from its group's ring slot
    auto read_scales = [&](int64_t a) {
        if (!MX) return;
        const LDS uint32_t *s = reinterpret_cast<const LDS uint32_t *>(
            lds + STAGES * STAGE + static_cast<int>((a >> 2) % 3) * SGROUP);
        // the rows are 32-aligned blocks plus lane % 32, so (row / 8) % 4 is
        // (lane / 8) % 4
        const int w = static_cast<int>(a & 3) ^ ((lane >> 3) & 3);
        const int sh = 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i) nsa[i] = int(s[4 * (wm * WTM + i * 32 + (lane & 31)) + w] >> sh);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            nsb[j] = int(s[4 * (F8_BM + wn * WTN + j * 32 + (lane & 31)) + w] >> sh);
    };
    auto take_scales = [&]() {
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = nsa[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) sb[j] = nsb[j];
    };
    // The empty volatile statement takes the results as operands, so the
    // instructions stay where they are written: the compiler otherwise sinks
    // them to the end of the loop body, past the workgroup barrier, and then
    // has to keep every fragment of the stage live.
    auto row = [&](int i, auto kk) {
        constexpr int KK = decltype(kk)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            acc[i][j] = mma8<FA, FB, KK>(fb[KK][j], fa[i & 1], acc[i][j], sb[j], sa[i]);
            pin<ACC_AGPR>(acc[i][j]);
        }
    };
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    // k step 0 of a stage in buffer `buf` (B fragments in slot 0); its last
    // row reads k step 1's fragments from the same buffer.
    auto first_step = [&](int buf) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if (i + 1 < FM) {
                read_a(buf, 0, i + 1);
            } else {
                read_b(buf, 1, 1);
                read_a(buf, 1, 0);
            }
            row(i, K0{});
            if (i + 1 < FM) hint_row<2, FN>();
            else hint_row<2 * FN + 2, FN>();
        }
    };

    read_b(0, 0, 0);
    read_a(0, 0, 0);
    read_scales(kb);
    take_scales();
    int buf = 0;
    const int64_t main_steps = steps - 1;
    for (int64_t s = 0; s < main_steps; ++s) {
        first_step(buf);
        // k step 1: rows 0 .. FM-2 read the next row from this buffer
#pragma unroll
        for (int i = 0; i + 1 < FM; ++i) {
            read_a(buf, 1, i + 1);
            row(i, K1{});
            hint_row<2, FN>();
        }
        const int64_t later = steps - 2 - s;
        wait_stages<PER_STAGE, STAGES>(int(later < STAGES - 2 ? later : STAGES - 2));
        wait_lgkmcnt0();
        __syncthreads();
        const int nbuf = buf + 1 == STAGES ? 0 : buf + 1;
        read_b(nbuf, 0, 0);
        read_a(nbuf, 0, 0);
        read_scales(kb + s + 1);
        const int64_t refill = s + STAGES;  // within the range
        const bool do_refill = refill < steps;
        const u32x4 ra = opa.rsrc(kb + refill), rb = opb.rsrc(kb + refill);
        const uint32_t la = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds + buf * STAGE));
        const int64_t kla = p.ka - (kb + refill) * (Fmt<FA>::STEPB / 2);
        const int64_t klb = p.kb - (kb + refill) * (Fmt<FB>::STEPB / 2);
        // the last row, with the refill of this buffer split around its
        // instructions
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            acc[FM - 1][j] = mma8<FA, FB, 1>(fb[1][j], fa[(FM - 1) & 1], acc[FM - 1][j], sb[j], sa[FM - 1]);
            pin<ACC_AGPR>(acc[FM - 1][j]);
            if (do_refill) {
#pragma unroll
                for (int q = j * PER_DATA / FN; q < (j + 1) * PER_DATA / FN; ++q) {
                    if (q < OpA::PER_WAVE) opa.load(ra, la, q, kla, wave);
                    else opb.load(rb, la + PANEL_A, q - OpA::PER_WAVE, klb, wave);
                }
                // two groups ahead of the stage that issues it, part a % 4
                if (j == 0) load_scales(((kb + s) >> 2) + 2, static_cast<int>((kb + s) & 3));
            }
        }
        take_scales();
        buf = nbuf;
    }
    // The last stage.  When it is the last of K and holds only 64 k (K = 64
    // mod 128), its second k step reads zeros from both panels; its scales
    // come from bytes past the last scale block, so they are replaced by 2^0
    // (a NaN pattern there would turn the zero products into NaN).
    first_step(buf);
    if (MX && ke * 128 > p.K) {
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = UNIT_SCALE;
#pragma unroll
        for (int j = 0; j < FN; ++j) sb[j] = UNIT_SCALE;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if (i + 1 < FM) read_a(buf, 1, i + 1);
        row(i, K1{});
        if (i + 1 < FM) hint_row<2, FN>();
    }
    return buf;
}

// The epilogue of a whole tile: C is staged in ring buffers the last stage
// (in `buf`) does not use: every wave finished reading them before the last
// barrier and no load targets them any more.  Staging takes NEED
// consecutive buffers: the next one when one suffices, else the first NEED
// or the NEED after them, whichever excludes the last stage's.
template <int FA, int FB, int OUT, int WAVES_M, int WAVES_N, int STAGES, bool MX>
__device__ __forceinline__ void f8_tile_store(
    const F8Args &p, LDS char *lds, const TileCoord &t, int buf,
    const f32x16 (&acc)[F8_BM / WAVES_M / 32][F8_BN / WAVES_N / 32]) {
    using L = F8Tile<FA, FB, WAVES_M, WAVES_N, MX>;
    constexpr int NEED = L::NEED;
    static_assert(NEED == 1 || 2 * NEED <= STAGES, "epilogue staging fits beside the last stage");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int free0 = NEED == 1 ? (buf + 1 == STAGES ? 0 : buf + 1) : (buf >= NEED ? 0 : NEED);
    LDS char *stage_free = lds + free0 * L::STAGE;
    store_tile_lds<OUT, L::FM, L::FN>(p.d, acc, t.batch, t.tm * F8_BM + wm * L::WTM,
                                      t.tn * F8_BN + wn * L::WTN, lane,
                                      reinterpret_cast<LDS float *>(stage_free) + wave * 32 * L::WTN);
}

// One workgroup per tile.
template <int FA, int FB, int OUT, int WAVES_M, int WAVES_N, int STAGES, bool MX>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, 1) void f8gemm_dma_kernel(F8Args p) {
    using L = F8Tile<FA, FB, WAVES_M, WAVES_N, MX>;
    static_assert(STAGES >= 2 && STAGES * L::STAGE + L::SRING <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * L::STAGE + L::SRING];
    LDS char *lds = (LDS char *)smem;
    TileCoord t = tile_of(p.d.grid, blockIdx.x);
    t.batch = uniform(t.batch);
    t.tm = uniform(t.tm);
    t.tn = uniform(t.tn);
    f32x16 acc[L::FM][L::FN];
#pragma unroll
    for (int i = 0; i < L::FM; ++i)
#pragma unroll
        for (int j = 0; j < L::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int buf = f8_tile_steps<FA, FB, WAVES_M, WAVES_N, STAGES, MX>(p, lds, t, 0,
                                                                        (p.K + 127) / 128, acc);
    f8_tile_store<FA, FB, OUT, WAVES_M, WAVES_N, STAGES, MX>(p, lds, t, buf, acc);
}

// The stream-K schedule of dma_streamk.hpp over the same tiles (a k step is
// one 128-k stage): G workgroups, one per compute unit, each computing its
// whole tiles and then its range of the cut tiles' k steps; a piece that
// covers a whole tile goes through the epilogue, any other to its slot in
// the workspace for dma_streamk_fixup.
template <int FA, int FB, int OUT, int WAVES_M, int WAVES_N, int STAGES, bool MX>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, 1) void f8gemm_dma_streamk_kernel(F8Args p,
                                                                                   DmaStreamK sk) {
    using L = F8Tile<FA, FB, WAVES_M, WAVES_N, MX>;
    static_assert(STAGES >= 2 && STAGES * L::STAGE + L::SRING <= 160 * 1024, "LDS budget");
    static_assert(L::FM * L::FN * 4 * L::WAVES * 64 * 16 == SK_SLOT * 4, "a slot holds one tile");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * L::STAGE + L::SRING];
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
        TileCoord t = tile_of(p.d.grid, tile);
        t.batch = uniform(t.batch);
        t.tm = uniform(t.tm);
        t.tn = uniform(t.tn);
        // every wave is done with the previous piece's buffers (its last
        // fragment reads and epilogue staging) before the ring is refilled
        if (item > 0) __syncthreads();
        f32x16 acc[L::FM][L::FN];
#pragma unroll
        for (int i = 0; i < L::FM; ++i)
#pragma unroll
            for (int j = 0; j < L::FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        const int buf = f8_tile_steps<FA, FB, WAVES_M, WAVES_N, STAGES, MX>(p, lds, t, kb, ke, acc);
        if (kb == 0 && ke == S)
            f8_tile_store<FA, FB, OUT, WAVES_M, WAVES_N, STAGES, MX>(p, lds, t, buf, acc);
        else
            store_partial<L::FM, L::FN, L::WAVES * 64>(sk, sk_slot(sk, w, local, end), acc);
    }
}

// ---- host side of the stream-K schedule (8-bit and MX launches)

// Step time over partial-tile time for streamk_groups, and the cost of the
// partial-tile exchange in k steps of one tile: about 0.14 per partial tile
// written and read back and 2 for the fix-up launch.  These are the 16-bit
// direct-load kernel's measured figures: its tiles are the same and a
// 128-k stage of 8-bit operands, twice its 64-k step's bytes at twice the
// instruction rate, takes about as long.
#ifndef LIBGEMM_F8_SK_RATIO
#define LIBGEMM_F8_SK_RATIO 14
#endif
constexpr double F8_SK_STEPS_PER_PIECE = 0.14;
constexpr double F8_SK_FIXED_STEPS = 2.0;

inline int64_t f8_tiles(int64_t M, int64_t N, int64_t batch) {
    return ((M + F8_BM - 1) / F8_BM) * ((N + F8_BN - 1) / F8_BN) * batch;
}

// The split of `tiles` tiles of K elements (128-k steps) over one workgroup
// per compute unit of MI355X (on a part with fewer units the schedule is
// still correct, the workgroups just do not all run at once).
inline StreamKSplit f8_streamk_split(int64_t tiles, int64_t K) {
    return streamk_split(tiles, (K + 127) / 128, HGEMM_STREAMK_MAX_GRID, LIBGEMM_F8_SK_RATIO);
}

// Some tiles are left over after the whole waves, and (unless forced) the k
// steps the cut last wave saves exceed the exchange: the last wave takes
// ceil(T_r * S / Gs) steps per workgroup instead of S, and the exchange grows
// with the pieces, about Gs + T_r partial tiles.
inline bool f8_streamk_worth(int64_t tiles, int64_t K, bool force) {
    const int64_t steps = (K + 127) / 128;
    const int64_t g = HGEMM_STREAMK_MAX_GRID;
    const int64_t cut = tiles % g;
    if (cut == 0 || tiles >= (int64_t(1) << 24) || steps >= (int64_t(1) << 24)) return false;
    if (force) return true;
    const int64_t gs = streamk_groups(g, cut, steps, LIBGEMM_F8_SK_RATIO);
    const int64_t tail = (cut * steps + gs - 1) / gs;
    return double(steps - tail) > F8_SK_STEPS_PER_PIECE * double(gs + cut) + F8_SK_FIXED_STEPS;
}

}  // namespace
}  // namespace libgemm
