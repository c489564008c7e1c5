// 8-bit float GEMM on the CDNA4 matrix cores: OCP E4M3 or E5M2 operands
// (each operand in its own format), exact products, fp32 accumulation, output
// in fp32, bf16 or fp16.  The pages name the 8-bit formats E4M3 and E5M2 as
// the next step down from fp16/bf16 for matrix units ("CUDA GEMM 矩阵乘法优化
// 指南", blog.zhenwei.site, section 13.2).
//
// Matrix instruction: v_mfma_scale_f32_32x32x64_f8f6f4 with both block
// scales 2^0, 64 k per instruction.  A lane's fragment of a 32 x 64 block is
// 32 bytes of one row (row lane % 32), read from a K-contiguous LDS panel as
// two 16-byte reads at logical chunks 4*kk + 2*(lane / 32) and the one after.
// Any assignment of the 64 k values to (lane half, byte) positions yields
// the same dot products as long as A's and B's fragments use the same one,
// which they do here.  The operands are swapped (C^T = B^T A^T) as in the
// 16-bit kernels, so a lane's accumulators hold consecutive columns of C.
//
// Two kernels:
//   * fast path, operands stored K-contiguous (row-major A, column-major B:
//     the "TN" layout 8-bit GEMMs are normally run in) with 16-byte aligned
//     rows and K a multiple of 16.  It is the 16-bit direct-load pipeline of
//     dma_tile.hpp (256 x 256 block tile, 2 x 4 waves, two LDS stages) run on
//     the bytes viewed as 16-bit pairs: a stage of 64 pairs is 128 k, and the
//     K-contiguous panel layout, its swizzle and the direct loads are the
//     same byte for byte.  Only the fragment reads and the matrix
//     instruction differ;
//   * general kernel, any order, alignment and shape: 128 x 128 block tile,
//     2 x 2 waves, 128 k per stage, operands staged through registers into
//     the same K-contiguous LDS layout (an operand stored contiguous along M
//     or N is transposed by the byte writes into LDS), 16-byte loads where a
//     chunk lies inside the matrix and is aligned, single bytes elsewhere,
//     zeros outside the matrix.
#include "dma_tile.hpp"

namespace libgemm {
namespace {

using namespace dmatile;

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Operand format codes of the scaled matrix instruction.
constexpr int FMT_E4M3 = 0, FMT_E5M2 = 1;

// The 32-byte fragment of row row0 + lane % 32 for k step kk (64 k) of a
// K-contiguous panel with 8 chunks of 16 bytes per row, swizzled by
// swz_k<8>.  row0 is a multiple of 32, so the row's swizzle is that of
// lane % 32 with bit 2 flipped when bit 5 of row0 is set; written this way
// the per-lane part of every fragment address is one of eight values
// shared by all rows of both panels, and the row enters as a constant or
// wave-uniform offset.
template <int CH>
__device__ inline i32x8 frag8(const LDS char *panel, int row0, int kk, int lane) {
    static_assert(CH == 8, "128-byte panel rows");
    const int l = lane & 31;
    const int s = swz_k<8>(l) ^ ((row0 >> 3) & 7);
    const int c = kk * 4 + (lane >> 5) * 2;
    const LDS char *r = panel + row0 * 128 + l * 128;
    const u32x4 lo = *reinterpret_cast<const LDS u32x4 *>(r + ((c ^ s) << 4));
    const u32x4 hi = *reinterpret_cast<const LDS u32x4 *>(r + (((c + 1) ^ s) << 4));
    return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                 int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
}

// acc + (B^T block) (A^T block): the first operand is B's fragment in B's
// format.  Scale arguments: operand selector 0 and the E8M0 exponent 127,
// a factor of 1 on both sides.
template <int FA, int FB>
__device__ inline f32x16 mma8(i32x8 b, i32x8 a, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FB, FA, 0, 127, 0, 127);
}

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

#ifndef LIBGEMM_F8_WM
#define LIBGEMM_F8_WM 2
#endif
#ifndef LIBGEMM_F8_WN
#define LIBGEMM_F8_WN 4
#endif
#ifndef LIBGEMM_F8_STAGES
#define LIBGEMM_F8_STAGES 2
#endif
#ifndef LIBGEMM_F8_GROUP_M
#define LIBGEMM_F8_GROUP_M 16
#endif

// Fast-path kernel.  2 x 4 waves, each with a 128 x 64 wave tile (4 x 2
// accumulator blocks, 128 registers); a stage is 64 16-bit units (128 k),
// two 64-k steps.  A lane's fragments are twice the size of the 16-bit
// kernel's, so double-buffering all of them would not fit beside the
// accumulators in the 256 registers a wave has at two waves per SIMD.
// Instead B's two fragments are double-buffered by k step and A's four
// rotate through two slots: the instructions of row i (two of them) run
// while row i + 1's fragment is read, and the last row's run while the next
// k step's fragments are read.  At the end of a stage those reads target
// the next stage's buffer, so they follow the wait for that stage and the
// workgroup barrier; the refill of the stage just consumed is issued between
// the last two instructions, after the barrier has shown that every wave
// has read it.
template <int FA, int FB, int OUT, int WAVES_M, int WAVES_N, int STAGES>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, 1) void f8gemm_dma_kernel(DmaArgs p) {
    constexpr int WAVES = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N, FM = WTM / 32, FN = WTN / 32;
    constexpr int BK = 64;  // 16-bit units per stage
    // Accumulators beyond 128 registers per lane live in the AGPRs (one
    // wave per SIMD); the statement that pins the instructions in place
    // must name the register file they are in.
    constexpr bool ACC_AGPR = FM * FN * 16 > 128;
    static_assert(FM % 2 == 0, "A fragments alternate between two slots");
    using Op = Operand<true, WAVES, BK>;
    constexpr int CH = Op::CH;
    constexpr int PANEL = Op::PANEL;
    constexpr int STAGE = 2 * PANEL;
    constexpr int PER_STAGE = 2 * Op::PER_WAVE;  // direct loads per wave per stage
    static_assert(STAGES >= 2 && STAGES * STAGE <= 160 * 1024, "LDS budget");
    static_assert(PER_STAGE % FN == 0, "refill split over the last row's instructions");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

    TileCoord t = tile_of(p.grid, blockIdx.x);
    t.batch = uniform(t.batch);
    t.tm = uniform(t.tm);
    t.tn = uniform(t.tn);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;

    Op opa, opb;
    opa.init(p.A + t.batch * p.sA, p.lda, p.M, m0, (p.M - 1) * p.lda + p.K, wave, lane);
    opb.init(p.B + t.batch * p.sB, p.ldb, p.N, n0, (p.N - 1) * p.ldb + p.K, wave, lane);

    LDS char *lds = (LDS char *)smem;
    const int64_t steps = (p.K + BK - 1) / BK;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
    for (int st = 0; st < STAGES; ++st) {
        if (st < steps) {
            opa.issue(lds + st * STAGE, st, p.K, wave);
            opb.issue(lds + st * STAGE + PANEL, st, p.K, wave);
        }
    }
    wait_stages<PER_STAGE, STAGES>(int(steps - 1 < STAGES - 1 ? steps - 1 : STAGES - 1));
    __syncthreads();

    i32x8 fb[2][FN], fa[2];
    auto read_b = [&](int buf, int kk, int slot) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[slot][j] = frag8<CH>(lds + buf * STAGE + PANEL, wn * WTN + j * 32, kk, lane);
    };
    auto read_a = [&](int buf, int kk, int i) {
        fa[i & 1] = frag8<CH>(lds + buf * STAGE, wm * WTM + i * 32, kk, lane);
    };
    // The empty volatile statement takes the results as operands, so the
    // instructions stay where they are written: the compiler otherwise sinks
    // them to the end of the loop body, past the workgroup barrier, and then
    // has to keep every fragment of the stage live.
    auto row = [&](int i, int slot) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            acc[i][j] = mma8<FA, FB>(fb[slot][j], fa[i & 1], acc[i][j]);
            pin<ACC_AGPR>(acc[i][j]);
        }
    };
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
            row(i, 0);
            if (i + 1 < FM) hint_row<2, FN>();
            else hint_row<2 * FN + 2, FN>();
        }
    };

    read_b(0, 0, 0);
    read_a(0, 0, 0);
    int buf = 0;
    const int64_t main_steps = steps - 1;
    for (int64_t s = 0; s < main_steps; ++s) {
        first_step(buf);
        // k step 1: rows 0 .. FM-2 read the next row from this buffer
#pragma unroll
        for (int i = 0; i + 1 < FM; ++i) {
            read_a(buf, 1, i + 1);
            row(i, 1);
            hint_row<2, FN>();
        }
        const int64_t later = steps - 2 - s;
        wait_stages<PER_STAGE, STAGES>(int(later < STAGES - 2 ? later : STAGES - 2));
        wait_lgkmcnt0();
        __syncthreads();
        const int nbuf = buf + 1 == STAGES ? 0 : buf + 1;
        read_b(nbuf, 0, 0);
        read_a(nbuf, 0, 0);
        const int64_t refill = s + STAGES;
        const bool do_refill = refill < steps;
        const u32x4 ra = opa.rsrc(refill), rb = opb.rsrc(refill);
        const uint32_t la = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds + buf * STAGE));
        const int64_t kleft = p.K - refill * BK;
        // the last row, with the refill of this buffer split around its
        // second instruction
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            acc[FM - 1][j] = mma8<FA, FB>(fb[1][j], fa[(FM - 1) & 1], acc[FM - 1][j]);
            pin<ACC_AGPR>(acc[FM - 1][j]);
            if (do_refill) {
#pragma unroll
                for (int q = j * PER_STAGE / FN; q < (j + 1) * PER_STAGE / FN; ++q) {
                    if (q < Op::PER_WAVE) opa.load(ra, la, q, kleft, wave);
                    else opb.load(rb, la + PANEL, q - Op::PER_WAVE, kleft, wave);
                }
            }
        }
        buf = nbuf;
    }
    // The last stage.
    first_step(buf);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if (i + 1 < FM) read_a(buf, 1, i + 1);
        row(i, 1);
        if (i + 1 < FM) hint_row<2, FN>();
    }

    // C is staged in the buffer after the last stage's: every wave finished
    // reading it before the last barrier and no load targets it any more.
    static_assert(WAVES * 32 * WTN * 4 <= STAGE, "epilogue staging fits in one stage buffer");
    LDS char *stage_free = lds + (buf + 1 == STAGES ? 0 : buf + 1) * STAGE;
    store_tile_lds<OUT, FM, FN>(p, acc, t.batch, m0 + wm * WTM, n0 + wn * WTN, lane,
                                reinterpret_cast<LDS float *>(stage_free) + wave * 32 * WTN);
}

// ---- general kernel

constexpr int GB = 128;            // block tile (rows of A, columns of B)
constexpr int GK = 128;            // k per stage (bytes)
constexpr int GCH = GK / 16;       // 16-byte chunks per panel row
constexpr int GPANEL = GB * GK;    // bytes per operand panel
constexpr int GTHREADS = 256;      // 2 x 2 waves of 64 x 64
constexpr int GPER = GB * GCH / GTHREADS;  // chunks per thread per operand

struct GeneralArgs {
    DmaArgs d;         // K, lda, ldb and strides in bytes
    int a_kmajor, b_kmajor;
    int vec_a, vec_b;  // 16-byte loads allowed (aligned base, ld and stride)
};

// One operand's 128 rows x 128 k of a stage, held in registers between the
// global loads and the LDS writes.  Row r, k of the operand is x[r*ld + k]
// when KMAJOR, else x[k*ld + r]; rows >= R or k >= K read as zero.
template <bool KMAJOR>
struct Stager {
    u32x4 v[GPER];

    // Both members are forced inline: called out of line, the object would
    // live in scratch memory.
    __device__ __forceinline__ void load(const uint8_t *x, int64_t ld, int64_t R, int64_t r0,
                                         int64_t K, int64_t k0, bool vec, int tid) {
#pragma unroll
        for (int i = 0; i < GPER; ++i) {
            const int q = tid + i * GTHREADS;
            // KMAJOR: 16 consecutive k of one row; else 16 consecutive rows at one k
            const int outer = q / GCH, inner = (q % GCH) * 16;
            const int64_t r = KMAJOR ? r0 + outer : r0 + inner;
            const int64_t k = KMAJOR ? k0 + inner : k0 + outer;
            // valid bytes of the 16 (none, or fewer at the matrix's edge)
            const int64_t n = KMAJOR ? (r < R ? K - k : 0) : (k < K ? R - r : 0);
            const uint8_t *src = KMAJOR ? x + r * ld + k : x + k * ld + r;
            if (vec && n >= 16) {
                v[i] = *reinterpret_cast<const u32x4 *>(src);
            } else {
                u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (e < n) w[e >> 2] |= uint32_t(src[e]) << (8 * (e & 3));
                v[i] = w;
            }
        }
    }

    // Into the K-contiguous panel: chunk c of row r at c ^ swz_k<GCH>(r).
    __device__ __forceinline__ void store(LDS char *panel, int tid) const {
#pragma unroll
        for (int i = 0; i < GPER; ++i) {
            const int q = tid + i * GTHREADS;
            const int outer = q / GCH, inner = (q % GCH) * 16;
            if (KMAJOR) {
                *reinterpret_cast<LDS u32x4 *>(panel + outer * GK +
                                               (((inner >> 4) ^ swz_k<GCH>(outer)) << 4)) = v[i];
            } else {
                // byte e is element (row inner + e, k outer)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = inner + e;
                    panel[row * GK + (((outer >> 4) ^ swz_k<GCH>(row)) << 4) + (outer & 15)] =
                        static_cast<char>(v[i][e >> 2] >> (8 * (e & 3)));
                }
            }
        }
    }
};

template <int FA, int FB, int OUT, bool AK, bool BKM>
__global__ __launch_bounds__(GTHREADS) void f8gemm_general_kernel(GeneralArgs g) {
    const DmaArgs &p = g.d;
    constexpr int FM = 2, FN = 2;  // 32 x 32 blocks per wave
    __shared__ __attribute__((aligned(1024))) char smem[2 * GPANEL];
    static_assert(4 * 32 * 64 * 4 <= 2 * GPANEL, "epilogue staging fits in the panels");
    LDS char *lds = (LDS char *)smem;
    LDS char *pa = lds, *pb = lds + GPANEL;

    const TileCoord t = tile_of(p.grid, blockIdx.x);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = t.tm * GB, n0 = t.tn * GB;
    const uint8_t *A = reinterpret_cast<const uint8_t *>(p.A) + t.batch * p.sA;
    const uint8_t *B = reinterpret_cast<const uint8_t *>(p.B) + t.batch * p.sB;
    const int64_t steps = (p.K + GK - 1) / GK;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    Stager<AK> sa;
    Stager<BKM> sb;
    sa.load(A, p.lda, p.M, m0, p.K, 0, g.vec_a, tid);
    sb.load(B, p.ldb, p.N, n0, p.K, 0, g.vec_b, tid);
    sa.store(pa, tid);
    sb.store(pb, tid);
    __syncthreads();
    for (int64_t s = 0; s < steps; ++s) {
        const bool more = s + 1 < steps;
        if (more) {
            sa.load(A, p.lda, p.M, m0, p.K, (s + 1) * GK, g.vec_a, tid);
            sb.load(B, p.ldb, p.N, n0, p.K, (s + 1) * GK, g.vec_b, tid);
        }
#pragma unroll
        for (int kk = 0; kk < GK / 64; ++kk) {
            i32x8 fa[FM], fb[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = frag8<GCH>(pb, wn * 64 + j * 32, kk, lane);
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = frag8<GCH>(pa, wm * 64 + i * 32, kk, lane);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mma8<FA, FB>(fb[j], fa[i], acc[i][j]);
        }
        __syncthreads();  // every wave is done reading the panels
        if (more) {
            sa.store(pa, tid);
            sb.store(pb, tid);
            __syncthreads();
        }
    }
    // The panels are free (last barrier above): stage C through them.
    store_tile_lds<OUT, FM, FN>(p, acc, t.batch, m0 + wm * 64, n0 + wn * 64, lane,
                                reinterpret_cast<LDS float *>(lds) + wave * 32 * 64);
}

// ---- launchers

template <int OUT, template <int, int, int> class L, class Args>
hipError_t by_formats(const Problem &p, Args &a, hipStream_t stream) {
    const bool a4 = p.in == Elem::E4M3, b4 = p.in_b == Elem::E4M3;
    if (a4) return b4 ? L<FMT_E4M3, FMT_E4M3, OUT>::go(p, a, stream)
                      : L<FMT_E4M3, FMT_E5M2, OUT>::go(p, a, stream);
    return b4 ? L<FMT_E5M2, FMT_E4M3, OUT>::go(p, a, stream)
              : L<FMT_E5M2, FMT_E5M2, OUT>::go(p, a, stream);
}

template <template <int, int, int> class L, class Args>
hipError_t by_output(const Problem &p, Args &a, hipStream_t stream) {
    if (p.out == Elem::F32) return by_formats<OUT_F32, L>(p, a, stream);
    if (p.out == Elem::BF16) return by_formats<OUT_BF16, L>(p, a, stream);
    return by_formats<OUT_F16, L>(p, a, stream);
}

template <int FA, int FB, int OUT>
struct LaunchDma {
    static hipError_t go(const Problem &, DmaArgs &a, hipStream_t stream) {
        void *args[] = {&a};
        return hipLaunchKernel(
            reinterpret_cast<const void *>(&f8gemm_dma_kernel<FA, FB, OUT, LIBGEMM_F8_WM,
                                                              LIBGEMM_F8_WN, LIBGEMM_F8_STAGES>),
            dim3(static_cast<unsigned>(a.grid.count())), dim3(LIBGEMM_F8_WM * LIBGEMM_F8_WN * 64),
            args, 0, stream);
    }
};

template <int FA, int FB, int OUT>
struct LaunchGeneral {
    static hipError_t go(const Problem &p, GeneralArgs &a, hipStream_t stream) {
        void *args[] = {&a};
        const void *k = p.a_kmajor ? (p.b_kmajor ? (const void *)&f8gemm_general_kernel<FA, FB, OUT, true, true>
                                                 : (const void *)&f8gemm_general_kernel<FA, FB, OUT, true, false>)
                                   : (p.b_kmajor ? (const void *)&f8gemm_general_kernel<FA, FB, OUT, false, true>
                                                 : (const void *)&f8gemm_general_kernel<FA, FB, OUT, false, false>);
        return hipLaunchKernel(k, dim3(static_cast<unsigned>(a.d.grid.count())), dim3(GTHREADS),
                               args, 0, stream);
    }
};

// The fields of the kernel arguments shared by both kernels (extents along
// K, leading dimensions and strides of A and B still in bytes).
DmaArgs common_args(const Problem &p, int64_t tile, int group_m) {
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
    a.grid = TileGrid{(p.M + tile - 1) / tile, (p.N + tile - 1) / tile, p.batch, group_m, 8};
    a.epi = p.epi;
    return a;
}

}  // namespace

// Every 16-byte chunk of an operand row lies wholly inside or wholly outside
// the matrix (K, leading dimensions and batch strides multiples of 16 bytes,
// 16-byte aligned bases), and an operand slice's byte extent fits the buffer
// range check.
bool f8gemm_dma_eligible(const Problem &p) {
    if (!elem_is_8bit(p.in) || !elem_is_8bit(p.in_b)) return false;
    if (!p.a_kmajor || !p.b_kmajor) return false;
    const int64_t sa = p.batch > 1 ? p.sA : 0, sb = p.batch > 1 ? p.sB : 0;
    if (!vec16_ok(p.A, p.lda, sa, 1) || !vec16_ok(p.B, p.ldb, sb, 1)) return false;
    if (p.K % 16) return false;
    const int64_t limit = int64_t(1) << 30;
    if ((p.M - 1) * p.lda + p.K >= limit || (p.N - 1) * p.ldb + p.K >= limit) return false;
    return true;
}

hipError_t launch_f8gemm_dma(const Problem &p, hipStream_t stream) {
    DmaArgs a = common_args(p, BM, LIBGEMM_F8_GROUP_M);
    if (a.grid.count() > 0x7fffffff) return hipErrorInvalidConfiguration;
    // The panels count in 16-bit units: every extent along K, leading
    // dimension and operand stride is halved (all are even here).
    a.K /= 2;
    a.lda /= 2;
    a.ldb /= 2;
    a.sA /= 2;
    a.sB /= 2;
    return by_output<LaunchDma>(p, a, stream);
}

hipError_t launch_f8gemm(const Problem &p, hipStream_t stream) {
    GeneralArgs g{};
    g.d = common_args(p, GB, 8);
    if (g.d.grid.count() > 0x7fffffff) return hipErrorInvalidConfiguration;
    g.a_kmajor = p.a_kmajor;
    g.b_kmajor = p.b_kmajor;
    const int64_t sa = p.batch > 1 ? p.sA : 0, sb = p.batch > 1 ? p.sB : 0;
    g.vec_a = vec16_ok(p.A, p.lda, sa, 1);
    g.vec_b = vec16_ok(p.B, p.ldb, sb, 1);
    return by_output<LaunchGeneral>(p, g, stream);
}

}  // namespace libgemm
