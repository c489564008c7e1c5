// fp32 SGEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// gfx950's matrix cores take fp32 operands at the same peak rate as its
// vector ALUs, but an fp32 matrix instruction does 32 x 32 x 2 multiply-adds
// from two registers per lane, so the operands a wave must fetch from LDS per
// multiply-add are a small fraction of what a register-tiled vector kernel
// needs, and no vector-register bank conflicts arise.  The tiling is the
// block tile -> wave tile -> matrix instruction hierarchy of "GPU GEMM
// 优化完全拆解（三）" (pinghaoyang.com.cn), section "从 kernel 到库":
//
//   * one workgroup of 256 threads (four wave64 waves, 2 x 2) computes a
//     128 x 128 tile of C; each wave owns 64 x 64 of it as 2 x 2
//     accumulators of 32 x 32 (16 fp32 per lane each);
//   * K advances 16 at a time through two LDS panels (128 x 16 of A,
//     16 x 128 of B).  A panel whose operand is K-contiguous in memory is
//     stored [row][k] with its four 16-byte chunks per row XOR-swizzled, and
//     a lane's operands for four consecutive matrix instructions are one
//     16-byte read (the instruction's K index, lane / 32, selects the first
//     or second group of four k, the instruction number the element inside
//     it, the same assignment for A and B: eight k per four instructions).
//     A panel whose operand is contiguous along M or N is stored [k][row]:
//     global loads of four consecutive rows go to LDS as one 16-byte store,
//     and a lane reads two adjacent rows at one k with one 8-byte read, so
//     the wave's two 32-row tiles interleave (tile t, lane index i is row
//     2i + t).  Neither layout has LDS bank conflicts on reads or writes;
//   * the instruction computes C^T = B^T A^T (B's operand in the first
//     slot), which leaves every lane with consecutive columns of one row of
//     C (four, or eight when B is N-contiguous): 16-byte loads and stores of
//     C in the epilogue, at any leading dimension;
//   * the next K step's global loads are issued before the current step's
//     matrix instructions and written to the other LDS buffer after them
//     (double buffering, section 9 of "CUDA GEMM 矩阵乘法优化指南",
//     blog.zhenwei.site); one barrier per step;
//   * edges: elements outside the matrices read as zero and stores outside C
//     are skipped (section 5.2 of the same guide), so any shape, leading
//     dimension and alignment is exact; 16-byte vector loads are used when
//     the operand allows them.
//
// The epilogue computes alpha*acc + beta*C_old in fp32 (C_old not read when
// beta == 0).
#include "gemm_problem.hpp"
#include "lds_dma.hpp"
#include "tile_schedule.hpp"

namespace libgemm {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int THREADS = 256;
constexpr int PANEL = BM * BK;  // floats per operand panel (8 KiB)
static_assert(BM == BN, "both panels share one layout");

struct SgemmArgs {
    int64_t M, N, K;
    float alpha, beta;
    const float *A;
    const float *B;
    float *C;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;
    TileGrid grid;
    int vec_a, vec_b;  // 16-byte vector loads allowed for the operand
    Epilogue epi;
    int64_t span_a, span_b;   // elements of one slice of A and of B the direct loads may touch
};

// Four consecutive elements x[0..3] of one operand row, zero outside
// [0, limit); `inside` says the whole row exists.  A chunk inside the matrix
// is one 16-byte load whatever its alignment: every fp32 element is 4-byte
// aligned, and the global load instructions need no more than that.
typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));

__device__ __attribute__((always_inline)) inline f4 load4(const float *x, bool, bool inside,
                                                          int64_t first, int64_t limit) {
    if (inside && first + 4 <= limit) {
        const f4u u = *reinterpret_cast<const f4u *>(x);
        return f4{u[0], u[1], u[2], u[3]};
    }
    f4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (inside && first + e < limit) ? x[e] : 0.0f;
    return v;
}

// One operand panel in LDS: 128 rows (of A: output rows; of B: output
// columns) by 16 k.
//
// KMAJOR (the operand is K-contiguous in memory): stored [row][k], chunk c
// of row r at chunk c ^ ((r >> 2) & 3).  A lane's operands for four
// instructions are one 16-byte read of four consecutive k, and the two
// 32-row tiles of a wave's 64 rows are rows 0..31 and 32..63.
//
// Otherwise (contiguous along rows in memory): stored [k][row], 128 floats
// per k.  A lane reads two adjacent rows at one k with one 8-byte read, and
// the two 32-row tiles of a wave's 64 rows interleave: tile t, lane index i
// is row 2*i + t.  Global loads of four consecutive rows are written as
// one 16-byte store.
template <bool KMAJOR>
struct Panel {
    __device__ static int at(int row, int k) {
        if (KMAJOR) return row * BK + ((((k >> 2) ^ (row >> 2)) & 3) << 2) + (k & 3);
        return k * BM + row;
    }

    // Row (within the wave's 64) that tile t, lane index i stands for.
    __device__ static int row_of(int t, int i) { return KMAJOR ? t * 32 + i : 2 * i + t; }

    // Global -> registers for the K step at k0: two 4-float chunks per
    // thread.  `rows` is the operand's M (or N) extent, `x` its batch slice;
    // element (row, k) at x[row*ld + k] if KMAJOR, else at x[k*ld + row].
    __device__ __attribute__((always_inline)) static void load(const float *x, int64_t ld, bool vec,
                                                               int64_t r0, int64_t rows, int64_t k0,
                                                               int64_t K, int tid, f4 v[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + THREADS * i;  // chunk id, 0..511
            if (KMAJOR) {                     // 128 rows x 4 chunks along k
                const int row = c >> 2, kq = c & 3;
                const int64_t gr = r0 + row, gk = k0 + kq * 4;
                v[i] = load4(x + gr * ld + gk, vec, gr < rows, gk, K);
            } else {  // 16 k-rows x 32 chunks along the row index
                const int k = c >> 5, rq = c & 31;
                const int64_t gk = k0 + k, gr = r0 + rq * 4;
                v[i] = load4(x + gk * ld + gr, vec, gk < K, gr, rows);
            }
        }
    }

    __device__ __attribute__((always_inline)) static void store(float *s, int tid, const f4 v[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + THREADS * i;
            if (KMAJOR)
                *reinterpret_cast<f4 *>(s + at(c >> 2, (c & 3) * 4)) = v[i];
            else
                *reinterpret_cast<f4 *>(s + at((c & 31) * 4, c >> 5)) = v[i];
        }
    }

    // Operands of the four instructions of k group g (k = 8g .. 8g+7) for
    // the wave's two tiles: f[t][e] is the value at k = 8g + 4*half + e of
    // the row tile t, lane index idx stands for.
    __device__ static void frag(const float *s, int w0, int g, int idx, int half, float f[2][4]) {
        const int k = 8 * g + 4 * half;
        if (KMAJOR) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const f4 v = *reinterpret_cast<const f4 *>(s + at(w0 + row_of(t, idx), k));
#pragma unroll
                for (int e = 0; e < 4; ++e) f[t][e] = v[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f2 v = *reinterpret_cast<const f2 *>(s + at(w0 + 2 * idx, k + e));
                f[0][e] = v[0];
                f[1][e] = v[1];
            }
        }
    }
};

// Epilogue of one wave: C = alpha*acc + beta*C_old for its 64 x 64 tile,
// whose top left corner is (mw, nw); C_old is not read when beta == 0.
template <bool A_KMAJOR, bool B_KMAJOR>
__device__ inline void store_c(const SgemmArgs &p, const f32x16 (&acc)[2][2], float *C, int64_t mw,
                               int64_t nw, int idx, int half, int64_t batch) {
    // Accumulator (i, j) register 4q + e of this lane holds
    // C[mw + Panel<A_KMAJOR>::row_of(i, idx)][nw + Panel<B_KMAJOR>::row_of(j, 8q + 4*half + e)]
    // (the instruction computes C^T, so B's tile index picks the column).
    // It is written as eight 4-column chunks per accumulator row: with a
    // K-contiguous B, chunk (j, q) is columns j*32 + 8q + 4*half + 0..3; with
    // an N-contiguous B, chunk (q, c) is columns 16q + 8*half + 4c + 0..3,
    // column 2e' + j of the eight holding register 4q + e' of tile j.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t row = mw + Panel<A_KMAJOR>::row_of(i, idx);
        if (row >= p.M) continue;
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
            int64_t col;
            f4 v;
            if (B_KMAJOR) {
                const int j = ch >> 2, q = ch & 3;
                col = nw + j * 32 + 8 * q + 4 * half;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = p.alpha * acc[i][j][4 * q + e];
            } else {
                const int q = ch >> 1, c = ch & 1;
                col = nw + 16 * q + 8 * half + 4 * c;
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = p.alpha * acc[i][u & 1][4 * q + 2 * c + (u >> 1)];
            }
            float *dst = C + row * p.ldc + col;
            if (col + 4 <= p.N) {
                if (p.beta != 0.0f) {
                    const f4 old = *reinterpret_cast<const f4u *>(dst);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(p.beta, old[e], v[e]);
                }
                if (p.epi.active())
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = epilogue_apply(p.epi, v[e], batch, row, col + e);
                *reinterpret_cast<f4u *>(dst) = v;
            } else {
                // the chunk's old values are loaded before any is used (from
                // element 0 of C where an element lies outside the matrix), so
                // the four loads are in flight together
                float old[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (p.beta != 0.0f) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) old[e] = *(col + e < p.N ? dst + e : C);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (col + e < p.N) {
                        float x = v[e];
                        if (p.beta != 0.0f) x = __builtin_fmaf(p.beta, old[e], x);
                        if (p.epi.active()) x = epilogue_apply(p.epi, x, batch, row, col + e);
                        dst[e] = x;
                    }
                }
            }
        }
    }
}

template <bool A_KMAJOR, bool B_KMAJOR>
__global__ __launch_bounds__(THREADS, 4) void sgemm_mfma_kernel(SgemmArgs p) {
    __shared__ __attribute__((aligned(16))) float smem[2][2][PANEL];  // [buffer][A, B]
    using PA = Panel<A_KMAJOR>;
    using PB = Panel<B_KMAJOR>;

    const TileCoord t = tile_of(p.grid, blockIdx.x);
    const float *A = p.A + t.batch * p.sA;
    const float *B = p.B + t.batch * p.sB;
    float *C = p.C + t.batch * p.sC;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int idx = lane & 31, half = lane >> 5;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t steps = (p.K + BK - 1) / BK;
    f4 va[2], vb[2];
    PA::load(A, p.lda, p.vec_a, m0, p.M, 0, p.K, tid, va);
    PB::load(B, p.ldb, p.vec_b, n0, p.N, 0, p.K, tid, vb);
    PA::store(smem[0][0], tid, va);
    PB::store(smem[0][1], tid, vb);
    __syncthreads();

    for (int64_t s = 0; s < steps; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < steps;
        if (more) {
            PA::load(A, p.lda, p.vec_a, m0, p.M, (s + 1) * BK, p.K, tid, va);
            PB::load(B, p.ldb, p.vec_b, n0, p.N, (s + 1) * BK, p.K, tid, vb);
        }
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
            float fa[2][4], fb[2][4];
            PA::frag(smem[cur][0], wm * 64, g, idx, half, fa);
            PB::frag(smem[cur][1], wn * 64, g, idx, half, fb);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[j][e], fa[i][e],
                                                                         acc[i][j], 0, 0, 0);
        }
        if (more) {
            PA::store(smem[cur ^ 1][0], tid, va);
            PB::store(smem[cur ^ 1][1], tid, vb);
        }
        __syncthreads();
    }

    store_c<A_KMAJOR, B_KMAJOR>(p, acc, C, m0 + wm * 64, n0 + wn * 64, idx, half, t.batch);
}

// Direct global -> LDS loads of one operand panel, same layouts as Panel:
// the 8 KiB panel is eight 1 KiB blocks, two per wave, and lane L of block b
// fills the panel's 16-byte chunk 64b + L.  A K-contiguous panel's chunk P
// is row P / 4, physical chunk P % 4, which holds logical chunk
// (P % 4) ^ ((row >> 2) & 3), so each lane fetches that global chunk (the
// swizzle is applied on the global side because the loads place lanes
// linearly).  An M/N-contiguous panel's chunk P is k = P / 32, rows
// 4(P % 32) .. +3.  Chunks outside the operand get an out-of-range offset
// and read as zero; that needs every chunk to be wholly inside or outside,
// which the eligibility test guarantees (contiguous extent a multiple of 4).
template <bool KMAJOR>
struct DmaPanel {
    static constexpr int PER_WAVE = PANEL * 4 / 1024 / (THREADS / 64);
    static_assert(PER_WAVE == 2, "two 1 KiB loads per wave per panel");
    uint32_t voff[PER_WAVE];  // byte offset of this lane's chunk in the first stage
    int kl[PER_WAVE];         // first k (within a stage) of this lane's chunk
    const float *base;
    int64_t bytes;            // extent of the operand slice in bytes
    int64_t step;             // bytes the slice start advances per stage

    // X(r, k): KMAJOR -> X[r*ld + k], else X[k*ld + r]; rows [r0, r0+128) of R.
    __device__ void init(const float *x, int64_t ld, int64_t R, int64_t r0, int64_t span, int wave,
                         int lane) {
        base = x;
        bytes = span * 4;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int P = (wave * PER_WAVE + i) * 64 + lane;
            if (KMAJOR) {
                const int row = P >> 2;
                const int c = (P & 3) ^ ((row >> 2) & 3);
                kl[i] = 4 * c;
                const int64_t gr = r0 + row;
                voff[i] = gr < R ? uint32_t((gr * ld + 4 * c) * 4) : dma::OOB;
            } else {
                const int k = P >> 5;
                const int64_t gr = r0 + 4 * (P & 31);
                kl[i] = k;
                voff[i] = gr < R ? uint32_t((k * ld + gr) * 4) : dma::OOB;
            }
        }
        step = KMAJOR ? int64_t(BK) * 4 : int64_t(BK) * ld * 4;
    }

    // The loads of stage `stage` (k from stage*BK) into the panel at LDS
    // address `lds`.
    __device__ void issue(uint32_t lds, int64_t stage, int64_t K, int wave) const {
        const int64_t off = dma::uniform(stage * step);
        const dma::u32x4 rs =
            dma::raw_buffer(static_cast<uint64_t>(dma::uniform(reinterpret_cast<int64_t>(base) + off)),
                            static_cast<uint32_t>(dma::uniform(bytes - off)));
        const int64_t kleft = K - stage * BK;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const uint32_t v = (kleft < BK && kl[i] >= kleft) ? dma::OOB : voff[i];
            dma::direct_load16(rs, lds + (wave * PER_WAVE + i) * 1024, v);
        }
    }
};

// Fast path for aligned operands: the loads of stage s + 1 land in one LDS
// buffer while the matrix instructions of stage s read the other, without
// passing through registers, which leaves the registers for double-buffered
// operand fragments: the reads of a stage's second k group are in flight
// during its first group's matrix instructions, and the reads of the next
// stage's first group (issued right after the barrier) during its second.
// One barrier per stage: it follows this wave's wait for the next stage's
// loads and for its own last reads of the current buffer, so after it every
// wave's data has landed and the current buffer is free to be refilled with
// stage s + 2.  Stages [kb, ke) of tile t are added into acc; the LDS
// buffers are still being read by other waves when this returns.
template <bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void sg_dma_steps(const SgemmArgs &p, float (*smem)[2][PANEL],
                                             const TileCoord &t, int64_t kb, int64_t ke,
                                             f32x16 (&acc)[2][2]) {
    using PA = Panel<A_KMAJOR>;
    using PB = Panel<B_KMAJOR>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int idx = lane & 31, half = lane >> 5;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;

    DmaPanel<A_KMAJOR> da;
    DmaPanel<B_KMAJOR> db;
    da.init(p.A + t.batch * p.sA, p.lda, p.M, m0, p.span_a, wave, lane);
    db.init(p.B + t.batch * p.sB, p.ldb, p.N, n0, p.span_b, wave, lane);
    auto addr = [&](int buf, int op) {
        return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS float *)&smem[buf][op][0]));
    };
    auto issue = [&](int buf, int64_t stage) {
        da.issue(addr(buf, 0), stage, p.K, wave);
        db.issue(addr(buf, 1), stage, p.K, wave);
    };

    float fa[2][2][4], fb[2][2][4];  // [k group slot][tile][instruction]
    auto read = [&](int buf, int g, int slot) {
        PA::frag(smem[buf][0], wm * 64, g, idx, half, fa[slot]);
        PB::frag(smem[buf][1], wn * 64, g, idx, half, fb[slot]);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[slot][j][e], fa[slot][i][e],
                                                                     acc[i][j], 0, 0, 0);
    };

    const int64_t steps = ke - kb;
    issue(0, kb);
    if (steps > 1) {
        issue(1, kb + 1);
        dma::wait_vmcnt<2 * DmaPanel<A_KMAJOR>::PER_WAVE>();
    } else {
        dma::wait_vmcnt<0>();
    }
    __syncthreads();
    read(0, 0, 0);
    for (int64_t s = 0; s + 1 < steps; ++s) {
        const int buf = s & 1;
        read(buf, 1, 1);
        mfmas(0);
        dma::wait_vmcnt<0>();
        dma::wait_lgkmcnt0();
        __syncthreads();
        if (s + 2 < steps) issue(buf, kb + s + 2);
        read(buf ^ 1, 0, 0);
        mfmas(1);
    }
    read((steps - 1) & 1, 1, 1);
    mfmas(0);
    mfmas(1);
}

template <bool A_KMAJOR, bool B_KMAJOR>
__global__ __launch_bounds__(THREADS, 4) void sgemm_mfma_dma_kernel(SgemmArgs p) {
    __shared__ __attribute__((aligned(1024))) float smem[2][2][PANEL];  // [buffer][A, B]
    TileCoord t = tile_of(p.grid, blockIdx.x);
    t.batch = dma::uniform(t.batch);
    t.tm = dma::uniform(t.tm);
    t.tn = dma::uniform(t.tn);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    sg_dma_steps<A_KMAJOR, B_KMAJOR>(p, smem, t, 0, (p.K + BK - 1) / BK, acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    store_c<A_KMAJOR, B_KMAJOR>(p, acc, p.C + t.batch * p.sC, t.tm * BM + (wave >> 1) * 64,
                                t.tn * BN + (wave & 1) * 64, lane & 31, lane >> 5, t.batch);
}

template <bool AK, bool BK_>
hipError_t launch(const SgemmArgs &a0, bool direct, hipStream_t stream) {
    SgemmArgs a = a0;
    void *args[] = {&a};
    const void *fn = direct ? reinterpret_cast<const void *>(&sgemm_mfma_dma_kernel<AK, BK_>)
                            : reinterpret_cast<const void *>(&sgemm_mfma_kernel<AK, BK_>);
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(a.grid.count())), dim3(THREADS), args, 0,
                           stream);
}

// Stream-K schedule of the general fp32 kernel (section 12.5 of "CUDA GEMM
// 矩阵乘法优化指南", blog.zhenwei.site, persistent kernels and Stream-K), the
// split of the 16-bit kernels' schedule with 128 x 128 tiles and four
// workgroups per compute unit (G = 4 per unit): the tiles filling whole
// waves of G are computed whole, tile w + n*G by workgroup w; the (tile, k
// step) iterations of the other tiles are split evenly over Gs workgroups; a
// piece covering a whole tile is stored through the epilogue, any other is
// written to the workgroup's slot 2w (the piece holding its last iteration)
// or 2w + 1 (its first), and sgemm_streamk_fixup adds the pieces of each cut
// tile in increasing workgroup order and applies the epilogue.
struct SgStreamK : StreamKSplit {
    float *partials;    // 2 * Gs slots of 128 x 128 floats
};

constexpr int SG_SLOT = BM * BN;  // floats per partial tile

// Slot `slot` as a raw buffer: register quad q of accumulator (i, j) of
// thread tid is the 16 bytes at ((i*2 + j)*4 + q) * THREADS * 16 + tid * 16.
__device__ inline __amdgpu_buffer_rsrc_t sg_slot(const SgStreamK &sk, int64_t slot) {
    return __builtin_amdgcn_make_buffer_rsrc(sk.partials + slot * SG_SLOT, 0, SG_SLOT * 4,
                                             0x00020000);
}

// k steps [kb, ke) of tile t into acc: the general kernel's loop.
template <bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void sg_tile_steps(const SgemmArgs &p, float (*smem)[2][PANEL],
                                              const TileCoord &t, int64_t kb, int64_t ke,
                                              f32x16 (&acc)[2][2]) {
    using PA = Panel<A_KMAJOR>;
    using PB = Panel<B_KMAJOR>;
    const float *A = p.A + t.batch * p.sA;
    const float *B = p.B + t.batch * p.sB;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int idx = lane & 31, half = lane >> 5;
    f4 va[2], vb[2];
    PA::load(A, p.lda, p.vec_a, m0, p.M, kb * BK, p.K, tid, va);
    PB::load(B, p.ldb, p.vec_b, n0, p.N, kb * BK, p.K, tid, vb);
    PA::store(smem[0][0], tid, va);
    PB::store(smem[0][1], tid, vb);
    __syncthreads();
    for (int64_t s = kb; s < ke; ++s) {
        const int cur = (s - kb) & 1;
        const bool more = s + 1 < ke;
        if (more) {
            PA::load(A, p.lda, p.vec_a, m0, p.M, (s + 1) * BK, p.K, tid, va);
            PB::load(B, p.ldb, p.vec_b, n0, p.N, (s + 1) * BK, p.K, tid, vb);
        }
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
            float fa[2][4], fb[2][4];
            PA::frag(smem[cur][0], wm * 64, g, idx, half, fa);
            PB::frag(smem[cur][1], wn * 64, g, idx, half, fb);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[j][e], fa[i][e],
                                                                         acc[i][j], 0, 0, 0);
        }
        if (more) {
            PA::store(smem[cur ^ 1][0], tid, va);
            PB::store(smem[cur ^ 1][1], tid, vb);
        }
        __syncthreads();
    }
}

// DIRECT: the direct-load k loop (aligned operands), else the general one.
template <bool A_KMAJOR, bool B_KMAJOR, bool DIRECT>
__global__ __launch_bounds__(THREADS, 4) void sgemm_streamk_kernel(SgemmArgs p, SgStreamK sk) {
    __shared__ __attribute__((aligned(1024))) float smem[2][2][PANEL];
    // logical workgroup: the hardware id regrouped per XCD
    const int64_t G = gridDim.x, S = sk.steps;
    const int64_t w = dma::uniform(xcd_remap(blockIdx.x, G, 8));
    const int64_t n_dp = dma::uniform(sk_whole_tiles(sk, w, G));
    const int64_t begin = dma::uniform(sk_begin(sk, w));
    const int64_t end = dma::uniform(sk_end(sk, w));
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int64_t it = begin;
    for (int64_t item = 0;; ++item) {
        int64_t tile, kb, ke, local = 0;
        if (item < n_dp) {
            tile = w + item * G;
            kb = 0;
            ke = S;
        } else {
            if (it >= end) break;
            local = dma::uniform(it / S);
            const StreamKPiece pc = sk_piece(sk, local, it, end);
            kb = pc.kb;
            ke = pc.ke;
            tile = sk.dp_tiles + local;
            it = local * S + ke;
        }
        TileCoord t = tile_of(p.grid, tile);
        t.batch = dma::uniform(t.batch);
        t.tm = dma::uniform(t.tm);
        t.tn = dma::uniform(t.tn);
        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        if (DIRECT) {
            // the previous item's last LDS reads are done in every wave
            // before this item's loads overwrite the buffers
            if (item > 0) __syncthreads();
            sg_dma_steps<A_KMAJOR, B_KMAJOR>(p, smem, t, kb, ke, acc);
        } else {
            sg_tile_steps<A_KMAJOR, B_KMAJOR>(p, smem, t, kb, ke, acc);
        }
        if (kb == 0 && ke == S) {
            store_c<A_KMAJOR, B_KMAJOR>(p, acc, p.C + t.batch * p.sC, t.tm * BM + wm * 64,
                                        t.tn * BN + wn * 64, lane & 31, lane >> 5, t.batch);
        } else {
            const __amdgpu_buffer_rsrc_t rs = sg_slot(sk, sk_slot(sk, w, local, end));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                      acc[i][j][4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(u4, v), rs,
                            tid * 16, ((i * 2 + j) * 4 + q) * THREADS * 16, 0);
                    }
        }
    }
}

// Workgroup (local tile, piece), piece = (i*2 + j)*4 + q: sums register quad
// q of accumulator (i, j) over the pieces of cut tile `local`, lowest
// workgroup first, and stores it.  Register 4q + e of accumulator (i, j) of a
// lane holds C[mw + row_of_A(i, idx)][nw + row_of_B(j, 8q + 4*half + e)].
template <bool A_KMAJOR, bool B_KMAJOR>
__global__ __launch_bounds__(THREADS) void sgemm_streamk_fixup(SgemmArgs p, SgStreamK sk) {
    constexpr int BATCH = 8;  // pieces whose loads are in flight together
    const int64_t S = sk.steps;
    const int64_t local = blockIdx.x / 16;
    const int piece = blockIdx.x % 16;
    const int64_t g0 = sk_owner(sk, local * S), g1 = sk_owner(sk, local * S + S - 1);
    if (g0 == g1) return;
    const int tid = threadIdx.x;
    // every owner but the last holds its last iteration here (slot 2g)
    const int64_t slot1 = sk_slot(sk, g1, local, sk_end(sk, g1));
    f4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t g = g0; g <= g1; g += BATCH) {
        f4 v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            // past the last piece: an offset beyond the buffer reads zeros
            const int64_t gu = g + u <= g1 ? g + u : g1;
            const uint32_t off = g + u <= g1 ? static_cast<uint32_t>(tid * 16) : 0x80000000u;
            v[u] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                                              sg_slot(sk, gu == g1 ? slot1 : 2 * gu), off,
                                              piece * THREADS * 16, 0));
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) sum += v[u];
    }
    const TileCoord t = tile_of(p.grid, sk.dp_tiles + local);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int idx = lane & 31, half = lane >> 5;
    const int i = piece >> 3, j = (piece >> 2) & 1, q = piece & 3;
    const int64_t row = t.tm * BM + wm * 64 + Panel<A_KMAJOR>::row_of(i, idx);
    if (row >= p.M) return;
    float *C = p.C + t.batch * p.sC;
    float old[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t col = t.tn * BN + wn * 64 + Panel<B_KMAJOR>::row_of(j, 8 * q + 4 * half + e);
        old[e] = p.beta != 0.0f ? C[row * p.ldc + (col < p.N ? col : 0)] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t col = t.tn * BN + wn * 64 + Panel<B_KMAJOR>::row_of(j, 8 * q + 4 * half + e);
        if (col >= p.N) continue;
        float x = p.alpha * sum[e];
        if (p.beta != 0.0f) x = __builtin_fmaf(p.beta, old[e], x);
        if (p.epi.active()) x = epilogue_apply(p.epi, x, t.batch, row, col);
        C[row * p.ldc + col] = x;
    }
}

template <bool AK, bool BKM, bool DIRECT>
hipError_t launch_sk(SgemmArgs &a, SgStreamK &sk, int64_t grid, hipStream_t stream) {
    void *args[] = {&a, &sk};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&sgemm_streamk_kernel<AK, BKM, DIRECT>),
                                   dim3(static_cast<unsigned>(grid)), dim3(THREADS), args, 0, stream);
    if (e != hipSuccess || sk.iters == 0) return e;
    const int64_t cut = a.grid.count() - sk.dp_tiles;
    return hipLaunchKernel(reinterpret_cast<const void *>(&sgemm_streamk_fixup<AK, BKM>),
                           dim3(static_cast<unsigned>(cut * 16)), dim3(THREADS), args, 0, stream);
}

}  // namespace

// The direct-load kernel needs 16-byte aligned operand rows (base, leading
// dimension and batch stride), a contiguous extent that is a multiple of 4
// (so every 16-byte chunk is wholly inside or outside the operand) and
// operand slices below 2^31 bytes (32-bit buffer offsets, with the
// out-of-range offset beyond every slice).
bool sgemm_dma_eligible(const Problem &p) {
    if (p.in != Elem::F32) return false;
    const int64_t sa = p.batch > 1 ? p.sA : 0, sb = p.batch > 1 ? p.sB : 0;
    if (!vec16_ok(p.A, p.lda, sa, 4) || !vec16_ok(p.B, p.ldb, sb, 4)) return false;
    if (!p.packed && ((p.a_kmajor ? p.K : p.M) % 4 || (p.b_kmajor ? p.K : p.N) % 4)) return false;
    const int64_t limit = int64_t(1) << 31;
    return 4 * operand_span_a(p) < limit && 4 * operand_span_b(p) < limit;
}

namespace {

SgemmArgs make_args(const Problem &p) {
    SgemmArgs a{};
    a.M = p.M;
    a.N = p.N;
    a.K = p.K;
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.A = static_cast<const float *>(p.A);
    a.B = static_cast<const float *>(p.B);
    a.C = static_cast<float *>(p.C);
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.sA = p.batch > 1 ? p.sA : 0;
    a.sB = p.batch > 1 ? p.sB : 0;
    a.sC = p.batch > 1 ? p.sC : 0;
    a.grid = TileGrid{(p.M + BM - 1) / BM, (p.N + BN - 1) / BN, p.batch, 8, 8};
    a.vec_a = vec16_ok(p.A, p.lda, a.sA, 4);
    a.vec_b = vec16_ok(p.B, p.ldb, a.sB, 4);
    a.epi = p.epi;
    a.span_a = operand_span_a(p);
    a.span_b = operand_span_b(p);
    return a;
}

hipError_t launch_any(const Problem &p, bool direct, hipStream_t stream) {
    const SgemmArgs a = make_args(p);
    if (a.grid.count() > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (p.a_kmajor)
        return p.b_kmajor ? launch<true, true>(a, direct, stream)
                          : launch<true, false>(a, direct, stream);
    return p.b_kmajor ? launch<false, true>(a, direct, stream)
                      : launch<false, false>(a, direct, stream);
}

}  // namespace

hipError_t launch_sgemm_mfma(const Problem &p, hipStream_t stream) {
    return launch_any(p, false, stream);
}

hipError_t launch_sgemm_dma(const Problem &p, hipStream_t stream) {
    return launch_any(p, true, stream);
}

namespace {

// Cost of the partial-tile exchange, in k steps (16 k) of one tile, and the
// step time over partial-tile time for streamk_groups (4.4 us per k step of
// a workgroup at 4096^3 with four per compute unit, 0.03 us per 64 KiB
// partial tile moved through HBM twice).
constexpr int64_t SG_SK_EXCHANGE_STEPS = 8;
#ifndef LIBGEMM_SG_SK_RATIO
#define LIBGEMM_SG_SK_RATIO 140
#endif

}  // namespace

// Worth it when the steps the cut last wave saves exceed the exchange:
// ceil(T_r * S / G) steps per workgroup instead of S, with G =
// SGEMM_STREAMK_MAX_GRID workgroups (four per compute unit of MI355X).
bool sgemm_streamk_eligible(const Problem &p, bool force) {
    if (p.in != Elem::F32) return false;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.batch;
    const int64_t steps = (p.K + BK - 1) / BK;
    const int64_t g = SGEMM_STREAMK_MAX_GRID;
    const int64_t cut = tiles % g;
    if (cut == 0 || tiles >= (int64_t(1) << 24) || steps >= (int64_t(1) << 24)) return false;
    const int64_t tail = (cut * steps + g - 1) / g;
    return force || steps - tail > SG_SK_EXCHANGE_STEPS;
}

namespace {

// The split over SGEMM_STREAMK_MAX_GRID workgroups (four per compute unit of
// MI355X; on a part with fewer units the schedule is still correct).
StreamKSplit sg_streamk_split(const Problem &p) {
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.batch;
    return streamk_split(tiles, (p.K + BK - 1) / BK, SGEMM_STREAMK_MAX_GRID, LIBGEMM_SG_SK_RATIO);
}

}  // namespace

int64_t sgemm_streamk_bytes(const Problem &p) {
    return 2 * sg_streamk_split(p).groups * int64_t(SG_SLOT) * 4;
}

bool sgemm_dma_streamk_eligible(const Problem &p, bool force) {
    return sgemm_dma_eligible(p) && sgemm_streamk_eligible(p, force);
}

namespace {

template <bool DIRECT>
hipError_t launch_streamk(const Problem &p, void *workspace, hipStream_t stream) {
    SgemmArgs a = make_args(p);
    a.grid.xcds = 1;  // the work order itself spreads tiles over the dies
    SgStreamK sk{};
    static_cast<StreamKSplit &>(sk) = sg_streamk_split(p);
    sk.partials = static_cast<float *>(workspace);
    const int64_t grid = streamk_grid(sk, SGEMM_STREAMK_MAX_GRID);
    if (grid == 0) return hipSuccess;
    if (p.a_kmajor)
        return p.b_kmajor ? launch_sk<true, true, DIRECT>(a, sk, grid, stream)
                          : launch_sk<true, false, DIRECT>(a, sk, grid, stream);
    return p.b_kmajor ? launch_sk<false, true, DIRECT>(a, sk, grid, stream)
                      : launch_sk<false, false, DIRECT>(a, sk, grid, stream);
}

}  // namespace

hipError_t launch_sgemm_streamk(const Problem &p, void *workspace, hipStream_t stream) {
    return launch_streamk<false>(p, workspace, stream);
}

hipError_t launch_sgemm_dma_streamk(const Problem &p, void *workspace, hipStream_t stream) {
    return launch_streamk<true>(p, workspace, stream);
}

}  // namespace libgemm
