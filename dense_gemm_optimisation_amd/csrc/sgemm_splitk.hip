// fp32 GEMM for problems with few output tiles: split-K inside one workgroup.
//
// The main fp32 kernel gives each workgroup a 128 x 128 tile; a problem with
// few such tiles (256 x 256, or a skinny M or N) leaves most compute units
// idle.  As for bf16 (split-K / sliced-K in the rasterization and split-K
// section of "GPU GEMM 优化完全拆解（三）", pinghaoyang.com.cn), the K
// dimension is split, inside one workgroup so that the partial sums need no
// memory outside the kernel and are added in a fixed order:
//
//   * a workgroup of 8 waves computes a 32 x 32 tile of C, so the grid has
//     (M/32) x (N/32) x batch workgroups;
//   * wave w takes the w-th of 8 contiguous slices of K (multiples of 32)
//     and streams it through its own 16 KiB of LDS: two 32-deep chunks of A
//     and B, filled with direct global -> LDS loads (16 bytes per lane;
//     loads outside the matrices or past the slice read as zero) and
//     consumed by v_mfma_f32_32x32x2_f32 with the operands swapped (C^T =
//     B^T A^T), as in the main kernel.  A K-contiguous operand chunk is
//     stored [32 rows][32 k] with its eight 16-byte chunks per row swizzled
//     (chunk c of row r at c ^ ((r >> 1) & 7), so 16 consecutive rows read at
//     one chunk touch 16 different bank groups) and read 16 bytes (four k)
//     at a time; an M/N-contiguous one is stored [32 k][32 rows] and read
//     one float at a time.  No wave waits for another until the reduction;
//   * the eight 32 x 32 partials are summed through LDS in wave order and the
//     epilogue computes alpha*sum + beta*C_old (C_old not read when
//     beta == 0).
#include "gemm_problem.hpp"
#include "lds_dma.hpp"
#include "tile_schedule.hpp"

namespace libgemm {
namespace {

using dma::OOB;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVES = 8;
constexpr int TILE = 32;                 // output tile is TILE x TILE
constexpr int CK = 32;                   // k values per chunk
constexpr int PANEL = TILE * CK * 4;     // bytes of one operand chunk (4 KiB)
constexpr int WAVE_LDS = 2 * 2 * PANEL;  // two chunks of A and B per wave
constexpr int LOADS = PANEL / 1024;      // 1 KiB direct loads per operand chunk

struct SplitArgs {
    int64_t M, N, K;
    float alpha, beta;
    const float *A;
    const float *B;
    float *C;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;
    int64_t tiles_m, tiles_n;
    int64_t kper;  // k values per wave slice (a multiple of CK)
    Epilogue epi;
};

// One operand of the tile: TILE rows (of A: m; of B: n) by a wave's K slice.
//   KMAJOR: element (r, k) at X[r*ld + k]; a chunk is [32 r][32 k], 128 bytes
//           per row, 8 rows per direct load.
//   else:   element (r, k) at X[k*ld + r]; a chunk is [32 k][32 r], 128 bytes
//           per k row, 8 k rows per direct load.
template <bool KMAJOR>
struct Slice {
    dma::u32x4 rs;     // raw buffer over the operand (this batch entry)
    int64_t ld, rows;  // leading dimension, extent along r
    int64_t r0;        // first row of the tile

    __device__ void init(const float *x, int64_t ld_, int64_t rows_, int64_t r0_, int64_t span) {
        rs = dma::raw_buffer(dma::uniform(reinterpret_cast<int64_t>(x)), uint32_t(span * 4));
        ld = ld_;
        rows = rows_;
        r0 = r0_;
    }

    // The direct loads of the chunk starting at k0 (k < kend valid).  Lane L
    // of load b fills 16-byte chunk 64b + L of the panel.
    __device__ void issue(uint32_t lds, int64_t k0, int64_t kend, int lane) const {
#pragma unroll
        for (int blk = 0; blk < LOADS; ++blk) {
            const int row = blk * 8 + lane / 8, q = lane % 8;  // row: r or k
            uint32_t v;
            if (KMAJOR) {
                const int c = q ^ ((row >> 1) & 7);
                const int64_t gr = r0 + row, gk = k0 + 4 * c;
                v = (gr < rows && gk < kend) ? uint32_t((gr * ld + gk) * 4) : OOB;
            } else {
                const int64_t gk = k0 + row, gr = r0 + 4 * q;
                v = (gr < rows && gk < kend) ? uint32_t((gk * ld + gr) * 4) : OOB;
            }
            dma::direct_load16(rs, lds + blk * 1024, v);
        }
    }

    // Operands of the four instructions of k group g (k = 8g .. 8g+7): lane
    // l gets row l % 32 at k = 8g + 4*(l / 32) + e in f[e].
    __device__ void frag(const LDS char *panel, int g, int lane, float f[4]) const {
        const int idx = lane & 31, half = lane >> 5;
        if (KMAJOR) {
            const int c = 2 * g + half;
            const f4 v = *reinterpret_cast<const LDS f4 *>(panel + idx * (4 * CK) +
                                                           ((c ^ ((idx >> 1) & 7)) << 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f[e] = *reinterpret_cast<const LDS float *>(panel + (8 * g + 4 * half + e) * (4 * TILE) +
                                                            idx * 4);
        }
    }
};

template <bool A_KMAJOR, bool B_KMAJOR>
__global__ __launch_bounds__(WAVES * 64, 1) void sgemm_splitk_kernel(SplitArgs p) {
    __shared__ __attribute__((aligned(1024))) char smem[WAVES * WAVE_LDS];

    // consecutive tiles (which share cache lines of B when it is N-contiguous)
    // go to one XCD
    const int64_t per_batch = p.tiles_m * p.tiles_n;
    const int64_t id = xcd_remap(blockIdx.x, gridDim.x, 8);
    const int64_t batch = id / per_batch;
    const int64_t local = id - batch * per_batch;
    const int64_t m0 = (local / p.tiles_n) * TILE, n0 = (local % p.tiles_n) * TILE;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    Slice<A_KMAJOR> sa;
    Slice<B_KMAJOR> sb;
    const int64_t span_a = A_KMAJOR ? (p.M - 1) * p.lda + p.K : (p.K - 1) * p.lda + p.M;
    const int64_t span_b = B_KMAJOR ? (p.N - 1) * p.ldb + p.K : (p.K - 1) * p.ldb + p.N;
    sa.init(p.A + batch * p.sA, p.lda, p.M, m0, span_a);
    sb.init(p.B + batch * p.sB, p.ldb, p.N, n0, span_b);

    // this wave's slice of K and its chunks
    const int64_t kw0 = wave * p.kper;
    const int64_t kw1 = kw0 + p.kper < p.K ? kw0 + p.kper : p.K;
    const int64_t nch = kw1 > kw0 ? (kw1 - kw0 + CK - 1) / CK : 0;

    LDS char *mine = (LDS char *)smem + wave * WAVE_LDS;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(mine));
    // chunk buffer b: A at b * 2 * PANEL, B right after it
    auto issue = [&](int64_t c) {
        const uint32_t base = lds0 + uint32_t(c & 1) * 2 * PANEL;
        sa.issue(base, kw0 + c * CK, kw1, lane);
        sb.issue(base + PANEL, kw0 + c * CK, kw1, lane);
    };

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    if (nch > 0) issue(0);
    if (nch > 1) issue(1);
    for (int64_t c = 0; c < nch; ++c) {
        // chunk c has landed when at most the next chunk's loads are pending
        if (c + 1 < nch)
            dma::wait_vmcnt<2 * LOADS>();
        else
            dma::wait_vmcnt<0>();
        const LDS char *pa = mine + (c & 1) * 2 * PANEL;
        const LDS char *pb = pa + PANEL;
        float fa[CK / 8][4], fb[CK / 8][4];
#pragma unroll
        for (int g = 0; g < CK / 8; ++g) {
            sa.frag(pa, g, lane, fa[g]);
            sb.frag(pb, g, lane, fb[g]);
        }
#pragma unroll
        for (int g = 0; g < CK / 8; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[g][e], fa[g][e], acc, 0, 0, 0);
        // the buffer is refilled only after this wave's reads of it are done
        dma::wait_lgkmcnt0();
        if (c + 2 < nch) issue(c + 2);
    }

    // Sum of the eight partials through LDS, in wave order.  Partial w,
    // register r, lane l is at red[(w * 16 + r) * 64 + l]; it is element
    // (m0 + l % 32, n0 + 8*(r / 4) + 4*(l / 32) + r % 4) of C (C^T blocks).
    __syncthreads();  // every wave is done with its chunk buffers
    LDS float *red = (LDS float *)smem;
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    __syncthreads();
    float *C = p.C + batch * p.sC;
#pragma unroll
    for (int h = 0; h < (16 * 64) / (WAVES * 64); ++h) {
        const int e = tid + h * WAVES * 64;  // entry (r, l) = (e / 64, e % 64)
        const int r = e / 64, l = e % 64;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[(w * 16 + r) * 64 + l];
        const int64_t m = m0 + (l & 31);
        const int64_t n = n0 + 8 * (r / 4) + 4 * (l >> 5) + (r & 3);
        if (m < p.M && n < p.N) {
            float *dst = C + m * p.ldc + n;
            float v = p.alpha * s;
            if (p.beta != 0.0f) v = __builtin_fmaf(p.beta, *dst, v);
            if (p.epi.active()) v = epilogue_apply(p.epi, v, batch, m, n);
            *dst = v;
        }
    }
}

template <bool AK, bool BKM>
hipError_t launch(SplitArgs &a, int64_t blocks, hipStream_t stream) {
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(&sgemm_splitk_kernel<AK, BKM>),
                           dim3(static_cast<unsigned>(blocks)), dim3(WAVES * 64), args, 0, stream);
}

}  // namespace

// Few output tiles for the main kernel's 128 x 128 tile (under 160, so at
// least 96 of MI355X's 256 compute units would idle; measured on MI355X the
// split wins at 144 tiles and loses at 256) and a K long enough to split
// eight ways, on operands the direct loads can read whole 16-byte chunks of.
#ifndef LIBGEMM_F32_SPLITK_TILES
#define LIBGEMM_F32_SPLITK_TILES 160
#endif

bool sgemm_splitk_eligible(const Problem &p) {
    if (!sgemm_dma_eligible(p)) return false;
    const int64_t tiles = ((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch;
    return tiles < LIBGEMM_F32_SPLITK_TILES && p.K >= WAVES * CK;
}

hipError_t launch_sgemm_splitk(const Problem &p, hipStream_t stream) {
    SplitArgs a{};
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
    a.tiles_m = (p.M + TILE - 1) / TILE;
    a.tiles_n = (p.N + TILE - 1) / TILE;
    a.kper = ((p.K + WAVES * CK - 1) / (WAVES * CK)) * CK;
    a.epi = p.epi;
    const int64_t blocks = a.tiles_m * a.tiles_n * p.batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (p.a_kmajor)
        return p.b_kmajor ? launch<true, true>(a, blocks, stream)
                          : launch<true, false>(a, blocks, stream);
    return p.b_kmajor ? launch<false, true>(a, blocks, stream)
                      : launch<false, false>(a, blocks, stream);
}

}  // namespace libgemm
