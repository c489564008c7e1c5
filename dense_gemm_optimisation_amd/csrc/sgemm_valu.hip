// fp32 SGEMM on the vector ALUs of gfx950.
//
// One workgroup of 256 threads (four wave64 waves) computes a 128 x 256 tile
// of C.  The K dimension is walked in steps of 16: each step stages a 128 x 16
// panel of A and a 16 x 256 panel of B in LDS, and every thread accumulates an
// 8 x 16 block of C in registers as a sum of outer products (register tiling,
// "CUDA GEMM 矩阵乘法优化指南" (blog.zhenwei.site) section 7; the 128/128/8
// block shape and 8 x 8 thread tile of section 4 of "第4章：经典算子实现 ——
// GEMM", widened along N).  An 8 x 16 thread tile issues six 16-byte LDS
// reads per 128 fused multiply-adds, against four per 64 for 8 x 8; the LDS
// read rate is what an 8 x 8 tile runs out of first on gfx950.  A is stored transposed in LDS (k-major) so that a thread's eight A
// values for one k are contiguous, with four floats of padding per row against
// bank conflicts (section 4.2 of the m.lqnn.cn SGEMM article).  Global loads
// are 16-byte vectors when the operand's base, leading dimension and batch
// stride allow it (section 8 of the zhenwei.site guide), and the LDS panels
// are double-buffered: the next step's global loads are issued before the
// current step's arithmetic and written to the other buffer after it
// (section 9 of the zhenwei.site guide), one barrier per step.
//
// Thread layout: thread t owns rows {4*ty + i, 64 + 4*ty + i} and columns
// {64*g + 4*tx + j} (ty = t / 16, tx = t % 16, i, j < 4, g < 4).  Within a
// wave the four ty values read four distinct 16-byte A words (broadcast to 16
// lanes each) and the sixteen tx values read 256 contiguous bytes of B.
//
// Edges: loads outside [0, M) x [0, K) and [0, K) x [0, N) read as zero
// (the zero-fill of section 5.2 of the zhenwei.site guide) and stores outside
// [0, M) x [0, N) are skipped, so any shape is exact.
#include "gemm_problem.hpp"
#include "tile_schedule.hpp"

namespace libgemm {
namespace {

constexpr int NB = 4;  // 64-column groups per thread row
constexpr int BM = 128, BN = 64 * NB, BK = 16;
constexpr int THREADS = 256;
constexpr int PAD = 4;
constexpr int SA = BM + PAD;  // floats per k-row of the A panel
constexpr int SB = BN + PAD;  // floats per k-row of the B panel

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
};

typedef float f4 __attribute__((ext_vector_type(4)));
// a 4-float chunk of C at 4-byte alignment (rows of C start wherever ldc
// puts them; the memory system takes a 16-byte access at any such address)
typedef float f4_ea __attribute__((ext_vector_type(4), aligned(4)));

// Four consecutive elements x[0..3] of one row of an operand, zero outside
// [0, limit).  `inside` says the whole row exists.
__device__ inline f4 load4(const float *x, bool vec, bool inside, int64_t first, int64_t limit) {
    if (vec && inside && first + 4 <= limit) return *reinterpret_cast<const f4 *>(x);
    f4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (inside && first + e < limit) ? x[e] : 0.0f;
    return v;
}

// Global -> registers for one K step: two 4-float chunks of A and NB of B.
template <bool A_KMAJOR, bool B_KMAJOR>
__device__ inline void load_step(const SgemmArgs &p, const float *A, const float *B, int64_t m0,
                                 int64_t n0, int64_t k0, int tid, f4 ra[2], f4 rb[NB]) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int c = tid + THREADS * r;  // chunk id, 0..511
        if (A_KMAJOR) {                   // 128 rows x 4 chunks along k
            const int row = c >> 2, kq = c & 3;
            const int64_t gm = m0 + row, gk = k0 + kq * 4;
            ra[r] = load4(A + gm * p.lda + gk, p.vec_a, gm < p.M, gk, p.K);
        } else {  // 16 k-rows x 32 chunks along m
            const int k = c >> 5, mq = c & 31;
            const int64_t gk = k0 + k, gm = m0 + mq * 4;
            ra[r] = load4(A + gk * p.lda + gm, p.vec_a, gk < p.K, gm, p.M);
        }
    }
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        const int c = tid + THREADS * r;  // chunk id, 0 .. 256*NB-1
        if (B_KMAJOR) {                   // BN columns x 4 chunks along k
            const int col = c >> 2, kq = c & 3;
            const int64_t gn = n0 + col, gk = k0 + kq * 4;
            rb[r] = load4(B + gn * p.ldb + gk, p.vec_b, gn < p.N, gk, p.K);
        } else {  // 16 k-rows x BN/4 chunks along n
            const int k = c / (BN / 4), nq = c % (BN / 4);
            const int64_t gk = k0 + k, gn = n0 + nq * 4;
            rb[r] = load4(B + gk * p.ldb + gn, p.vec_b, gk < p.K, gn, p.N);
        }
    }
}

// Registers -> LDS panels (A transposed to k-major, B k-major).
template <bool A_KMAJOR, bool B_KMAJOR>
__device__ inline void store_step(float (*sA)[SA], float (*sB)[SB], int tid, const f4 ra[2],
                                  const f4 rb[NB]) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int c = tid + THREADS * r;
        if (A_KMAJOR) {
            const int row = c >> 2, kq = c & 3;
#pragma unroll
            for (int e = 0; e < 4; ++e) sA[kq * 4 + e][row] = ra[r][e];
        } else {
            const int k = c >> 5, mq = c & 31;
            *reinterpret_cast<f4 *>(&sA[k][mq * 4]) = ra[r];
        }
    }
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        const int c = tid + THREADS * r;
        if (B_KMAJOR) {
            const int col = c >> 2, kq = c & 3;
#pragma unroll
            for (int e = 0; e < 4; ++e) sB[kq * 4 + e][col] = rb[r][e];
        } else {
            const int k = c / (BN / 4), nq = c % (BN / 4);
            *reinterpret_cast<f4 *>(&sB[k][nq * 4]) = rb[r];
        }
    }
}

template <bool A_KMAJOR, bool B_KMAJOR>
__global__ __launch_bounds__(THREADS, 1) void sgemm_kernel(SgemmArgs p) {
    __shared__ float sA[2][BK][SA];
    __shared__ float sB[2][BK][SB];

    const TileCoord t = tile_of(p.grid, blockIdx.x);
    const float *A = p.A + t.batch * p.sA;
    const float *B = p.B + t.batch * p.sB;
    float *C = p.C + t.batch * p.sC;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;

    float acc[8][4 * NB];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4 * NB; ++j) acc[i][j] = 0.0f;

    const int64_t steps = (p.K + BK - 1) / BK;
    f4 ra[2], rb[NB];
    load_step<A_KMAJOR, B_KMAJOR>(p, A, B, m0, n0, 0, tid, ra, rb);
    store_step<A_KMAJOR, B_KMAJOR>(sA[0], sB[0], tid, ra, rb);
    __syncthreads();

    for (int64_t s = 0; s < steps; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < steps;
        if (more) load_step<A_KMAJOR, B_KMAJOR>(p, A, B, m0, n0, (s + 1) * BK, tid, ra, rb);
        // Unrolled by two: unrolled further, the compiler issues more
        // k-steps' LDS reads up front and runs out of registers.
#pragma unroll 2
        for (int k = 0; k < BK; ++k) {
            const f4 a0 = *reinterpret_cast<const f4 *>(&sA[cur][k][ty * 4]);
            const f4 a1 = *reinterpret_cast<const f4 *>(&sA[cur][k][64 + ty * 4]);
            f4 b[NB];
#pragma unroll
            for (int g = 0; g < NB; ++g) b[g] = *reinterpret_cast<const f4 *>(&sB[cur][k][64 * g + tx * 4]);
            const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int g = 0; g < NB; ++g)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][4 * g + j] = __builtin_fmaf(a[i], b[g][j], acc[i][4 * g + j]);
        }
        if (more) store_step<A_KMAJOR, B_KMAJOR>(sA[cur ^ 1], sB[cur ^ 1], tid, ra, rb);
        __syncthreads();
    }

    // Epilogue: C = alpha*acc + beta*C_old, 16-byte stores where possible.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + (i - 4));
        if (row >= p.M) continue;
#pragma unroll
        for (int h = 0; h < NB; ++h) {
            const int64_t col = n0 + h * 64 + tx * 4;
            float *dst = C + row * p.ldc + col;
            f4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = p.alpha * acc[i][h * 4 + j];
            if (col + 4 <= p.N) {
                if (p.beta != 0.0f) {
                    const f4 old = *reinterpret_cast<const f4_ea *>(dst);
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = __builtin_fmaf(p.beta, old[j], v[j]);
                }
                if (p.epi.active())
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = epilogue_apply(p.epi, v[j], t.batch, row, col + j);
                *reinterpret_cast<f4_ea *>(dst) = v;
            } else {
                // the chunk across the right edge: its old values are loaded
                // before any is used (element col stands in for those past
                // the edge), so the loads are in flight together
                float old[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (p.beta != 0.0f) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) old[j] = dst[col + j < p.N ? j : 0];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (col + j < p.N) {
                        float x = v[j];
                        if (p.beta != 0.0f) x = __builtin_fmaf(p.beta, old[j], x);
                        if (p.epi.active()) x = epilogue_apply(p.epi, x, t.batch, row, col + j);
                        dst[j] = x;
                    }
                }
            }
        }
    }
}

template <bool AK, bool BK_>
hipError_t launch(SgemmArgs &a, hipStream_t stream) {
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(&sgemm_kernel<AK, BK_>),
                           dim3(static_cast<unsigned>(a.grid.count())), dim3(THREADS), args, 0,
                           stream);
}

}  // namespace

hipError_t launch_sgemm(const Problem &p, hipStream_t stream) {
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
    if (a.grid.count() > 0x7fffffff) return hipErrorInvalidConfiguration;
    a.vec_a = vec16_ok(p.A, p.lda, a.sA, 4);
    a.vec_b = vec16_ok(p.B, p.ldb, a.sB, 4);
    a.epi = p.epi;
    if (p.a_kmajor)
        return p.b_kmajor ? launch<true, true>(a, stream) : launch<true, false>(a, stream);
    return p.b_kmajor ? launch<false, true>(a, stream) : launch<false, false>(a, stream);
}

}  // namespace libgemm
