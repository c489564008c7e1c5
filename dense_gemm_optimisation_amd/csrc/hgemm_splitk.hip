// bf16 / fp16 GEMM for problems with few output tiles and a long K: split-K
// inside one workgroup.
//
// A GEMM whose C has few 256 x 256 tiles (a skinny M or N, as in a
// 16 x 4096 x 4096 product) leaves most compute units idle on the main
// kernel, and such problems are bound by reading the long operand from HBM,
// not by the matrix cores.  The pages' remedy is to split the K dimension
// (split-K / sliced-K in the rasterization and split-K section of "GPU GEMM
// 优化完全拆解（三）", pinghaoyang.com.cn); here the split stays inside one
// workgroup, so the partial sums need no memory outside the kernel and are
// added in a fixed order:
//
//   * a workgroup of 8 waves computes a 32 x 32 tile of C, so the grid has
//     (M/32) x (N/32) x batch workgroups, enough to occupy every compute unit
//     for the shapes that take this path;
//   * wave w takes the w-th of 8 contiguous slices of K (multiples of 64)
//     and streams its slice of A and B through its own 16 KiB of LDS: two
//     64-deep chunks, filled with direct global -> LDS loads (16 bytes per
//     lane; loads outside the matrices or past the slice read as zero) and
//     consumed by v_mfma_f32_32x32x16 with the operands swapped (C^T = B^T
//     A^T), as in the main kernel.  An operand contiguous along K is read with
//     16-byte LDS reads, one contiguous along M or N with transposing reads
//     (ds_read_b64_tr_b16).  No wave waits for another until the reduction;
//   * the eight 32 x 32 partials are summed through LDS in wave order, and the
//     fp32 epilogue computes alpha*sum + beta*C_old (C_old not read when
//     beta == 0) and rounds to the output type to nearest-even.
#include "gemm_problem.hpp"
#include "lds_dma.hpp"
#include "tile_schedule.hpp"

namespace libgemm {
namespace {

using dma::OOB;
using dma::direct_load16;
using dma::wait_lgkmcnt0;
using dma::wait_vmcnt;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));


constexpr int WAVES = 8;
constexpr int TILE = 32;                     // output tile is TILE x TILE
constexpr int CK = 64;                       // k values per chunk
constexpr int PANEL = TILE * CK * 2;         // bytes of one operand chunk (4 KiB)
constexpr int WAVE_LDS = 2 * 2 * PANEL;      // two chunks of A and B per wave
constexpr int OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2;

struct SplitArgs {
    int64_t M, N, K;
    float alpha, beta;
    const uint16_t *A;
    const uint16_t *B;
    void *C;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;
    int64_t tiles_m, tiles_n;
    int64_t kper;  // k values per wave slice (a multiple of CK)
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

// One operand of the tile: TILE rows (of A: m; of B: n) by a wave's K slice.
//   KMAJOR: element (r, k) at X[r*ld + k]; a chunk is stored [32 r][64 k],
//           128 bytes per row, loaded 8 rows per instruction.
//   else:   element (r, k) at X[k*ld + r]; a chunk is stored [64 k][32 r],
//           64 bytes per k row, loaded 16 k rows per instruction.
template <bool KMAJOR>
struct Slice {
    u32x4 rs;          // raw buffer over the operand (this batch entry)
    int64_t ld, rows;  // leading dimension, extent along r
    int64_t r0;        // first row of the tile

    __device__ void init(const uint16_t *x, int64_t ld_, int64_t rows_, int64_t r0_, int64_t span) {
        rs = dma::raw_buffer(dma::uniform(reinterpret_cast<int64_t>(x)), uint32_t(span * 2));
        ld = ld_;
        rows = rows_;
        r0 = r0_;
    }

    // The four direct loads of the chunk starting at k0 (k < kend valid).
    __device__ void issue(uint32_t lds, int64_t k0, int64_t kend, int lane) const {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            uint32_t v;
            if (KMAJOR) {
                const int row = blk * 8 + lane / 8, q = lane % 8;
                const int64_t gr = r0 + row, gk = k0 + q * 8;
                v = (gr < rows && gk < kend) ? uint32_t((gr * ld + gk) * 2) : OOB;
            } else {
                const int krow = blk * 16 + lane / 4, q = lane % 4;
                const int64_t gk = k0 + krow, gr = r0 + q * 8;
                v = (gr < rows && gk < kend) ? uint32_t((gk * ld + gr) * 2) : OOB;
            }
            direct_load16(rs, lds + blk * 1024, v);
        }
    }

    // Fragment of the 32 rows for k16 step kk of the chunk at `panel`: lane l
    // gets row l % 32, k values 8*(l / 32) .. +7.
    __device__ u32x4 frag(const LDS char *panel, int kk, int lane) const {
        if (KMAJOR) {
            const int row = lane & 31, c = kk * 2 + (lane >> 5);
            return *reinterpret_cast<const LDS u32x4 *>(panel + row * (2 * CK) + c * 16);
        } else {
            const int g = lane >> 5, h = (lane >> 4) & 1, ii = lane & 15;
            const int col = h * 16 + 4 * (ii & 3);
            u32x4 out;
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const int krow = kk * 16 + g * 8 + e2 * 4 + (ii >> 2);
                const LDS s16x4 *p =
                    reinterpret_cast<const LDS s16x4 *>(panel + krow * (2 * TILE) + col * 2);
                const u32x2 v = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<LDS s16x4 *>(p)));
                out[2 * e2] = v[0];
                out[2 * e2 + 1] = v[1];
            }
            return out;
        }
    }
};

template <int OUT>
__device__ inline float load_c(const void *C, int64_t off) {
    if (OUT == OUT_F32) return static_cast<const float *>(C)[off];
    const uint16_t bits = static_cast<const uint16_t *>(C)[off];
    if (OUT == OUT_BF16) return __builtin_bit_cast(float, uint32_t(bits) << 16);
    return static_cast<float>(__builtin_bit_cast(_Float16, bits));
}

template <int OUT>
__device__ inline void store_c(void *C, int64_t off, float v) {
    if (OUT == OUT_F32)
        static_cast<float *>(C)[off] = v;
    else if (OUT == OUT_BF16)
        static_cast<uint16_t *>(C)[off] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    else
        static_cast<uint16_t *>(C)[off] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

template <class T, int OUT, bool A_KMAJOR, bool B_KMAJOR>
__global__ __launch_bounds__(WAVES * 64, 1) void hgemm_splitk_kernel(SplitArgs p) {
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
        // chunk c has landed when at most the next chunk's 8 loads are pending
        if (c + 1 < nch)
            wait_vmcnt<8>();
        else
            wait_vmcnt<0>();
        const LDS char *pa = mine + (c & 1) * 2 * PANEL;
        const LDS char *pb = pa + PANEL;
        u32x4 fa[CK / 16], fb[CK / 16];
#pragma unroll
        for (int kk = 0; kk < CK / 16; ++kk) {
            fa[kk] = sa.frag(pa, kk, lane);
            fb[kk] = sb.frag(pb, kk, lane);
        }
#pragma unroll
        for (int kk = 0; kk < CK / 16; ++kk) acc = mfma32<T>(fb[kk], fa[kk], acc);
        // the buffer is refilled only after this wave's reads of it are done
        wait_lgkmcnt0();
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
    char *Cb = static_cast<char *>(p.C) + batch * p.sC * (OUT == OUT_F32 ? 4 : 2);
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
            const int64_t off = m * p.ldc + n;
            float v = p.alpha * s;
            if (p.beta != 0.0f) v = __builtin_fmaf(p.beta, load_c<OUT>(Cb, off), v);
            if (p.epi.active()) v = epilogue_apply(p.epi, v, batch, m, n);
            store_c<OUT>(Cb, off, v);
        }
    }
}

template <class T, int OUT, bool AK, bool BKM>
hipError_t launch(SplitArgs &a, int64_t blocks, hipStream_t stream) {
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(&hgemm_splitk_kernel<T, OUT, AK, BKM>),
                           dim3(static_cast<unsigned>(blocks)), dim3(WAVES * 64), args, 0, stream);
}

template <class T, int OUT>
hipError_t launch_layout(const Problem &p, SplitArgs &a, int64_t blocks, hipStream_t stream) {
    if (p.a_kmajor)
        return p.b_kmajor ? launch<T, OUT, true, true>(a, blocks, stream)
                          : launch<T, OUT, true, false>(a, blocks, stream);
    return p.b_kmajor ? launch<T, OUT, false, true>(a, blocks, stream)
                      : launch<T, OUT, false, false>(a, blocks, stream);
}

}  // namespace

// Few output tiles for the main kernel's 256 x 256 tile (under a quarter of
// MI355X's 256 compute units) and a K long enough to split eight ways, on
// operands the direct loads can read whole 16-byte chunks of.
bool hgemm_splitk_eligible(const Problem &p) {
    if (!hgemm_dma_eligible(p)) return false;
    const int64_t big_tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
    return big_tiles < 64 && p.K >= 8 * CK;
}

hipError_t launch_hgemm_splitk(const Problem &p, hipStream_t stream) {
    SplitArgs a{};
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
    a.tiles_m = (p.M + TILE - 1) / TILE;
    a.tiles_n = (p.N + TILE - 1) / TILE;
    a.kper = ((p.K + WAVES * CK - 1) / (WAVES * CK)) * CK;
    a.epi = p.epi;
    const int64_t blocks = a.tiles_m * a.tiles_n * p.batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool bf = p.in == Elem::BF16;
    if (p.out == Elem::F32)
        return bf ? launch_layout<BF16, OUT_F32>(p, a, blocks, stream)
                  : launch_layout<F16, OUT_F32>(p, a, blocks, stream);
    return bf ? launch_layout<BF16, OUT_BF16>(p, a, blocks, stream)
              : launch_layout<F16, OUT_F16>(p, a, blocks, stream);
}

}  // namespace libgemm
