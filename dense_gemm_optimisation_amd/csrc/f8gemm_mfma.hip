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
#include "f8_dma.hpp"

namespace libgemm {
namespace {

using namespace dmatile;

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
            for (int j = 0; j < FN; ++j) fb[j] = frag8(pb, wn * 64 + j * 32, kk, lane);
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = frag8(pa, wm * 64 + i * 32, kk, lane);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mma8<FA, FB, 0>(fb[j], fa[i], acc[i][j], UNIT_SCALE, UNIT_SCALE);
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
    static hipError_t go(const Problem &, F8Args &a, hipStream_t stream) {
        void *args[] = {&a};
        return hipLaunchKernel(
            reinterpret_cast<const void *>(&f8gemm_dma_kernel<FA, FB, OUT, LIBGEMM_F8_WM,
                                                              LIBGEMM_F8_WN, f8_stages<FA, FB>(), false>),
            dim3(static_cast<unsigned>(a.d.grid.count())), dim3(LIBGEMM_F8_WM * LIBGEMM_F8_WN * 64),
            args, 0, stream);
    }
};

// The stream-K launch: its arguments, split and grid, then the fix-up of
// the cut tiles.
struct F8StreamKLaunch {
    F8Args a;
    DmaStreamK sk;
    int64_t grid;
};

template <int FA, int FB, int OUT>
struct LaunchDmaStreamK {
    static hipError_t go(const Problem &, F8StreamKLaunch &l, hipStream_t stream) {
        constexpr int WM = LIBGEMM_F8_WM, WN = LIBGEMM_F8_WN;
        void *args[] = {&l.a, &l.sk};
        const hipError_t e = hipLaunchKernel(
            reinterpret_cast<const void *>(
                &f8gemm_dma_streamk_kernel<FA, FB, OUT, WM, WN, f8_stages<FA, FB>(), false>),
            dim3(static_cast<unsigned>(l.grid)), dim3(WM * WN * 64), args, 0, stream);
        if (e != hipSuccess) return e;
        return launch_dma_streamk_fixup<OUT, WM, WN>(l.a.d, l.sk, l.a.d.grid.count(), stream);
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

namespace {

// The direct-load kernel's arguments; xcds: the tile grid's regrouping per
// die (1 when the work order does it).  The panels count in 16-bit units:
// every extent along K, leading dimension and operand stride is halved (all
// are even here).
F8Args dma_args(const Problem &p, int32_t xcds) {
    F8Args a{};
    a.d = common_args(p, F8_BM, LIBGEMM_F8_GROUP_M);
    a.d.grid.xcds = xcds;
    a.K = p.K;
    a.ka = a.kb = p.K / 2;
    a.d.K = p.K / 2;
    a.d.lda /= 2;
    a.d.ldb /= 2;
    a.d.sA /= 2;
    a.d.sB /= 2;
    return a;
}

}  // namespace

hipError_t launch_f8gemm_dma(const Problem &p, hipStream_t stream) {
    F8Args a = dma_args(p, 8);
    if (a.d.grid.count() > 0x7fffffff) return hipErrorInvalidConfiguration;
    return by_output<LaunchDma>(p, a, stream);
}

bool f8gemm_dma_streamk_eligible(const Problem &p, bool force) {
    return f8gemm_dma_eligible(p) && f8_streamk_worth(f8_tiles(p.M, p.N, p.batch), p.K, force);
}

int64_t f8gemm_dma_streamk_bytes(const Problem &p) {
    return 2 * f8_streamk_split(f8_tiles(p.M, p.N, p.batch), p.K).groups * int64_t(SK_SLOT) * 4;
}

hipError_t launch_f8gemm_dma_streamk(const Problem &p, void *workspace, hipStream_t stream) {
    F8StreamKLaunch l{};
    l.a = dma_args(p, 1);  // the work order itself spreads tiles over the dies
    static_cast<StreamKSplit &>(l.sk) = f8_streamk_split(f8_tiles(p.M, p.N, p.batch), p.K);
    l.sk.partials = static_cast<float *>(workspace);
    l.grid = streamk_grid(l.sk, HGEMM_STREAMK_MAX_GRID);
    if (l.grid == 0) return hipSuccess;
    return by_output<LaunchDmaStreamK>(p, l, stream);
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
