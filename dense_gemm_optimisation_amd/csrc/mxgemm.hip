// Block-scaled (MX) GEMM: the launchers of the direct-load narrow-float
// kernel of f8_dma.hpp with its E8M0 scales switched on (MXFP8, MXFP6,
// MXFP4: "CUDA GEMM 矩阵乘法优化指南", blog.zhenwei.site, section 13.2).
//
// The file is compiled once per element width with LIBGEMM_MX_PART = 0, 1, 2
// (8-, 6- and 4-bit elements), so the parts' kernels build in parallel; part
// 0 also holds the host code.  Without the macro one object holds
// everything.  A and B take formats of one width (E4M3/E5M2, E2M3/E3M2 or
// E2M1): the kernel's stage layout is shared by both operands.
#include "f8_dma.hpp"
#include "gemm_problem.hpp"

#ifndef LIBGEMM_MX_PART
#define LIBGEMM_MX_PART -1
#endif
#define LIBGEMM_MX_HAS(part) (LIBGEMM_MX_PART < 0 || LIBGEMM_MX_PART == (part))

namespace libgemm {

// The launch for one element width (defined in that width's part): one
// workgroup per tile when split is null, else the stream-K schedule `split`
// with its partial tiles at `partials`, then its fix-up.
template <int WIDTH>
hipError_t mx_launch_width(const MxProblem &m, const StreamKSplit *split, float *partials,
                           hipStream_t stream);

namespace {

// The kernel arguments of m.  The panels count in 16-bit units: element
// extents along K, leading dimensions and operand strides times width / 16
// (all whole: multiples of 64 elements).
F8Args mx_args(const MxProblem &m) {
    const Problem &p = m.p;
    const int wa = mx_width(m.fa), wb = mx_width(m.fb);
    F8Args a{};
    DmaArgs &d = a.d;
    d.M = p.M;
    d.N = p.N;
    d.K = p.K * wa / 16;
    d.alpha = p.alpha;
    d.beta = p.beta;
    d.A = static_cast<const uint16_t *>(p.A);
    d.B = static_cast<const uint16_t *>(p.B);
    d.C = p.C;
    d.lda = p.lda * wa / 16;
    d.ldb = p.ldb * wb / 16;
    d.ldc = p.ldc;
    d.sA = p.batch > 1 ? p.sA * wa / 16 : 0;
    d.sB = p.batch > 1 ? p.sB * wb / 16 : 0;
    d.sC = p.batch > 1 ? p.sC : 0;
    d.grid = TileGrid{(p.M + F8_BM - 1) / F8_BM, (p.N + F8_BN - 1) / F8_BN, p.batch,
                      LIBGEMM_F8_GROUP_M, 8};
    d.epi = p.epi;
    a.K = p.K;
    a.ka = p.K * wa / 16;
    a.kb = p.K * wb / 16;
    a.sa = m.sa;
    a.sb = m.sb;
    a.ldsa = m.ldsa;
    a.ldsb = m.ldsb;
    a.ssa = p.batch > 1 ? m.ssa : 0;
    a.ssb = p.batch > 1 ? m.ssb : 0;
    return a;
}

template <int FA, int FB, int OUT>
hipError_t mx_go(const MxProblem &m, const StreamKSplit *split, float *partials,
                 hipStream_t stream) {
    constexpr int WM = LIBGEMM_F8_WM, WN = LIBGEMM_F8_WN;
    F8Args a = mx_args(m);
    if (split == nullptr) {
        void *args[] = {&a};
        return hipLaunchKernel(
            reinterpret_cast<const void *>(
                &f8gemm_dma_kernel<FA, FB, OUT, WM, WN, f8_stages<FA, FB>(), true>),
            dim3(static_cast<unsigned>(a.d.grid.count())), dim3(WM * WN * 64), args, 0, stream);
    }
    a.d.grid.xcds = 1;  // the work order itself spreads tiles over the dies
    DmaStreamK sk{};
    static_cast<StreamKSplit &>(sk) = *split;
    sk.partials = partials;
    const int64_t grid = streamk_grid(sk, HGEMM_STREAMK_MAX_GRID);
    if (grid == 0) return hipSuccess;
    void *args[] = {&a, &sk};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void *>(
            &f8gemm_dma_streamk_kernel<FA, FB, OUT, WM, WN, f8_stages<FA, FB>(), true>),
        dim3(static_cast<unsigned>(grid)), dim3(WM * WN * 64), args, 0, stream);
    if (e != hipSuccess) return e;
    return launch_dma_streamk_fixup<OUT, WM, WN>(a.d, sk, a.d.grid.count(), stream);
}

template <int FA, int FB>
hipError_t mx_out(const MxProblem &m, const StreamKSplit *split, float *partials,
                  hipStream_t stream) {
    if (m.p.out == Elem::F32) return mx_go<FA, FB, OUT_F32>(m, split, partials, stream);
    if (m.p.out == Elem::BF16) return mx_go<FA, FB, OUT_BF16>(m, split, partials, stream);
    return mx_go<FA, FB, OUT_F16>(m, split, partials, stream);
}

}  // namespace

#if LIBGEMM_MX_HAS(0)
template <>
hipError_t mx_launch_width<8>(const MxProblem &m, const StreamKSplit *split, float *partials,
                              hipStream_t stream) {
    if (m.fa == FMT_E4M3)
        return m.fb == FMT_E4M3 ? mx_out<FMT_E4M3, FMT_E4M3>(m, split, partials, stream)
                                : mx_out<FMT_E4M3, FMT_E5M2>(m, split, partials, stream);
    return m.fb == FMT_E4M3 ? mx_out<FMT_E5M2, FMT_E4M3>(m, split, partials, stream)
                            : mx_out<FMT_E5M2, FMT_E5M2>(m, split, partials, stream);
}
#endif
#if LIBGEMM_MX_HAS(1)
template <>
hipError_t mx_launch_width<6>(const MxProblem &m, const StreamKSplit *split, float *partials,
                              hipStream_t stream) {
    if (m.fa == FMT_E2M3)
        return m.fb == FMT_E2M3 ? mx_out<FMT_E2M3, FMT_E2M3>(m, split, partials, stream)
                                : mx_out<FMT_E2M3, FMT_E3M2>(m, split, partials, stream);
    return m.fb == FMT_E2M3 ? mx_out<FMT_E3M2, FMT_E2M3>(m, split, partials, stream)
                            : mx_out<FMT_E3M2, FMT_E3M2>(m, split, partials, stream);
}
#endif
#if LIBGEMM_MX_HAS(2)
template <>
hipError_t mx_launch_width<4>(const MxProblem &m, const StreamKSplit *split, float *partials,
                              hipStream_t stream) {
    return mx_out<FMT_E2M1, FMT_E2M1>(m, split, partials, stream);
}
#endif

#if LIBGEMM_MX_PART <= 0
namespace {

hipError_t mx_launch(const MxProblem &m, const StreamKSplit *split, float *partials,
                     hipStream_t stream) {
    const int w = mx_width(m.fa);
    if (w != mx_width(m.fb)) return hipErrorInvalidValue;
    if (f8_tiles(m.p.M, m.p.N, m.p.batch) > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (w == 8) return mx_launch_width<8>(m, split, partials, stream);
    if (w == 6) return mx_launch_width<6>(m, split, partials, stream);
    return mx_launch_width<4>(m, split, partials, stream);
}

}  // namespace

hipError_t launch_mxgemm(const MxProblem &m, hipStream_t stream) {
    return mx_launch(m, nullptr, nullptr, stream);
}

bool mxgemm_streamk_eligible(const MxProblem &m, bool force) {
    return f8_streamk_worth(f8_tiles(m.p.M, m.p.N, m.p.batch), m.p.K, force);
}

int64_t mxgemm_streamk_bytes(const MxProblem &m) {
    return 2 * f8_streamk_split(f8_tiles(m.p.M, m.p.N, m.p.batch), m.p.K).groups *
           int64_t(SK_SLOT) * 4;
}

hipError_t launch_mxgemm_streamk(const MxProblem &m, void *workspace, hipStream_t stream) {
    const StreamKSplit split = f8_streamk_split(f8_tiles(m.p.M, m.p.N, m.p.batch), m.p.K);
    return mx_launch(m, &split, static_cast<float *>(workspace), stream);
}
#endif

}  // namespace libgemm
