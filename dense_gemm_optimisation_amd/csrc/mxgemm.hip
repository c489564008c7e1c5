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

// The launch for one element width (defined in that width's part).
template <int WIDTH>
hipError_t mx_launch_width(const MxProblem &m, hipStream_t stream);

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
hipError_t mx_go(const MxProblem &m, hipStream_t stream) {
    F8Args a = mx_args(m);
    void *args[] = {&a};
    return hipLaunchKernel(
        reinterpret_cast<const void *>(&f8gemm_dma_kernel<FA, FB, OUT, LIBGEMM_F8_WM, LIBGEMM_F8_WN,
                                                          LIBGEMM_F8_STAGES, true>),
        dim3(static_cast<unsigned>(a.d.grid.count())), dim3(LIBGEMM_F8_WM * LIBGEMM_F8_WN * 64), args,
        0, stream);
}

template <int FA, int FB>
hipError_t mx_out(const MxProblem &m, hipStream_t stream) {
    if (m.p.out == Elem::F32) return mx_go<FA, FB, OUT_F32>(m, stream);
    if (m.p.out == Elem::BF16) return mx_go<FA, FB, OUT_BF16>(m, stream);
    return mx_go<FA, FB, OUT_F16>(m, stream);
}

}  // namespace

#if LIBGEMM_MX_HAS(0)
template <>
hipError_t mx_launch_width<8>(const MxProblem &m, hipStream_t stream) {
    if (m.fa == FMT_E4M3)
        return m.fb == FMT_E4M3 ? mx_out<FMT_E4M3, FMT_E4M3>(m, stream)
                                : mx_out<FMT_E4M3, FMT_E5M2>(m, stream);
    return m.fb == FMT_E4M3 ? mx_out<FMT_E5M2, FMT_E4M3>(m, stream)
                            : mx_out<FMT_E5M2, FMT_E5M2>(m, stream);
}
#endif
#if LIBGEMM_MX_HAS(1)
template <>
hipError_t mx_launch_width<6>(const MxProblem &m, hipStream_t stream) {
    if (m.fa == FMT_E2M3)
        return m.fb == FMT_E2M3 ? mx_out<FMT_E2M3, FMT_E2M3>(m, stream)
                                : mx_out<FMT_E2M3, FMT_E3M2>(m, stream);
    return m.fb == FMT_E2M3 ? mx_out<FMT_E3M2, FMT_E2M3>(m, stream)
                            : mx_out<FMT_E3M2, FMT_E3M2>(m, stream);
}
#endif
#if LIBGEMM_MX_HAS(2)
template <>
hipError_t mx_launch_width<4>(const MxProblem &m, hipStream_t stream) {
    return mx_out<FMT_E2M1, FMT_E2M1>(m, stream);
}
#endif

#if LIBGEMM_MX_PART <= 0
hipError_t launch_mxgemm(const MxProblem &m, hipStream_t stream) {
    const int w = mx_width(m.fa);
    if (w != mx_width(m.fb)) return hipErrorInvalidValue;
    const int64_t tiles = ((m.p.M + F8_BM - 1) / F8_BM) * ((m.p.N + F8_BN - 1) / F8_BN) * m.p.batch;
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (w == 8) return mx_launch_width<8>(m, stream);
    if (w == 6) return mx_launch_width<6>(m, stream);
    return mx_launch_width<4>(m, stream);
}
#endif

}  // namespace libgemm
