// The canonical problem the host layer hands to the kernels, and the kernel
// launch entry points.  The host layer has already validated every argument
// and rewritten a column-major C as the row-major C^T = B^T A^T, so every
// kernel writes a row-major C.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "epilogue.hpp"
#include "streamk_schedule.hpp"

namespace libgemm {

// E4M3 and E5M2 are the OCP 8-bit floating-point formats (1 sign bit; 4
// exponent bits with bias 7 and 3 fraction bits, no infinities; 5 exponent
// bits with bias 15 and 2 fraction bits, IEEE-style infinities and NaNs).
enum class Elem : int { F32 = 0, BF16 = 1, F16 = 2, E4M3 = 3, E5M2 = 4 };

struct Problem {
    int64_t M, N, K;
    float alpha, beta;
    // a_kmajor: A(i, k) at A[i*lda + k] (K contiguous); else at A[k*lda + i].
    const void *A;
    int64_t lda;
    bool a_kmajor;
    // b_kmajor: B(k, j) at B[j*ldb + k] (K contiguous); else at B[k*ldb + j].
    const void *B;
    int64_t ldb;
    bool b_kmajor;
    // C(i, j) at C[i*ldc + j].
    void *C;
    int64_t ldc;
    int64_t batch, sA, sB, sC;  // batch count and per-batch strides (elements)
    Elem in, in_b, out;         // types of A, of B (differs from A's only for 8-bit), of C
    Epilogue epi;               // bias and activation applied before the store
    // packed: A and B are zero-padded copies whose contiguous extents are
    // whole 16-byte chunks (K itself padded when it is contiguous), so the
    // direct-load kernels may read whole chunks past M, N or K; span_a and
    // span_b are then the elements of one slice of each copy (0 otherwise:
    // the operand's own extent).
    bool packed = false;
    int64_t span_a = 0, span_b = 0;
};

// Element size in bytes.
inline int elem_bytes(Elem e) {
    return e == Elem::F32 ? 4 : (e == Elem::BF16 || e == Elem::F16) ? 2 : 1;
}
inline bool elem_is_8bit(Elem e) { return e == Elem::E4M3 || e == Elem::E5M2; }

// True when a pointer, leading dimension and batch stride allow 16-byte
// vector access to every row of the operand.
inline bool vec16_ok(const void *p, int64_t ld, int64_t stride, int esize) {
    const int64_t per = 16 / esize;
    return (reinterpret_cast<uintptr_t>(p) % 16) == 0 && ld % per == 0 && stride % per == 0;
}

// Elements of one slice of operand A (B) that the kernels may read: the
// matrix's own extent, or the whole padded copy of a packed problem.
inline int64_t operand_span_a(const Problem &p) {
    if (p.span_a) return p.span_a;
    return p.a_kmajor ? (p.M - 1) * p.lda + p.K : (p.K - 1) * p.lda + p.M;
}
inline int64_t operand_span_b(const Problem &p) {
    if (p.span_b) return p.span_b;
    return p.b_kmajor ? (p.N - 1) * p.ldb + p.K : (p.K - 1) * p.ldb + p.N;
}

// An operand copy for a packed problem: `outer` rows of `inner` contiguous
// elements of `esize` bytes (leading dimension ld, `batch` slices `stride`
// apart, stride 0 = one shared slice) become outer_p x inner_p, zero-padded,
// inner_p * esize a multiple of 16, slices outer_p * inner_p apart.
struct PackSpec {
    const void *src;
    int64_t outer, inner, ld, stride, batch;
    int64_t outer_p, inner_p;
    int esize;
};
int64_t packed_bytes(const PackSpec &s);
hipError_t launch_pack(const PackSpec &s, void *dst, hipStream_t stream);

// fp32 operands split into bf16 pieces for the three-product fp32 GEMM
// (split_bf16.hip): Kp = K rounded up to a multiple of 8; a copy holds
// [batch][rows][3 Kp] bf16, pieces (hi, hi, lo) for A and (hi, lo, hi) for
// B, each zero-padded from K to Kp; split_bytes is its size rounded up to
// 256 bytes.  Source element (r, k): src[b*stride + r*ld + k] when kmajor,
// else src[b*stride + k*ld + r].
int64_t split_kp(int64_t K);
int64_t split_bytes(int64_t rows, int64_t K, int64_t batch);
hipError_t launch_split_a(const float *A, int64_t lda, int64_t sA, bool kmajor, int64_t M,
                          int64_t K, int64_t batch, uint16_t *dst, hipStream_t stream);
hipError_t launch_split_b(const float *B, int64_t ldb, int64_t sB, bool kmajor, int64_t N,
                          int64_t K, int64_t batch, uint16_t *dst, hipStream_t stream);

// Address of this library's scratch array on the device `stream` belongs to
// (looked up once per device; see noalloc.hip).
hipError_t scratch_address(hipStream_t stream, void **ptr);

// Kernel launchers; each returns the launch status.
hipError_t launch_sgemm(const Problem &p, hipStream_t stream);       // fp32 on the vector ALUs
hipError_t launch_sgemm_mfma(const Problem &p, hipStream_t stream);  // fp32 on the matrix cores
// fp32 on the matrix cores with direct global->LDS loads; only for problems
// where sgemm_dma_eligible() holds (aligned operands, extents multiple of 4).
bool sgemm_dma_eligible(const Problem &p);
hipError_t launch_sgemm_dma(const Problem &p, hipStream_t stream);
// fp32 split-K inside a workgroup, for problems with few output tiles
// (sgemm_splitk_eligible()).
bool sgemm_splitk_eligible(const Problem &p);
hipError_t launch_sgemm_splitk(const Problem &p, hipStream_t stream);
// The general fp32 kernel's stream-K schedule, through the same workspace as
// the 16-bit kernels' (two 128 x 128 fp32 partial tiles per workgroup, four
// workgroups per compute unit: the same bytes); only where
// sgemm_streamk_eligible() holds.
constexpr int64_t SGEMM_STREAMK_MAX_GRID = 1024;
bool sgemm_streamk_eligible(const Problem &p, bool force = false);
hipError_t launch_sgemm_streamk(const Problem &p, void *workspace, hipStream_t stream);
// Workspace bytes launch_sgemm_streamk and launch_sgemm_dma_streamk use for
// p (their partial tiles).
int64_t sgemm_streamk_bytes(const Problem &p);
// The same schedule on the direct-load k loop, for problems where both
// sgemm_dma_eligible() and sgemm_streamk_eligible() hold.
bool sgemm_dma_streamk_eligible(const Problem &p, bool force = false);
hipError_t launch_sgemm_dma_streamk(const Problem &p, void *workspace, hipStream_t stream);
hipError_t launch_hgemm(const Problem &p, hipStream_t stream);  // bf16/fp16 on MFMA, any shape
// The *_streamk_eligible functions check whether a problem can run on the
// schedule and, unless `force`, whether the cost model says it pays.
// The same kernel's stream-K schedule, which cuts tiles across workgroups
// through a caller-provided workspace of hgemm_streamk_workspace_bytes()
// (two fp32 partial 256 x 256 tiles per workgroup); only where
// hgemm_streamk_eligible() holds.
constexpr int64_t HGEMM_STREAMK_MAX_GRID = 256;
constexpr int64_t hgemm_streamk_workspace_bytes() {
    return 2 * HGEMM_STREAMK_MAX_GRID * 256 * 256 * 4;
}
static_assert(2 * 1024 * 128 * 128 * 4 == hgemm_streamk_workspace_bytes(),
              "the fp32 stream-K schedule (1024 workgroups, 128 x 128 tiles) fits the workspace");
bool hgemm_streamk_eligible(const Problem &p, bool force = false);
hipError_t launch_hgemm_streamk(const Problem &p, void *workspace, hipStream_t stream);
// Workspace bytes launch_hgemm_streamk uses for p (its partial tiles).
int64_t hgemm_streamk_bytes(const Problem &p);
// bf16/fp16 on MFMA with direct global->LDS loads; only for problems where
// hgemm_dma_eligible() holds (aligned operands, extents multiple of 8).
bool hgemm_dma_eligible(const Problem &p);
hipError_t launch_hgemm_dma(const Problem &p, hipStream_t stream);
// Its stream-K schedule, through the same workspace as the general kernel's
// (hgemm_streamk_workspace_bytes()); only where hgemm_dma_streamk_eligible()
// holds.
bool hgemm_dma_streamk_eligible(const Problem &p, bool force = false);
hipError_t launch_hgemm_dma_streamk(const Problem &p, void *workspace, hipStream_t stream);
// Workspace bytes launch_hgemm_dma_streamk uses for p (its partial tiles).
int64_t hgemm_dma_streamk_bytes(const Problem &p);
// bf16/fp16 split-K inside a workgroup, for problems with few output tiles
// and a long K (hgemm_splitk_eligible()).
bool hgemm_splitk_eligible(const Problem &p);
hipError_t launch_hgemm_splitk(const Problem &p, hipStream_t stream);
// Any input type, at most 16 rows of C: B streamed at HBM rate, split-K
// inside a workgroup (skinny_eligible()).
bool skinny_eligible(const Problem &p);
hipError_t launch_skinny(const Problem &p, hipStream_t stream);
// The same problems with an N-contiguous 16-bit B, split over K across
// workgroups through a workspace of skinny_sk_bytes(p) (partial blocks), then
// reduced in fixed order by a second kernel (skinny_sk_eligible()).
bool skinny_sk_eligible(const Problem &p);
int64_t skinny_sk_bytes(const Problem &p);
hipError_t launch_skinny_sk(const Problem &p, void *workspace, hipStream_t stream);
// 8-bit floats (E4M3/E5M2) on the scaled 8-bit matrix instructions: the
// direct-load kernel for K-contiguous aligned operands (f8gemm_dma_eligible())
// and a general kernel for any order, alignment and shape.
bool f8gemm_dma_eligible(const Problem &p);
hipError_t launch_f8gemm_dma(const Problem &p, hipStream_t stream);
// The direct-load kernel's stream-K schedule, through the same workspace as
// the 16-bit kernels' (hgemm_streamk_workspace_bytes()); only where
// f8gemm_dma_streamk_eligible() holds.
bool f8gemm_dma_streamk_eligible(const Problem &p, bool force = false);
// Workspace bytes launch_f8gemm_dma_streamk uses for p (its partial tiles).
int64_t f8gemm_dma_streamk_bytes(const Problem &p);
hipError_t launch_f8gemm_dma_streamk(const Problem &p, void *workspace, hipStream_t stream);
hipError_t launch_f8gemm(const Problem &p, hipStream_t stream);
hipError_t launch_scale(const Problem &p, hipStream_t stream);  // C <- beta*C only

// A block-scaled (MX) problem.  p holds the extents, scalars, C and the batch
// with A and B K-contiguous (A(i, k) at element i*lda + k, B(k, j) at
// element j*ldb + k of their packed element streams; lda, ldb, sA and sB in
// elements); fa and fb are the matrix instruction's format codes (0 E4M3,
// 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1); A(i, k)'s E8M0 scale is
// sa[i*ldsa + k/32] (+ ssa per batch entry, bytes), B(k, j)'s sb[j*ldsb + k/32].
struct MxProblem {
    Problem p;
    int fa, fb;
    const uint8_t *sa, *sb;
    int64_t ldsa, ldsb, ssa, ssb;
};
// Bits per element of a format code.
inline int mx_width(int fmt) { return fmt == 4 ? 4 : (fmt == 2 || fmt == 3) ? 6 : 8; }
// The direct-load 8-bit kernel with scales; needs K a multiple of 64, lda,
// ldb, sA, sB multiples of 64 elements, 16-byte aligned A and B, ldsa and
// ldsb multiples of 4 of at least 4*ceil(K/128) bytes, 4-byte aligned
// scales, and fa, fb of one width (the api checks all of it).
hipError_t launch_mxgemm(const MxProblem &m, hipStream_t stream);
// Its stream-K schedule (the 8-bit kernel's split: 256 x 256 tiles, 128-k
// steps) through a workspace of mxgemm_streamk_bytes(m) bytes, where
// mxgemm_streamk_eligible() holds (some tiles left over after the whole
// waves, and worth the exchange unless forced).
bool mxgemm_streamk_eligible(const MxProblem &m, bool force = false);
int64_t mxgemm_streamk_bytes(const MxProblem &m);
hipError_t launch_mxgemm_streamk(const MxProblem &m, void *workspace, hipStream_t stream);

}  // namespace libgemm
