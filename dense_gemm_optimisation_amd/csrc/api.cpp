// C ABI of libgemm: argument validation, canonicalisation and dispatch.
//
// Every check runs before any HIP call, so an invalid call has no effect.
// A column-major C is handled by computing its transpose, which is row-major:
// C^T = B^T A^T (the transpose identity used with the column-major BLAS call
// in section 7.1 of "第4章：经典算子实现 —— GEMM", aiinfra.vidrealm.tech).
// The kernels therefore only ever write a row-major C.
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "gemm_problem.hpp"

namespace libgemm {
// The copies of both operands of a packed plan in one launch (pack.hip).
hipError_t launch_pack2(const PackSpec &sa, void *dst_a, const PackSpec &sb, void *dst_b,
                        hipStream_t stream);
}  // namespace libgemm
#include "libgemm.h"

using namespace libgemm;

namespace {

bool valid_order(int o) { return o == GEMM_ROW_MAJOR || o == GEMM_COL_MAJOR; }

// Elements spanned by one rows x cols matrix stored with leading dimension ld.
int64_t span(int64_t rows, int64_t cols, int order, int64_t ld) {
    if (rows == 0 || cols == 0) return 0;
    const int64_t outer = order == GEMM_ROW_MAJOR ? rows : cols;
    const int64_t inner = order == GEMM_ROW_MAJOR ? cols : rows;
    return (outer - 1) * ld + inner;
}

// Byte range [lo, hi) that a batched operand touches.
struct Range {
    uintptr_t lo, hi;
};

Range range_of(const void *p, int64_t span_elems, int64_t batch, int64_t stride, int esize) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    const int64_t elems = span_elems == 0 ? 0 : (batch - 1) * stride + span_elems;
    return {lo, lo + static_cast<uintptr_t>(elems) * static_cast<uintptr_t>(esize)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

// Product of non-negative dimensions overflowing int64 (or the 2^31 grid).
bool too_big(int64_t a, int64_t b) { return a != 0 && b > INT64_MAX / a; }

// Kernel-choice overrides for testing (gemm_test_switches): one atomic word
// for the whole process, read on every call.
std::atomic<int> g_switches{0};
bool force_general() { return g_switches.load(std::memory_order_relaxed) & GEMM_TEST_FORCE_GENERAL; }
bool no_splitk() { return g_switches.load(std::memory_order_relaxed) & GEMM_TEST_NO_SPLITK; }
bool force_streamk() { return g_switches.load(std::memory_order_relaxed) & GEMM_TEST_FORCE_STREAMK; }
bool f32_valu() { return g_switches.load(std::memory_order_relaxed) & GEMM_TEST_F32_VALU; }

// The kernels a call can end in.
enum class Kernel {
    None,        // empty problem: nothing to do
    Scale,       // C <- beta*C only
    SgemmValu,   // fp32, vector ALUs (opt-in)
    SgemmMfma,   // fp32, matrix cores, any shape
    SgemmDma,    // fp32, matrix cores, direct loads
    SgemmSplitk, // fp32, few tiles: split-K inside a workgroup
    Skinny,      // any type, at most 16 rows of C
    HgemmMfma,   // bf16/fp16, any shape
    HgemmDma,    // bf16/fp16, direct loads
    HgemmSplitk, // bf16/fp16, few tiles: split-K inside a workgroup
    F8Mfma,      // 8-bit floats, any shape and order
    F8Dma,       // 8-bit floats, K-contiguous aligned operands, direct loads
    HgemmStreamK,  // bf16/fp16 general kernel on the stream-K schedule (workspace)
    HgemmDmaStreamK,  // bf16/fp16 direct-load kernel on the stream-K schedule (workspace)
    SgemmStreamK,  // fp32 general kernel on the stream-K schedule (workspace)
    SgemmDmaStreamK,  // fp32 direct-load kernel on the stream-K schedule (workspace)
    // operands copied into aligned, zero-padded copies in the workspace first
    HgemmPackDma,         // then the bf16/fp16 direct-load kernel
    HgemmPackDmaStreamK,  // then its stream-K schedule
    SgemmPackDma,         // then the fp32 direct-load kernel
    SgemmPackDmaStreamK,  // then its stream-K schedule
    Mx,                   // block-scaled narrow floats (gemm_mx), direct loads
    F8DmaStreamK,         // 8-bit direct-load kernel on the stream-K schedule (workspace)
    MxStreamK,            // block-scaled kernel on the stream-K schedule (workspace)
    SkinnySplitK,         // at most 16 rows, N-contiguous B: split-K across workgroups (workspace)
};

bool is_packed(Kernel k) {
    return k == Kernel::HgemmPackDma || k == Kernel::HgemmPackDmaStreamK ||
           k == Kernel::SgemmPackDma || k == Kernel::SgemmPackDmaStreamK;
}

const char *kernel_name(Kernel k) {
    switch (k) {
    case Kernel::None: return "";
    case Kernel::Scale: return "scale";
    case Kernel::SgemmValu: return "sgemm_valu";
    case Kernel::SgemmMfma: return "sgemm_mfma";
    case Kernel::SgemmDma: return "sgemm_mfma_dma";
    case Kernel::SgemmSplitk: return "sgemm_splitk";
    case Kernel::Skinny: return "gemm_skinny";
    case Kernel::HgemmMfma: return "hgemm_mfma";
    case Kernel::HgemmDma: return "hgemm_mfma_dma";
    case Kernel::HgemmSplitk: return "hgemm_splitk";
    case Kernel::F8Mfma: return "f8gemm_mfma";
    case Kernel::F8Dma: return "f8gemm_mfma_dma";
    case Kernel::HgemmStreamK: return "hgemm_mfma_streamk";
    case Kernel::HgemmDmaStreamK: return "hgemm_mfma_dma_streamk";
    case Kernel::SgemmStreamK: return "sgemm_mfma_streamk";
    case Kernel::SgemmDmaStreamK: return "sgemm_mfma_dma_streamk";
    case Kernel::HgemmPackDma: return "hgemm_mfma_dma_packed";
    case Kernel::HgemmPackDmaStreamK: return "hgemm_mfma_dma_streamk_packed";
    case Kernel::SgemmPackDma: return "sgemm_mfma_dma_packed";
    case Kernel::SgemmPackDmaStreamK: return "sgemm_mfma_dma_streamk_packed";
    case Kernel::Mx: return "mxgemm_mfma_dma";
    case Kernel::F8DmaStreamK: return "f8gemm_mfma_dma_streamk";
    case Kernel::MxStreamK: return "mxgemm_mfma_dma_streamk";
    case Kernel::SkinnySplitK: return "gemm_skinny_splitk";
    }
    return "";
}

// Kernel choice for a canonical problem that reads A and B: the skinny
// kernel for at most 16 rows of C, split-K for other few-tile problems, the
// direct-load kernel for aligned operands, the register-staged kernel for
// everything else.
Kernel choose(const Problem &p, bool valu) {
    const bool splits = !force_general() && !no_splitk();
    if (elem_is_8bit(p.in))
        return !force_general() && f8gemm_dma_eligible(p) ? Kernel::F8Dma : Kernel::F8Mfma;
    if (p.in == Elem::F32) {
        if (valu || f32_valu()) return Kernel::SgemmValu;
        if (force_general()) return Kernel::SgemmMfma;
        if (splits && skinny_eligible(p)) return Kernel::Skinny;
        if (splits && sgemm_splitk_eligible(p)) return Kernel::SgemmSplitk;
        return sgemm_dma_eligible(p) ? Kernel::SgemmDma : Kernel::SgemmMfma;
    }
    if (splits && skinny_eligible(p)) return Kernel::Skinny;
    if (splits && hgemm_splitk_eligible(p)) return Kernel::HgemmSplitk;
    if (!force_general() && hgemm_dma_eligible(p)) return Kernel::HgemmDma;
    return Kernel::HgemmMfma;
}

hipError_t launch(Kernel k, const Problem &p, hipStream_t stream) {
    switch (k) {
    case Kernel::None: return hipSuccess;
    case Kernel::Scale: return launch_scale(p, stream);
    case Kernel::SgemmValu: return launch_sgemm(p, stream);
    case Kernel::SgemmMfma: return launch_sgemm_mfma(p, stream);
    case Kernel::SgemmDma: return launch_sgemm_dma(p, stream);
    case Kernel::SgemmSplitk: return launch_sgemm_splitk(p, stream);
    case Kernel::Skinny: return launch_skinny(p, stream);
    case Kernel::HgemmMfma: return launch_hgemm(p, stream);
    case Kernel::HgemmDma: return launch_hgemm_dma(p, stream);
    case Kernel::HgemmSplitk: return launch_hgemm_splitk(p, stream);
    case Kernel::F8Mfma: return launch_f8gemm(p, stream);
    case Kernel::F8Dma: return launch_f8gemm_dma(p, stream);
    case Kernel::HgemmStreamK:
    case Kernel::HgemmDmaStreamK:
    case Kernel::SgemmStreamK:
    case Kernel::SgemmDmaStreamK:
    case Kernel::HgemmPackDma:
    case Kernel::HgemmPackDmaStreamK:
    case Kernel::SgemmPackDma:
    case Kernel::SgemmPackDmaStreamK: return hipErrorInvalidValue;  // need the workspace: run()
    case Kernel::Mx:
    case Kernel::MxStreamK: return hipErrorInvalidValue;  // needs the scales: gemm_mx
    case Kernel::F8DmaStreamK: return hipErrorInvalidValue;  // needs the workspace: run()
    case Kernel::SkinnySplitK: return hipErrorInvalidValue;  // needs the workspace: run()
    }
    return hipErrorInvalidValue;
}

// Validates a call and builds its canonical problem and kernel choice.  No
// HIP call is made.  `in` is A's type and `in_b` B's (they differ only for
// 8-bit inputs); a bias has A's type.
gemm_status_t plan(Elem in, Elem in_b, Elem out, int64_t M, int64_t N, int64_t K, float alpha,
                   const void *A, int64_t lda, int orderA, const void *B, int64_t ldb, int orderB,
                   float beta, void *C, int64_t ldc, int orderC, int64_t batch, int64_t strideA,
                   int64_t strideB, int64_t strideC, const void *bias, int64_t strideBias, int act,
                   Problem &p, Kernel &kernel, bool valu = false) {
    kernel = Kernel::None;
    // ---- argument checks (no HIP call before this block is done)
    if (M < 0 || N < 0 || K < 0 || batch < 0) return GEMM_ERR_INVALID_ARG;
    if (strideA < 0 || strideB < 0 || strideC < 0 || strideBias < 0) return GEMM_ERR_INVALID_ARG;
    if (act != GEMM_ACT_NONE && act != GEMM_ACT_RELU && act != GEMM_ACT_GELU)
        return GEMM_ERR_INVALID_ARG;
    if (!valid_order(orderA) || !valid_order(orderB) || !valid_order(orderC))
        return GEMM_ERR_INVALID_ARG;
    auto min_ld = [](int order, int64_t rows, int64_t cols) {
        const int64_t inner = order == GEMM_ROW_MAJOR ? cols : rows;
        return inner > 1 ? inner : int64_t(1);
    };
    if (lda < min_ld(orderA, M, K) || ldb < min_ld(orderB, K, N) || ldc < min_ld(orderC, M, N))
        return GEMM_ERR_INVALID_ARG;
    if (too_big(M, N) || too_big(M * N, batch) || too_big(M, K) || too_big(K, N))
        return GEMM_ERR_INVALID_ARG;

    if (M == 0 || N == 0 || batch == 0) return GEMM_OK;  // kernel stays None

    const bool reads_ab = K > 0 && alpha != 0.0f;
    const int ein = elem_bytes(in), ein_b = elem_bytes(in_b), eout = elem_bytes(out);
    const int64_t span_a = span(M, K, orderA, lda);
    const int64_t span_b = span(K, N, orderB, ldb);
    const int64_t span_c = span(M, N, orderC, ldc);
    if (C == nullptr) return GEMM_ERR_INVALID_ARG;
    if (reads_ab && (A == nullptr || B == nullptr)) return GEMM_ERR_INVALID_ARG;
    // every pointer at a multiple of its element size
    auto misaligned = [](const void *x, int e) { return reinterpret_cast<uintptr_t>(x) % e != 0; };
    if (misaligned(C, eout) || (reads_ab && (misaligned(A, ein) || misaligned(B, ein_b))) ||
        (bias != nullptr && misaligned(bias, ein)))
        return GEMM_ERR_INVALID_ARG;
    if (batch > 1 && strideC < span_c) return GEMM_ERR_INVALID_ARG;  // C slices overlap
    if (too_big(batch - 1, strideC) || too_big(batch - 1, strideA) || too_big(batch - 1, strideB) ||
        too_big(batch - 1, strideBias))
        return GEMM_ERR_INVALID_ARG;
    const Range rc = range_of(C, span_c, batch, strideC, eout);
    if (bias != nullptr && overlap(rc, range_of(bias, N, batch, strideBias, ein)))
        return GEMM_ERR_INVALID_ARG;
    if (reads_ab) {
        if (overlap(rc, range_of(A, span_a, batch, strideA, ein)) ||
            overlap(rc, range_of(B, span_b, batch, strideB, ein_b)))
            return GEMM_ERR_INVALID_ARG;
    }

    // ---- canonical problem: row-major C
    p = Problem{};
    p.K = K;
    p.alpha = alpha;
    p.beta = beta;
    p.C = C;
    p.ldc = ldc;
    p.batch = batch;
    p.sC = strideC;
    p.out = out;
    // the bias runs along the caller's columns: along the kernel's rows when
    // C is computed transposed
    p.epi.bias = bias;
    p.epi.bias_stride = batch > 1 ? strideBias : 0;
    p.epi.per_row = orderC == GEMM_COL_MAJOR;
    p.epi.bias_type = static_cast<int>(in);
    p.epi.act = act;
    if (orderC == GEMM_ROW_MAJOR) {
        p.M = M;
        p.N = N;
        p.in = in;
        p.in_b = in_b;
        p.A = A;
        p.lda = lda;
        p.a_kmajor = orderA == GEMM_ROW_MAJOR;
        p.sA = strideA;
        p.B = B;
        p.ldb = ldb;
        p.b_kmajor = orderB == GEMM_COL_MAJOR;
        p.sB = strideB;
    } else {
        // C^T (N x M, row-major) = B^T (N x K) * A^T (K x M).
        p.M = N;
        p.N = M;
        p.in = in_b;
        p.in_b = in;
        p.A = B;
        p.lda = ldb;
        p.a_kmajor = orderB == GEMM_COL_MAJOR;
        p.sA = strideB;
        p.B = A;
        p.ldb = lda;
        p.b_kmajor = orderA == GEMM_ROW_MAJOR;
        p.sB = strideA;
    }

    kernel = reads_ab ? choose(p, valu) : Kernel::Scale;
    return GEMM_OK;
}

// What a workspace call runs: the kernel, the problem it runs on (a packed
// copy of the canonical problem, or that problem itself), the operand copies
// to make first and where everything sits in the workspace.
struct WsPlan {
    Kernel k = Kernel::None;
    Problem q;
    PackSpec pa{}, pb{};
    int64_t off_a = 0, off_b = 0;  // byte offsets of the copies (partial tiles at 0)
    int64_t used = 0;              // workspace bytes the plan touches
    // the last few columns of a packed problem, run as a problem of their
    // own after q (kt None when there is no such split)
    Kernel kt = Kernel::None;
    Problem qt;
};

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Copy of operand X (rows `rows` x cols `cols` of the canonical problem, K
// contiguous when kmajor) for a packed problem with K padded to kp.
PackSpec pack_spec(const void *x, int64_t ld, int64_t stride, int64_t batch, bool kmajor,
                   int64_t mn, int64_t K, int64_t kp, int esize) {
    const int64_t v = 16 / esize;
    PackSpec s{};
    s.src = x;
    s.ld = ld;
    s.stride = batch > 1 ? stride : 0;
    s.batch = batch;
    s.esize = esize;
    if (kmajor) {  // mn rows of K contiguous elements
        s.outer = mn;
        s.inner = K;
        s.outer_p = mn;
        s.inner_p = kp;
    } else {  // K rows of mn contiguous elements
        s.outer = K;
        s.inner = mn;
        s.outer_p = kp;
        s.inner_p = round_up(mn, v);
    }
    return s;
}

// The canonical problem p with its operands replaced by packed copies at
// `a` and `b` (device addresses inside the workspace).
Problem packed_problem(const Problem &p, const PackSpec &sa, const PackSpec &sb, const void *a,
                       const void *b, int64_t kp) {
    Problem q = p;
    q.packed = true;
    q.K = kp;
    q.A = a;
    q.lda = sa.inner_p;
    q.sA = sa.stride == 0 ? 0 : sa.outer_p * sa.inner_p;
    q.span_a = sa.outer_p * sa.inner_p;
    q.B = b;
    q.ldb = sb.inner_p;
    q.sB = sb.stride == 0 ? 0 : sb.outer_p * sb.inner_p;
    q.span_b = sb.outer_p * sb.inner_p;
    return q;
}

// Unaligned operands of a problem big enough to fill the chip (at least 64
// tiles of 256 x 256 for 16-bit inputs, where smaller problems go to the
// split-K and stream-K kernels, or 160 tiles of 128 x 128 for fp32) are
// copied into the workspace so the direct-load kernels can run: the copy
// reads and writes each operand once at HBM rate, against a general kernel
// that runs two to three times slower than the direct-load one.  Returns
// false when the copies (and the partial tiles of a stream-K schedule) do not
// fit the workspace or the problem does not qualify.
bool plan_packed(const Problem &p, Kernel k, const void *workspace, size_t bytes, bool force,
                 WsPlan &w) {
    const bool h16 = k == Kernel::HgemmMfma || k == Kernel::HgemmStreamK;
    const bool f32 = k == Kernel::SgemmMfma;
    if (!h16 && !f32) return false;
    const int esize = elem_bytes(p.in);
    const int64_t tile = h16 ? 256 : 128;
    const int64_t tiles = ((p.M + tile - 1) / tile) * ((p.N + tile - 1) / tile) * p.batch;
    if (tiles < (h16 ? 64 : 160)) return false;
    const int64_t kp = round_up(p.K, 16 / esize);
    const PackSpec sa = pack_spec(p.A, p.lda, p.sA, p.batch, p.a_kmajor, p.M, p.K, kp, esize);
    const PackSpec sb = pack_spec(p.B, p.ldb, p.sB, p.batch, p.b_kmajor, p.N, p.K, kp, esize);
    // the copy kernel addresses a source slice with 32-bit byte offsets
    const int64_t limit = (int64_t(1) << 31) - 64;
    if (((sa.outer - 1) * sa.ld + sa.inner) * esize >= limit ||
        ((sb.outer - 1) * sb.ld + sb.inner) * esize >= limit)
        return false;
    const int64_t bytes_a = round_up(packed_bytes(sa), 256), bytes_b = round_up(packed_bytes(sb), 256);
    // where the copies go once the partial-tile area is known
    auto place = [&](int64_t partials, Kernel kk) {
        if (partials + bytes_a + bytes_b > static_cast<int64_t>(bytes)) return false;
        const char *ws = static_cast<const char *>(workspace);
        w.k = kk;
        w.pa = sa;
        w.pb = sb;
        w.off_a = partials;
        w.off_b = partials + bytes_a;
        w.used = w.off_b + bytes_b;
        w.q = packed_problem(p, sa, sb, ws + w.off_a, ws + w.off_b, kp);
        return true;
    };
    if (!place(0, h16 ? Kernel::HgemmPackDma : Kernel::SgemmPackDma)) return false;
    if (!(h16 ? hgemm_dma_eligible(w.q) : sgemm_dma_eligible(w.q))) return false;
    // A last tile column with at most TAIL_COLS columns (N = 4097 leaves one)
    // would cost the direct-load kernel a whole wave of tiles for a sliver of
    // C; those columns run instead as a problem of their own on the packed
    // copies, after the main part, when that problem goes to a split-K
    // kernel (32 x 32 tiles, K split inside the workgroup).  No fused
    // epilogue: the workspace entry points have none.
    constexpr int64_t TAIL_COLS = 32;
    auto split_tail = [&](WsPlan &x) {
        const int64_t nt = x.q.N % tile;
        if (nt == 0 || nt > TAIL_COLS || x.q.N < tile || x.q.epi.active()) return false;
        Problem qt = x.q;
        const int64_t nm = x.q.N - nt;
        const int64_t boff = x.q.b_kmajor ? nm * x.q.ldb : nm;  // elements
        qt.N = nt;
        qt.B = static_cast<const char *>(x.q.B) + boff * esize;
        qt.span_b = x.q.span_b - boff;
        qt.C = static_cast<char *>(x.q.C) + nm * elem_bytes(x.q.out);  // canonical C is row-major
        const Kernel kt = choose(qt, false);
        if (kt != Kernel::HgemmSplitk && kt != Kernel::SgemmSplitk) return false;
        x.q.N = nm;
        x.qt = qt;
        x.kt = kt;
        return true;
    };
    WsPlan cand = w;
    const bool tail = split_tail(cand);
    const Problem &part = tail ? cand.q : w.q;  // what the direct-load kernel computes
    if (h16 ? hgemm_dma_streamk_eligible(part, force) : sgemm_dma_streamk_eligible(part, force)) {
        const int64_t partials = round_up(h16 ? hgemm_dma_streamk_bytes(part) : sgemm_streamk_bytes(part), 256);
        WsPlan keep = tail ? cand : w;
        if (place(partials, h16 ? Kernel::HgemmPackDmaStreamK : Kernel::SgemmPackDmaStreamK)) {
            if (tail) split_tail(w);  // the copies moved: the tail's pointers again
        } else {
            w = keep;  // no room: plain schedule
        }
    } else if (tail) {
        w = cand;
    }
    return true;
}

// The checks of a workspace argument: 256-byte aligned, not NULL when it has
// bytes, and not overlapping A, B, C or the bias.
gemm_status_t check_workspace(const Problem &p, int64_t M, int64_t N, int64_t K, int orderA,
                              int64_t lda, int orderB, int64_t ldb, int orderC, int64_t ldc,
                              int64_t strideA, int64_t strideB, int64_t strideC,
                              const void *bias, int64_t strideBias, const void *A, const void *B,
                              const void *C, const void *workspace, size_t bytes) {
    if (bytes == 0) return GEMM_OK;
    if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return GEMM_ERR_INVALID_ARG;
    const int esz = elem_bytes(p.in), eout = elem_bytes(p.out);
    const Range rw{reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) + bytes};
    if (overlap(rw, range_of(C, span(M, N, orderC, ldc), p.batch, strideC, eout)) ||
        overlap(rw, range_of(A, span(M, K, orderA, lda), p.batch, strideA, esz)) ||
        overlap(rw, range_of(B, span(K, N, orderB, ldb), p.batch, strideB, esz)) ||
        (bias != nullptr && overlap(rw, range_of(bias, N, p.batch, strideBias, esz))))
        return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

// The plan for a checked workspace of `bytes` bytes at `workspace` (only its
// address is used, to place the operand copies).  Unaligned operands of large
// problems are copied into aligned buffers for the direct-load kernels
// (plan_packed); otherwise the 16-bit and fp32 kernels (the direct-load and
// the general ones) and the 8-bit direct-load kernel switch to their
// stream-K schedule where it applies.  w.k holds the kernel chosen without a workspace.
void plan_workspace(const Problem &p, const void *workspace, size_t bytes, WsPlan &w) {
    w.q = p;
    w.used = 0;
    const bool room = bytes >= static_cast<size_t>(hgemm_streamk_workspace_bytes());
    if (!room || force_general()) return;
    const bool force = force_streamk();
    if (plan_packed(p, w.k, workspace, bytes, force, w)) return;
    Kernel &k = w.k;
    if (k == Kernel::HgemmMfma && hgemm_streamk_eligible(p, force)) {
        k = Kernel::HgemmStreamK;
        w.used = hgemm_streamk_bytes(p);
    } else if (k == Kernel::HgemmDma && hgemm_dma_streamk_eligible(p, force)) {
        k = Kernel::HgemmDmaStreamK;
        w.used = hgemm_dma_streamk_bytes(p);
    } else if (k == Kernel::SgemmMfma && sgemm_streamk_eligible(p, force)) {
        k = Kernel::SgemmStreamK;
        w.used = sgemm_streamk_bytes(p);
    } else if (k == Kernel::SgemmDma && sgemm_dma_streamk_eligible(p, force)) {
        k = Kernel::SgemmDmaStreamK;
        w.used = sgemm_streamk_bytes(p);
    } else if (k == Kernel::F8Dma && f8gemm_dma_streamk_eligible(p, force)) {
        k = Kernel::F8DmaStreamK;
        w.used = f8gemm_dma_streamk_bytes(p);
    } else if (k == Kernel::Skinny && skinny_sk_eligible(p) &&
               skinny_sk_bytes(p) <= static_cast<int64_t>(bytes)) {
        k = Kernel::SkinnySplitK;
        w.used = skinny_sk_bytes(p);
    }
}

gemm_status_t use_workspace(const Problem &p, int64_t M, int64_t N, int64_t K, int orderA,
                            int64_t lda, int orderB, int64_t ldb, int orderC, int64_t ldc,
                            int64_t strideA, int64_t strideB, int64_t strideC,
                            const void *bias, int64_t strideBias, const void *A, const void *B,
                            const void *C, const void *workspace, size_t bytes, WsPlan &w) {
    const gemm_status_t st = check_workspace(p, M, N, K, orderA, lda, orderB, ldb, orderC, ldc,
                                             strideA, strideB, strideC, bias, strideBias, A, B,
                                             C, workspace, bytes);
    if (st != GEMM_OK) return st;
    plan_workspace(p, workspace, bytes, w);
    return GEMM_OK;
}

hipError_t launch_planned(const WsPlan &w, void *workspace, hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    if (is_packed(w.k)) {
        const hipError_t e = launch_pack2(w.pa, ws + w.off_a, w.pb, ws + w.off_b, stream);
        if (e != hipSuccess) return e;
    }
    switch (w.k) {
    case Kernel::HgemmStreamK: return launch_hgemm_streamk(w.q, workspace, stream);
    case Kernel::HgemmDmaStreamK:
    case Kernel::HgemmPackDmaStreamK: return launch_hgemm_dma_streamk(w.q, workspace, stream);
    case Kernel::SgemmStreamK: return launch_sgemm_streamk(w.q, workspace, stream);
    case Kernel::SgemmDmaStreamK:
    case Kernel::SgemmPackDmaStreamK: return launch_sgemm_dma_streamk(w.q, workspace, stream);
    case Kernel::SkinnySplitK: return launch_skinny_sk(w.q, workspace, stream);
    case Kernel::F8DmaStreamK: return launch_f8gemm_dma_streamk(w.q, workspace, stream);
    case Kernel::HgemmPackDma: return launch_hgemm_dma(w.q, stream);
    case Kernel::SgemmPackDma: return launch_sgemm_dma(w.q, stream);
    default: return launch(w.k, w.q, stream);
    }
}

// A planned call: the plan's main launches, then its tail columns if split off.
hipError_t launch_plan(const WsPlan &w, void *workspace, hipStream_t stream) {
    const hipError_t e = launch_planned(w, workspace, stream);
    if (e != hipSuccess || w.kt == Kernel::None) return e;
    return launch(w.kt, w.qt, stream);
}

gemm_status_t run(Elem in, Elem in_b, Elem out, int64_t M, int64_t N, int64_t K, float alpha,
                  const void *A, int64_t lda, int orderA, const void *B, int64_t ldb, int orderB,
                  float beta, void *C, int64_t ldc, int orderC, int64_t batch, int64_t strideA,
                  int64_t strideB, int64_t strideC, const void *bias, int64_t strideBias, int act,
                  hipStream_t stream, void *workspace = nullptr, size_t workspace_bytes = 0,
                  bool valu = false) {
    Problem p;
    WsPlan w;
    gemm_status_t st =
        plan(in, in_b, out, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta, C, ldc, orderC,
             batch, strideA, strideB, strideC, bias, strideBias, act, p, w.k, valu);
    if (st == GEMM_OK && w.k != Kernel::None)
        st = use_workspace(p, M, N, K, orderA, lda, orderB, ldb, orderC, ldc, strideA, strideB,
                           strideC, bias, strideBias, A, B, C, workspace, workspace_bytes, w);
    if (st != GEMM_OK || w.k == Kernel::None) return st;
    const hipError_t err = launch_plan(w, workspace, stream);
    if (err == hipErrorInvalidConfiguration) return GEMM_ERR_UNSUPPORTED;
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

Elem out_type(Elem in, gemm_dtype_t c_dtype) { return c_dtype == GEMM_DTYPE_F32 ? Elem::F32 : in; }

// An fp32 call computed as three bf16 products (gemm_f32_bf16x3): the
// canonical fp32 problem, and the bf16 problem on the split copies in the
// workspace (A' at its start, B' after it).  k is None or Scale when nothing
// is multiplied (then the call is gemm_f32's), else the bf16 kernel.
struct SplitPlan {
    Problem p, q;
    Kernel k = Kernel::None;
    int64_t batch_a = 0, batch_b = 0;  // copies of A and B (1 for a broadcast operand)
    int64_t off_b = 0;                 // byte offset of B' in the workspace
};

int64_t split_copies(const Problem &p, bool a) {
    return p.batch > 1 && (a ? p.sA : p.sB) == 0 ? 1 : p.batch;
}

// Validates the call and the workspace; no HIP call.
gemm_status_t split_plan(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
                         int orderA, const void *B, int64_t ldb, int orderB, float beta,
                         const void *C, int64_t ldc, int orderC, int64_t batch, int64_t strideA,
                         int64_t strideB, int64_t strideC, const void *workspace, size_t bytes,
                         SplitPlan &s) {
    gemm_status_t st = plan(Elem::F32, Elem::F32, Elem::F32, M, N, K, alpha, A, lda, orderA, B,
                            ldb, orderB, beta, const_cast<void *>(C), ldc, orderC, batch, strideA,
                            strideB, strideC, nullptr, 0, GEMM_ACT_NONE, s.p, s.k);
    if (st != GEMM_OK || s.k == Kernel::None || s.k == Kernel::Scale) return st;
    const Problem &p = s.p;
    s.batch_a = split_copies(p, true);
    s.batch_b = split_copies(p, false);
    const int64_t need_a = split_bytes(p.M, p.K, s.batch_a);
    const int64_t need_b = split_bytes(p.N, p.K, s.batch_b);
    if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
        bytes < static_cast<size_t>(need_a + need_b))
        return GEMM_ERR_INVALID_ARG;
    st = check_workspace(p, M, N, K, orderA, lda, orderB, ldb, orderC, ldc, strideA, strideB,
                         strideC, nullptr, 0, A, B, C, workspace, bytes);
    if (st != GEMM_OK) return st;
    s.off_b = need_a;
    const int64_t K3 = 3 * split_kp(p.K);
    Problem q = p;
    q.in = q.in_b = Elem::BF16;
    q.out = Elem::F32;
    q.K = K3;
    q.A = workspace;
    q.lda = K3;
    q.a_kmajor = true;
    q.sA = s.batch_a > 1 ? p.M * K3 : 0;
    q.B = static_cast<const char *>(workspace) + need_a;
    q.ldb = K3;
    q.b_kmajor = true;
    q.sB = s.batch_b > 1 ? p.N * K3 : 0;
    s.q = q;
    s.k = choose(q, false);
    return GEMM_OK;
}

// 8-bit format and output-type enumerators; false when out of range.
bool f8_type(gemm_f8_format_t f, Elem &e) {
    if (f == GEMM_F8_E4M3) e = Elem::E4M3;
    else if (f == GEMM_F8_E5M2) e = Elem::E5M2;
    else return false;
    return true;
}
bool output_type(gemm_output_t t, Elem &e) {
    if (t == GEMM_OUTPUT_F32) e = Elem::F32;
    else if (t == GEMM_OUTPUT_BF16) e = Elem::BF16;
    else if (t == GEMM_OUTPUT_F16) e = Elem::F16;
    else return false;
    return true;
}

// Validates a gemm_mx call and builds its canonical problem (row-major C;
// a column-major C is computed as C^T = B^T A^T, which swaps the roles of
// the two K-contiguous operands and their scales).  No HIP call.
gemm_status_t mx_plan(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
                      gemm_mx_format_t formatA, const uint8_t *scaleA, int64_t ldsa,
                      const void *B, int64_t ldb, gemm_mx_format_t formatB,
                      const uint8_t *scaleB, int64_t ldsb, float beta, const void *C,
                      int64_t ldc, gemm_order_t orderC, gemm_output_t typeC, int64_t batch,
                      int64_t strideA, int64_t strideB, int64_t strideScaleA,
                      int64_t strideScaleB, int64_t strideC, MxProblem &m, Kernel &kernel,
                      const void *workspace = nullptr, size_t ws_bytes = 0) {
    kernel = Kernel::None;
    Elem ec;
    auto fmt_ok = [](gemm_mx_format_t f) { return f >= GEMM_MX_E4M3 && f <= GEMM_MX_E2M1; };
    if (!fmt_ok(formatA) || !fmt_ok(formatB) || !output_type(typeC, ec) || !valid_order(orderC))
        return GEMM_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0 || batch < 0 || strideA < 0 || strideB < 0 || strideC < 0 ||
        strideScaleA < 0 || strideScaleB < 0)
        return GEMM_ERR_INVALID_ARG;
    if (K % 64 != 0) return GEMM_ERR_INVALID_ARG;
    const int64_t min_ldc = orderC == GEMM_ROW_MAJOR ? N : M;
    if (ldc < (min_ldc > 1 ? min_ldc : 1)) return GEMM_ERR_INVALID_ARG;
    if (too_big(M, N) || too_big(M * N, batch) || too_big(M, K) || too_big(K, N) ||
        too_big(batch - 1, strideC) || too_big(batch - 1, strideA) || too_big(batch - 1, strideB) ||
        too_big(batch - 1, strideScaleA) || too_big(batch - 1, strideScaleB))
        return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || batch == 0) return GEMM_OK;

    const bool reads = K > 0 && alpha != 0.0f;
    const int eout = elem_bytes(ec);
    const int wa = mx_width(formatA), wb = mx_width(formatB);
    const int64_t span_c = span(M, N, orderC, ldc);
    if (C == nullptr || reinterpret_cast<uintptr_t>(C) % eout != 0) return GEMM_ERR_INVALID_ARG;
    if (batch > 1 && strideC < span_c) return GEMM_ERR_INVALID_ARG;  // C slices overlap
    const Range rc = range_of(C, span_c, batch, strideC, eout);
    const int64_t sbytes = 4 * ((K + 127) / 128);  // scale bytes per row the kernel reads
    // a workspace: 256-byte aligned, not NULL when it has bytes, and not
    // overlapping C (nor, below, A, B or their scales)
    const Range rw{reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) + ws_bytes};
    if (ws_bytes > 0 && (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
                         overlap(rw, rc)))
        return GEMM_ERR_INVALID_ARG;
    if (reads) {
        if (A == nullptr || B == nullptr || scaleA == nullptr || scaleB == nullptr)
            return GEMM_ERR_INVALID_ARG;
        if (lda < K || ldb < K || lda % 64 != 0 || ldb % 64 != 0) return GEMM_ERR_INVALID_ARG;
        if (batch > 1 && (strideA % 64 != 0 || strideB % 64 != 0)) return GEMM_ERR_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(A) % 16 != 0 || reinterpret_cast<uintptr_t>(B) % 16 != 0)
            return GEMM_ERR_INVALID_ARG;
        if (ldsa < sbytes || ldsb < sbytes || ldsa % 4 != 0 || ldsb % 4 != 0)
            return GEMM_ERR_INVALID_ARG;
        if (batch > 1 && (strideScaleA % 4 != 0 || strideScaleB % 4 != 0)) return GEMM_ERR_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(scaleA) % 4 != 0 ||
            reinterpret_cast<uintptr_t>(scaleB) % 4 != 0)
            return GEMM_ERR_INVALID_ARG;
        // byte extents of one slice of each operand and of its scales
        const int64_t bytes_a = ((M - 1) * lda + K) * wa / 8, bytes_b = ((N - 1) * ldb + K) * wb / 8;
        const int64_t sc_a = (M - 1) * ldsa + sbytes, sc_b = (N - 1) * ldsb + sbytes;
        const Range ra = range_of(A, bytes_a, batch, strideA * wa / 8, 1);
        const Range rb = range_of(B, bytes_b, batch, strideB * wb / 8, 1);
        const Range rsa = range_of(scaleA, sc_a, batch, strideScaleA, 1);
        const Range rsb = range_of(scaleB, sc_b, batch, strideScaleB, 1);
        if (overlap(rc, ra) || overlap(rc, rb) || overlap(rc, rsa) || overlap(rc, rsb))
            return GEMM_ERR_INVALID_ARG;
        if (overlap(rw, ra) || overlap(rw, rb) || overlap(rw, rsa) || overlap(rw, rsb))
            return GEMM_ERR_INVALID_ARG;
        if (wa != wb) return GEMM_ERR_UNSUPPORTED;
        // the kernel addresses a slice with 32-bit byte offsets
        const int64_t limit = int64_t(1) << 30;
        if (bytes_a >= limit || bytes_b >= limit || M * ldsa >= limit || N * ldsb >= limit)
            return GEMM_ERR_UNSUPPORTED;
    }

    Problem &p = m.p;
    p = Problem{};
    p.K = K;
    p.alpha = alpha;
    p.beta = beta;
    p.C = const_cast<void *>(C);
    p.ldc = ldc;
    p.batch = batch;
    p.sC = strideC;
    p.out = ec;
    p.in = p.in_b = Elem::E4M3;  // unused: the formats are in m
    p.a_kmajor = p.b_kmajor = true;
    const bool row = orderC == GEMM_ROW_MAJOR;
    p.M = row ? M : N;
    p.N = row ? N : M;
    p.A = row ? A : B;
    p.lda = row ? lda : ldb;
    p.sA = row ? strideA : strideB;
    p.B = row ? B : A;
    p.ldb = row ? ldb : lda;
    p.sB = row ? strideB : strideA;
    m.fa = static_cast<int>(row ? formatA : formatB);
    m.fb = static_cast<int>(row ? formatB : formatA);
    m.sa = row ? scaleA : scaleB;
    m.sb = row ? scaleB : scaleA;
    m.ldsa = row ? ldsa : ldsb;
    m.ldsb = row ? ldsb : ldsa;
    m.ssa = row ? strideScaleA : strideScaleB;
    m.ssb = row ? strideScaleB : strideScaleA;
    kernel = reads ? Kernel::Mx : Kernel::Scale;
    // with a workspace of at least gemm_workspace_size() bytes: the stream-K
    // schedule where it applies
    if (kernel == Kernel::Mx && ws_bytes >= static_cast<size_t>(hgemm_streamk_workspace_bytes()) &&
        !force_general() && mxgemm_streamk_eligible(m, force_streamk()))
        kernel = Kernel::MxStreamK;
    return GEMM_OK;
}

// Runs a planned gemm_mx call.
gemm_status_t mx_run(const MxProblem &m, Kernel k, void *workspace, hipStream_t stream) {
    if (k == Kernel::None) return GEMM_OK;
    const hipError_t err = k == Kernel::MxStreamK ? launch_mxgemm_streamk(m, workspace, stream)
                           : k == Kernel::Mx      ? launch_mxgemm(m, stream)
                                                  : launch_scale(m.p, stream);
    if (err == hipErrorInvalidConfiguration) return GEMM_ERR_UNSUPPORTED;
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

}  // namespace

extern "C" {

gemm_status_t gemm_mx(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
                      gemm_mx_format_t formatA, const uint8_t *scaleA, int64_t ldsa,
                      const void *B, int64_t ldb, gemm_mx_format_t formatB,
                      const uint8_t *scaleB, int64_t ldsb, float beta, void *C, int64_t ldc,
                      gemm_order_t orderC, gemm_output_t typeC, int64_t batch, int64_t strideA,
                      int64_t strideB, int64_t strideScaleA, int64_t strideScaleB,
                      int64_t strideC, hipStream_t stream) {
    MxProblem m;
    Kernel k;
    const gemm_status_t st =
        mx_plan(M, N, K, alpha, A, lda, formatA, scaleA, ldsa, B, ldb, formatB, scaleB, ldsb, beta, C,
                ldc, orderC, typeC, batch, strideA, strideB, strideScaleA, strideScaleB, strideC, m, k);
    if (st != GEMM_OK) return st;
    return mx_run(m, k, nullptr, stream);
}

gemm_status_t gemm_mx_ws(int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
                         gemm_mx_format_t formatA, const uint8_t *scaleA, int64_t ldsa,
                         const void *B, int64_t ldb, gemm_mx_format_t formatB,
                         const uint8_t *scaleB, int64_t ldsb, float beta, void *C, int64_t ldc,
                         gemm_order_t orderC, gemm_output_t typeC, int64_t batch, int64_t strideA,
                         int64_t strideB, int64_t strideScaleA, int64_t strideScaleB,
                         int64_t strideC, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    MxProblem m;
    Kernel k;
    const gemm_status_t st =
        mx_plan(M, N, K, alpha, A, lda, formatA, scaleA, ldsa, B, ldb, formatB, scaleB, ldsb, beta, C,
                ldc, orderC, typeC, batch, strideA, strideB, strideScaleA, strideScaleB, strideC, m, k,
                workspace, workspace_bytes);
    if (st != GEMM_OK) return st;
    return mx_run(m, k, workspace, stream);
}

const char *gemm_mx_kernel_name(int64_t M, int64_t N, int64_t K, float alpha, const void *A,
                                int64_t lda, gemm_mx_format_t formatA, const uint8_t *scaleA,
                                int64_t ldsa, const void *B, int64_t ldb,
                                gemm_mx_format_t formatB, const uint8_t *scaleB, int64_t ldsb,
                                float beta, const void *C, int64_t ldc, gemm_order_t orderC,
                                gemm_output_t typeC, int64_t batch, int64_t strideA,
                                int64_t strideB, int64_t strideScaleA, int64_t strideScaleB,
                                int64_t strideC) {
    return gemm_mx_kernel_name_ws(M, N, K, alpha, A, lda, formatA, scaleA, ldsa, B, ldb, formatB,
                                  scaleB, ldsb, beta, C, ldc, orderC, typeC, batch, strideA,
                                  strideB, strideScaleA, strideScaleB, strideC, nullptr, 0);
}

const char *gemm_mx_kernel_name_ws(int64_t M, int64_t N, int64_t K, float alpha, const void *A,
                                   int64_t lda, gemm_mx_format_t formatA, const uint8_t *scaleA,
                                   int64_t ldsa, const void *B, int64_t ldb,
                                   gemm_mx_format_t formatB, const uint8_t *scaleB, int64_t ldsb,
                                   float beta, const void *C, int64_t ldc, gemm_order_t orderC,
                                   gemm_output_t typeC, int64_t batch, int64_t strideA,
                                   int64_t strideB, int64_t strideScaleA, int64_t strideScaleB,
                                   int64_t strideC, const void *workspace,
                                   size_t workspace_bytes) {
    MxProblem m;
    Kernel k;
    if (mx_plan(M, N, K, alpha, A, lda, formatA, scaleA, ldsa, B, ldb, formatB, scaleB, ldsb, beta, C,
                ldc, orderC, typeC, batch, strideA, strideB, strideScaleA, strideScaleB, strideC, m,
                k, workspace, workspace_bytes) != GEMM_OK)
        return nullptr;
    return kernel_name(k);
}

gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                       gemm_order_t orderA, const float *B, int64_t ldb, gemm_order_t orderB,
                       float beta, float *C, int64_t ldc, gemm_order_t orderC, int64_t batch,
                       int64_t strideA, int64_t strideB, int64_t strideC, hipStream_t stream) {
    return run(Elem::F32, Elem::F32, Elem::F32, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta, C, ldc,
               orderC, batch, strideA, strideB, strideC, nullptr, 0, GEMM_ACT_NONE, stream);
}

gemm_status_t gemm_f32_valu(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                            int64_t lda, gemm_order_t orderA, const float *B, int64_t ldb,
                            gemm_order_t orderB, float beta, float *C, int64_t ldc,
                            gemm_order_t orderC, int64_t batch, int64_t strideA, int64_t strideB,
                            int64_t strideC, hipStream_t stream) {
    return run(Elem::F32, Elem::F32, Elem::F32, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta,
               C, ldc, orderC, batch, strideA, strideB, strideC, nullptr, 0, GEMM_ACT_NONE, stream,
               nullptr, 0, true);
}

// A quantised-output call (gemm_bf16_quant / gemm_f16_quant): the canonical
// problem with an 8-bit C and the epilogue's scale, and its kernel (the
// 16-bit direct-load kernel, or the scale kernel when nothing is
// multiplied).  GEMM_ERR_UNSUPPORTED for operands the direct-load kernel
// cannot read.  No HIP call.
gemm_status_t quant_plan(Elem in, int64_t M, int64_t N, int64_t K, float alpha, const void *A,
                         int64_t lda, int orderA, const void *B, int64_t ldb, int orderB, void *C,
                         int64_t ldc, int orderC, gemm_f8_format_t c_format, float c_scale,
                         int64_t batch, int64_t strideA, int64_t strideB, int64_t strideC,
                         const void *bias, int64_t strideBias, int act, Problem &p, Kernel &k) {
    Elem out;
    if (!f8_type(c_format, out)) return GEMM_ERR_INVALID_ARG;
    gemm_status_t st = plan(in, in, out, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, 0.0f, C,
                            ldc, orderC, batch, strideA, strideB, strideC, bias, strideBias, act, p,
                            k);
    if (st != GEMM_OK || k == Kernel::None) return st;
    p.epi.out_scale = c_scale;
    p.epi.out_e5m2 = out == Elem::E5M2 ? 1 : 0;
    if (k != Kernel::Scale) {
        if (!hgemm_dma_eligible(p)) {
            k = Kernel::None;
            return GEMM_ERR_UNSUPPORTED;
        }
        k = Kernel::HgemmDma;
    }
    return GEMM_OK;
}

gemm_status_t run_quant(Elem in, int64_t M, int64_t N, int64_t K, float alpha, const void *A,
                        int64_t lda, int orderA, const void *B, int64_t ldb, int orderB, void *C,
                        int64_t ldc, int orderC, gemm_f8_format_t c_format, float c_scale,
                        int64_t batch, int64_t strideA, int64_t strideB, int64_t strideC,
                        const void *bias, int64_t strideBias, int act, hipStream_t stream) {
    Problem p;
    Kernel k;
    const gemm_status_t st =
        quant_plan(in, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, C, ldc, orderC, c_format,
                   c_scale, batch, strideA, strideB, strideC, bias, strideBias, act, p, k);
    if (st != GEMM_OK || k == Kernel::None) return st;
    const hipError_t e = launch(k, p, stream);
    if (e == hipErrorInvalidConfiguration) return GEMM_ERR_UNSUPPORTED;
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

size_t gemm_f32_bf16x3_workspace_size(int64_t M, int64_t N, int64_t K, int64_t batch) {
    if (M < 0 || N < 0 || K < 0 || batch < 0 || too_big(M, K) || too_big(N, K)) return 0;
    const int64_t kp = split_kp(K);
    if (too_big(6 * kp, M + N) || too_big(6 * kp * (M + N), batch)) return 0;
    return static_cast<size_t>(split_bytes(M, K, batch) + split_bytes(N, K, batch));
}

gemm_status_t gemm_f32_bf16x3(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                              int64_t lda, gemm_order_t orderA, const float *B, int64_t ldb,
                              gemm_order_t orderB, float beta, float *C, int64_t ldc,
                              gemm_order_t orderC, int64_t batch, int64_t strideA,
                              int64_t strideB, int64_t strideC, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    SplitPlan s;
    const gemm_status_t st = split_plan(M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta, C,
                                        ldc, orderC, batch, strideA, strideB, strideC, workspace,
                                        workspace_bytes, s);
    if (st != GEMM_OK || s.k == Kernel::None) return st;
    hipError_t e;
    if (s.k == Kernel::Scale) {
        e = launch(s.k, s.p, stream);
    } else {
        const Problem &p = s.p;
        uint16_t *wa = static_cast<uint16_t *>(workspace);
        uint16_t *wb = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + s.off_b);
        e = launch_split_a(static_cast<const float *>(p.A), p.lda, p.sA, p.a_kmajor, p.M, p.K,
                           s.batch_a, wa, stream);
        if (e == hipSuccess)
            e = launch_split_b(static_cast<const float *>(p.B), p.ldb, p.sB, p.b_kmajor, p.N,
                               p.K, s.batch_b, wb, stream);
        if (e == hipSuccess) e = launch(s.k, s.q, stream);
    }
    if (e == hipErrorInvalidConfiguration) return GEMM_ERR_UNSUPPORTED;
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

gemm_status_t gemm_bf16_quant(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                              int64_t lda, gemm_order_t orderA, const uint16_t *B, int64_t ldb,
                              gemm_order_t orderB, uint8_t *C, int64_t ldc, gemm_order_t orderC,
                              gemm_f8_format_t c_format, float c_scale, int64_t batch,
                              int64_t strideA, int64_t strideB, int64_t strideC,
                              const uint16_t *bias, int64_t strideBias, gemm_activation_t act,
                              hipStream_t stream) {
    return run_quant(Elem::BF16, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, C, ldc, orderC,
                     c_format, c_scale, batch, strideA, strideB, strideC, bias, strideBias, act,
                     stream);
}

gemm_status_t gemm_f16_quant(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                             int64_t lda, gemm_order_t orderA, const uint16_t *B, int64_t ldb,
                             gemm_order_t orderB, uint8_t *C, int64_t ldc, gemm_order_t orderC,
                             gemm_f8_format_t c_format, float c_scale, int64_t batch,
                             int64_t strideA, int64_t strideB, int64_t strideC,
                             const uint16_t *bias, int64_t strideBias, gemm_activation_t act,
                             hipStream_t stream) {
    return run_quant(Elem::F16, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, C, ldc, orderC,
                     c_format, c_scale, batch, strideA, strideB, strideC, bias, strideBias, act,
                     stream);
}

int gemm_test_switches(int flags) {
    return g_switches.exchange(flags & (GEMM_TEST_FORCE_GENERAL | GEMM_TEST_NO_SPLITK |
                                        GEMM_TEST_FORCE_STREAMK | GEMM_TEST_F32_VALU));
}

gemm_status_t gemm_f32_ws(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                          int64_t lda, gemm_order_t orderA, const float *B, int64_t ldb,
                          gemm_order_t orderB, float beta, float *C, int64_t ldc, gemm_order_t orderC,
                          int64_t batch, int64_t strideA, int64_t strideB, int64_t strideC,
                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return run(Elem::F32, Elem::F32, Elem::F32, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta, C, ldc,
               orderC, batch, strideA, strideB, strideC, nullptr, 0, GEMM_ACT_NONE, stream, workspace,
               workspace_bytes);
}

gemm_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                        int64_t lda, gemm_order_t orderA, const uint16_t *B, int64_t ldb,
                        gemm_order_t orderB, float beta, void *C, int64_t ldc, gemm_order_t orderC,
                        gemm_dtype_t c_dtype, int64_t batch, int64_t strideA, int64_t strideB,
                        int64_t strideC, hipStream_t stream) {
    if (c_dtype != GEMM_DTYPE_SAME && c_dtype != GEMM_DTYPE_F32) return GEMM_ERR_INVALID_ARG;
    return run(Elem::BF16, Elem::BF16, out_type(Elem::BF16, c_dtype), M, N, K, alpha, A, lda, orderA, B, ldb,
               orderB, beta, C, ldc, orderC, batch, strideA, strideB, strideC, nullptr, 0,
               GEMM_ACT_NONE, stream);
}

gemm_status_t gemm_f16(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                       int64_t lda, gemm_order_t orderA, const uint16_t *B, int64_t ldb,
                       gemm_order_t orderB, float beta, void *C, int64_t ldc, gemm_order_t orderC,
                       gemm_dtype_t c_dtype, int64_t batch, int64_t strideA, int64_t strideB,
                       int64_t strideC, hipStream_t stream) {
    if (c_dtype != GEMM_DTYPE_SAME && c_dtype != GEMM_DTYPE_F32) return GEMM_ERR_INVALID_ARG;
    return run(Elem::F16, Elem::F16, out_type(Elem::F16, c_dtype), M, N, K, alpha, A, lda, orderA, B, ldb,
               orderB, beta, C, ldc, orderC, batch, strideA, strideB, strideC, nullptr, 0,
               GEMM_ACT_NONE, stream);
}

gemm_status_t gemm_f32_bias_act(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                                int64_t lda, gemm_order_t orderA, const float *B, int64_t ldb,
                                gemm_order_t orderB, float beta, float *C, int64_t ldc,
                                gemm_order_t orderC, int64_t batch, int64_t strideA,
                                int64_t strideB, int64_t strideC, const float *bias,
                                int64_t strideBias, gemm_activation_t act, hipStream_t stream) {
    return run(Elem::F32, Elem::F32, Elem::F32, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta, C, ldc,
               orderC, batch, strideA, strideB, strideC, bias, strideBias, act, stream);
}

gemm_status_t gemm_bf16_bias_act(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                                 int64_t lda, gemm_order_t orderA, const uint16_t *B, int64_t ldb,
                                 gemm_order_t orderB, float beta, void *C, int64_t ldc,
                                 gemm_order_t orderC, gemm_dtype_t c_dtype, int64_t batch,
                                 int64_t strideA, int64_t strideB, int64_t strideC,
                                 const uint16_t *bias, int64_t strideBias, gemm_activation_t act,
                                 hipStream_t stream) {
    if (c_dtype != GEMM_DTYPE_SAME && c_dtype != GEMM_DTYPE_F32) return GEMM_ERR_INVALID_ARG;
    return run(Elem::BF16, Elem::BF16, out_type(Elem::BF16, c_dtype), M, N, K, alpha, A, lda, orderA, B, ldb,
               orderB, beta, C, ldc, orderC, batch, strideA, strideB, strideC, bias, strideBias,
               act, stream);
}

gemm_status_t gemm_f16_bias_act(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                                int64_t lda, gemm_order_t orderA, const uint16_t *B, int64_t ldb,
                                gemm_order_t orderB, float beta, void *C, int64_t ldc,
                                gemm_order_t orderC, gemm_dtype_t c_dtype, int64_t batch,
                                int64_t strideA, int64_t strideB, int64_t strideC,
                                const uint16_t *bias, int64_t strideBias, gemm_activation_t act,
                                hipStream_t stream) {
    if (c_dtype != GEMM_DTYPE_SAME && c_dtype != GEMM_DTYPE_F32) return GEMM_ERR_INVALID_ARG;
    return run(Elem::F16, Elem::F16, out_type(Elem::F16, c_dtype), M, N, K, alpha, A, lda, orderA, B, ldb,
               orderB, beta, C, ldc, orderC, batch, strideA, strideB, strideC, bias, strideBias,
               act, stream);
}

gemm_status_t gemm_f8(int64_t M, int64_t N, int64_t K, float alpha, const uint8_t *A, int64_t lda,
                      gemm_order_t orderA, gemm_f8_format_t formatA, const uint8_t *B,
                      int64_t ldb, gemm_order_t orderB, gemm_f8_format_t formatB, float beta,
                      void *C, int64_t ldc, gemm_order_t orderC, gemm_output_t typeC,
                      int64_t batch, int64_t strideA, int64_t strideB, int64_t strideC,
                      hipStream_t stream) {
    Elem ea, eb, ec;
    if (!f8_type(formatA, ea) || !f8_type(formatB, eb) || !output_type(typeC, ec))
        return GEMM_ERR_INVALID_ARG;
    return run(ea, eb, ec, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta, C, ldc, orderC,
               batch, strideA, strideB, strideC, nullptr, 0, GEMM_ACT_NONE, stream);
}

gemm_status_t gemm_f8_ws(int64_t M, int64_t N, int64_t K, float alpha, const uint8_t *A,
                         int64_t lda, gemm_order_t orderA, gemm_f8_format_t formatA,
                         const uint8_t *B, int64_t ldb, gemm_order_t orderB,
                         gemm_f8_format_t formatB, float beta, void *C, int64_t ldc,
                         gemm_order_t orderC, gemm_output_t typeC, int64_t batch, int64_t strideA,
                         int64_t strideB, int64_t strideC, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    Elem ea, eb, ec;
    if (!f8_type(formatA, ea) || !f8_type(formatB, eb) || !output_type(typeC, ec))
        return GEMM_ERR_INVALID_ARG;
    return run(ea, eb, ec, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta, C, ldc, orderC,
               batch, strideA, strideB, strideC, nullptr, 0, GEMM_ACT_NONE, stream, workspace,
               workspace_bytes);
}

size_t gemm_workspace_size(void) { return static_cast<size_t>(hgemm_streamk_workspace_bytes()); }

gemm_status_t gemm_bf16_ws(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                           int64_t lda, gemm_order_t orderA, const uint16_t *B, int64_t ldb,
                           gemm_order_t orderB, float beta, void *C, int64_t ldc,
                           gemm_order_t orderC, gemm_dtype_t c_dtype, int64_t batch,
                           int64_t strideA, int64_t strideB, int64_t strideC, void *workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    if (c_dtype != GEMM_DTYPE_SAME && c_dtype != GEMM_DTYPE_F32) return GEMM_ERR_INVALID_ARG;
    return run(Elem::BF16, Elem::BF16, out_type(Elem::BF16, c_dtype), M, N, K, alpha, A, lda,
               orderA, B, ldb, orderB, beta, C, ldc, orderC, batch, strideA, strideB, strideC,
               nullptr, 0, GEMM_ACT_NONE, stream, workspace, workspace_bytes);
}

gemm_status_t gemm_f16_ws(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                          int64_t lda, gemm_order_t orderA, const uint16_t *B, int64_t ldb,
                          gemm_order_t orderB, float beta, void *C, int64_t ldc,
                          gemm_order_t orderC, gemm_dtype_t c_dtype, int64_t batch,
                          int64_t strideA, int64_t strideB, int64_t strideC, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    if (c_dtype != GEMM_DTYPE_SAME && c_dtype != GEMM_DTYPE_F32) return GEMM_ERR_INVALID_ARG;
    return run(Elem::F16, Elem::F16, out_type(Elem::F16, c_dtype), M, N, K, alpha, A, lda,
               orderA, B, ldb, orderB, beta, C, ldc, orderC, batch, strideA, strideB, strideC,
               nullptr, 0, GEMM_ACT_NONE, stream, workspace, workspace_bytes);
}

gemm_status_t gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                                int64_t lda, gemm_order_t orderA, const uint16_t *B, int64_t ldb,
                                gemm_order_t orderB, float beta, void *C, int64_t ldc,
                                gemm_order_t orderC, gemm_dtype_t c_dtype, int64_t batch,
                                int64_t strideA, int64_t strideB, int64_t strideC,
                                hipStream_t stream) {
    if (c_dtype != GEMM_DTYPE_SAME && c_dtype != GEMM_DTYPE_F32) return GEMM_ERR_INVALID_ARG;
    Problem p;
    WsPlan w;
    gemm_status_t st = plan(Elem::BF16, Elem::BF16, out_type(Elem::BF16, c_dtype), M, N, K, alpha,
                            A, lda, orderA, B, ldb, orderB, beta, C, ldc, orderC, batch, strideA,
                            strideB, strideC, nullptr, 0, GEMM_ACT_NONE, p, w.k);
    if (st != GEMM_OK || w.k == Kernel::None) return st;
    // The plan gemm_bf16_ws would make with a workspace of
    // gemm_workspace_size() bytes, first at a stand-in address (only the
    // bytes it uses matter here), so an oversized call is refused before any
    // HIP call.
    const size_t full = static_cast<size_t>(hgemm_streamk_workspace_bytes());
    const Kernel chosen = w.k;
    plan_workspace(p, reinterpret_cast<const void *>(uintptr_t(256)), full, w);
    if (w.used > static_cast<int64_t>(GEMM_NOALLOC_SCRATCH_BYTES)) return GEMM_ERR_SCRATCH;
    void *scratch = nullptr;
    if (w.used > 0) {
        if (scratch_address(stream, &scratch) != hipSuccess) return GEMM_ERR_HIP;
        w.k = chosen;
        plan_workspace(p, scratch, full, w);  // the same plan, placed in the scratch
    }
    const hipError_t err = launch_plan(w, scratch, stream);
    if (err == hipErrorInvalidConfiguration) return GEMM_ERR_UNSUPPORTED;
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

const char *gemm_status_string(gemm_status_t status) {
    switch (status) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG: invalid argument";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED: combination not supported";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP: kernel launch failed";
    case GEMM_ERR_SCRATCH:
        return "GEMM_ERR_SCRATCH: the call needs more than the 64 MiB of scratch memory of the "
               "allocation-free entry point";
    }
    return "unknown gemm_status_t";
}

int gemm_abi_version(void) { return 1; }

const char *gemm_kernel_name(gemm_input_t in, int64_t M, int64_t N, int64_t K, float alpha,
                             const void *A, int64_t lda, gemm_order_t orderA, const void *B,
                             int64_t ldb, gemm_order_t orderB, float beta, const void *C,
                             int64_t ldc, gemm_order_t orderC, gemm_dtype_t c_dtype, int64_t batch,
                             int64_t strideA, int64_t strideB, int64_t strideC) {
    Elem ein;
    if (in == GEMM_INPUT_F32)
        ein = Elem::F32;
    else if (in == GEMM_INPUT_BF16)
        ein = Elem::BF16;
    else if (in == GEMM_INPUT_F16)
        ein = Elem::F16;
    else
        return nullptr;
    if (ein != Elem::F32 && c_dtype != GEMM_DTYPE_SAME && c_dtype != GEMM_DTYPE_F32) return nullptr;
    Problem p;
    Kernel k;
    const gemm_status_t st =
        plan(ein, ein, ein == Elem::F32 ? Elem::F32 : out_type(ein, c_dtype), M, N, K, alpha, A, lda,
             orderA, B, ldb, orderB, beta, const_cast<void *>(C), ldc, orderC, batch, strideA,
             strideB, strideC, nullptr, 0, GEMM_ACT_NONE, p, k);
    return st == GEMM_OK ? kernel_name(k) : nullptr;
}

const char *gemm_f8_kernel_name(int64_t M, int64_t N, int64_t K, float alpha, const uint8_t *A,
                                int64_t lda, gemm_order_t orderA, gemm_f8_format_t formatA,
                                const uint8_t *B, int64_t ldb, gemm_order_t orderB,
                                gemm_f8_format_t formatB, float beta, const void *C, int64_t ldc,
                                gemm_order_t orderC, gemm_output_t typeC, int64_t batch,
                                int64_t strideA, int64_t strideB, int64_t strideC) {
    Elem ea, eb, ec;
    if (!f8_type(formatA, ea) || !f8_type(formatB, eb) || !output_type(typeC, ec)) return nullptr;
    Problem p;
    Kernel k;
    const gemm_status_t st =
        plan(ea, eb, ec, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta,
             const_cast<void *>(C), ldc, orderC, batch, strideA, strideB, strideC, nullptr, 0,
             GEMM_ACT_NONE, p, k);
    return st == GEMM_OK ? kernel_name(k) : nullptr;
}

const char *gemm_f8_kernel_name_ws(int64_t M, int64_t N, int64_t K, float alpha,
                                   const uint8_t *A, int64_t lda, gemm_order_t orderA,
                                   gemm_f8_format_t formatA, const uint8_t *B, int64_t ldb,
                                   gemm_order_t orderB, gemm_f8_format_t formatB, float beta,
                                   const void *C, int64_t ldc, gemm_order_t orderC,
                                   gemm_output_t typeC, int64_t batch, int64_t strideA,
                                   int64_t strideB, int64_t strideC, const void *workspace,
                                   size_t workspace_bytes) {
    Elem ea, eb, ec;
    if (!f8_type(formatA, ea) || !f8_type(formatB, eb) || !output_type(typeC, ec)) return nullptr;
    Problem p;
    WsPlan w;
    gemm_status_t st =
        plan(ea, eb, ec, M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta,
             const_cast<void *>(C), ldc, orderC, batch, strideA, strideB, strideC, nullptr, 0,
             GEMM_ACT_NONE, p, w.k);
    if (st == GEMM_OK && w.k != Kernel::None)
        st = use_workspace(p, M, N, K, orderA, lda, orderB, ldb, orderC, ldc, strideA, strideB,
                           strideC, nullptr, 0, A, B, C, workspace, workspace_bytes, w);
    return st == GEMM_OK ? kernel_name(w.k) : nullptr;
}

const char *gemm_kernel_name_ws(gemm_input_t in, int64_t M, int64_t N, int64_t K, float alpha,
                                const void *A, int64_t lda, gemm_order_t orderA, const void *B,
                                int64_t ldb, gemm_order_t orderB, float beta, const void *C,
                                int64_t ldc, gemm_order_t orderC, gemm_dtype_t c_dtype,
                                int64_t batch, int64_t strideA, int64_t strideB, int64_t strideC,
                                const void *workspace, size_t workspace_bytes) {
    Elem ein;
    if (in == GEMM_INPUT_BF16)
        ein = Elem::BF16;
    else if (in == GEMM_INPUT_F16)
        ein = Elem::F16;
    else if (in == GEMM_INPUT_F32)
        ein = Elem::F32;
    else
        return nullptr;
    if (ein == Elem::F32) c_dtype = GEMM_DTYPE_SAME;  // gemm_f32_ws has no c_dtype
    if (c_dtype != GEMM_DTYPE_SAME && c_dtype != GEMM_DTYPE_F32) return nullptr;
    Problem p;
    WsPlan w;
    gemm_status_t st =
        plan(ein, ein, out_type(ein, c_dtype), M, N, K, alpha, A, lda, orderA, B, ldb, orderB,
             beta, const_cast<void *>(C), ldc, orderC, batch, strideA, strideB, strideC, nullptr,
             0, GEMM_ACT_NONE, p, w.k);
    if (st == GEMM_OK && w.k != Kernel::None)
        st = use_workspace(p, M, N, K, orderA, lda, orderB, ldb, orderC, ldc, strideA, strideB,
                           strideC, nullptr, 0, A, B, C, workspace, workspace_bytes, w);
    return st == GEMM_OK ? kernel_name(w.k) : nullptr;
}

const char *gemm_kernel_name_quant(gemm_input_t in, int64_t M, int64_t N, int64_t K, float alpha,
                                   const void *A, int64_t lda, gemm_order_t orderA, const void *B,
                                   int64_t ldb, gemm_order_t orderB, const void *C, int64_t ldc,
                                   gemm_order_t orderC, gemm_f8_format_t c_format, int64_t batch,
                                   int64_t strideA, int64_t strideB, int64_t strideC) {
    if (in != GEMM_INPUT_BF16 && in != GEMM_INPUT_F16) return nullptr;
    Problem p;
    Kernel k;
    const gemm_status_t st =
        quant_plan(in == GEMM_INPUT_BF16 ? Elem::BF16 : Elem::F16, M, N, K, alpha, A, lda, orderA,
                   B, ldb, orderB, const_cast<void *>(C), ldc, orderC, c_format, 1.0f, batch,
                   strideA, strideB, strideC, nullptr, 0, GEMM_ACT_NONE, p, k);
    return st == GEMM_OK ? kernel_name(k) : nullptr;
}

const char *gemm_kernel_name_bf16x3(int64_t M, int64_t N, int64_t K, float alpha, const void *A,
                                    int64_t lda, gemm_order_t orderA, const void *B, int64_t ldb,
                                    gemm_order_t orderB, float beta, const void *C, int64_t ldc,
                                    gemm_order_t orderC, int64_t batch, int64_t strideA,
                                    int64_t strideB, int64_t strideC, const void *workspace,
                                    size_t workspace_bytes) {
    SplitPlan s;
    const gemm_status_t st = split_plan(M, N, K, alpha, A, lda, orderA, B, ldb, orderB, beta, C,
                                        ldc, orderC, batch, strideA, strideB, strideC, workspace,
                                        workspace_bytes, s);
    return st == GEMM_OK ? kernel_name(s.k) : nullptr;
}

}  // extern "C"
