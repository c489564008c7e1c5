// bf16 / fp16 GEMM on the CDNA4 matrix cores with fp32 accumulation.
//
// Structure (the block tile -> wave tile -> matrix instruction hierarchy of
// "GPU GEMM 优化完全拆解（三）" (pinghaoyang.com.cn), section "从 kernel 到库",
// realised with gfx950 instructions):
//
//   * one workgroup of 256 threads (four wave64 waves, 2 x 2) computes a
//     256 x 256 tile of C; each wave owns a 128 x 128 sub-tile held as 4 x 4
//     accumulators of v_mfma_f32_32x32x16_{bf16,f16} (16 fp32 per lane each,
//     256 per lane in all);
//   * K advances 64 at a time.  Both operand panels (256 x 64 of A, 64 x 256
//     of B) are stored in LDS "K-contiguous": one 128-byte row of 64 elements
//     per output row/column, eight 16-byte chunks per row.  A lane's matrix
//     operand is then one 16-byte ds_read (eight consecutive k);
//   * chunks are XOR-swizzled: logical chunk c of row r sits at chunk
//     c ^ ((r ^ (r >> 3)) & 7).  Eight consecutive rows read at one logical
//     chunk, and eight rows 8 apart written at one logical chunk, both land
//     on eight different 16-byte bank groups (the XOR swizzle of section 6.3
//     of "CUDA GEMM 矩阵乘法优化指南", blog.zhenwei.site, applied to 16-byte
//     chunks as in section 4 of the hgemm sm120 article, wingedge777.com);
//   * an operand whose global storage is K-contiguous (row-major A,
//     column-major B) is copied chunk for chunk; one that is contiguous along
//     M or N is loaded as 8 x 8 blocks and transposed in registers with
//     byte permutes before it is written, so both land in the same layout;
//   * global loads for the next K step are issued before the current step's
//     matrix instructions and written to the other LDS buffer after them
//     (double buffering, section 9 of the zhenwei.site guide); one barrier
//     per step;
//   * edges: elements outside the matrices read as zero and stores outside C
//     are skipped, so any M, N, K, leading dimension and alignment is exact;
//     16-byte vector loads are used when the operand allows them.
//
// The epilogue computes alpha*acc + beta*C_old in fp32 (C_old is not read
// when beta == 0) and rounds to the output type to nearest-even.
#include "gemm_problem.hpp"
#include "tile_schedule.hpp"

namespace libgemm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int THREADS = 256;
constexpr int ROW_CHUNKS = BK / 8;         // 16-byte chunks per LDS row
constexpr int PANEL = BM * ROW_CHUNKS;     // chunks per operand panel (32 KiB)
static_assert(BM == BN, "both panels share one layout");

constexpr int OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2;

struct HgemmArgs {
    int64_t M, N, K;
    float alpha, beta;
    const uint16_t *A;
    const uint16_t *B;
    void *C;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;
    TileGrid grid;
    int vec_a, vec_b;
    int ubuf_a, ubuf_b;  // the operand's span fits a raw buffer (unaligned vector path)
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

__device__ inline int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Eight consecutive 16-bit elements x[0..7] of one operand row, zero outside
// [0, limit); `inside` says the row itself exists.
__device__ inline u32x4 load8(const uint16_t *x, bool vec, bool inside, int64_t first,
                              int64_t limit) {
    if (vec && inside && first + 8 <= limit) return *reinterpret_cast<const u32x4 *>(x);
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (inside && first + 2 * q < limit) ? x[2 * q] : 0u;
        const uint32_t hi = (inside && first + 2 * q + 1 < limit) ? x[2 * q + 1] : 0u;
        v[q] = lo | (hi << 16);
    }
    return v;
}

// Unaligned operands (a leading dimension or base that is not a multiple of
// 16 bytes) are read through a raw buffer whose base is the operand's first
// byte rounded down to 4 bytes and whose size is the operand's span: eight
// consecutive elements are one 16-byte load plus one 4-byte load at the
// enclosing dword boundary, shifted into place by two bytes when the chunk
// starts at an odd 16-bit position, instead of eight 2-byte loads.
struct UBuf {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t mis;    // bytes between the buffer base and element 0
    uint32_t limit;  // buffer size in bytes
};

__device__ inline UBuf make_ubuf(const uint16_t *x, int64_t span) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x);
    const uintptr_t base = a & ~uintptr_t(3);
    UBuf u;
    u.mis = static_cast<uint32_t>(a - base);
    u.limit = static_cast<uint32_t>(u.mis + 2 * span);
    u.rs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), 0,
                                             static_cast<int>(u.limit), 0x00020000);
    return u;
}

// Elements x[e .. e+7] with those at index >= valid (0..8) zero, in two
// halves so that a panel's loads are all in flight before any is used.
// load8u_issue issues the 16-byte and the 4-byte load at the enclosing dword
// boundary; a chunk with nothing to load, or whose 20-byte window would pass
// the end of the buffer, is sent to an offset beyond any buffer (the loads
// return zeros and cost no memory traffic).  load8u_finish shifts the loaded
// words into place, masks the elements past `valid`, and reads the chunks at
// the end of the buffer element by element (a load only partly inside the
// buffer's range may come back as all zeros).
struct Raw8 {
    u32x4 lo;
    uint32_t hi;
};

__device__ inline Raw8 load8u_issue(const UBuf &u, int64_t e, int valid) {
    const uint32_t bo = u.mis + static_cast<uint32_t>(e) * 2;
    const uint32_t dw = bo & ~3u;
    const uint32_t off = (valid > 0 && dw + 20 <= u.limit) ? dw : 0x80000000u;
    Raw8 r;
    r.lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(u.rs, off, 0, 0));
    r.hi = __builtin_amdgcn_raw_buffer_load_b32(u.rs, off + 16, 0, 0);
    return r;
}

__device__ inline u32x4 load8u_finish(const UBuf &u, const uint16_t *x, int64_t e, int valid,
                                      const Raw8 &r) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if (valid <= 0) return zero;
    const uint32_t bo = u.mis + static_cast<uint32_t>(e) * 2;
    const uint32_t dw = bo & ~3u;
    u32x4 v;
    if (dw + 20 > u.limit) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo = 2 * q < valid ? x[e + 2 * q] : 0u;
            const uint32_t hi = 2 * q + 1 < valid ? x[e + 2 * q + 1] : 0u;
            v[q] = lo | (hi << 16);
        }
        return v;
    }
    const bool odd = (bo & 2) != 0;
    v[0] = odd ? __builtin_amdgcn_alignbyte(r.lo[1], r.lo[0], 2) : r.lo[0];
    v[1] = odd ? __builtin_amdgcn_alignbyte(r.lo[2], r.lo[1], 2) : r.lo[1];
    v[2] = odd ? __builtin_amdgcn_alignbyte(r.lo[3], r.lo[2], 2) : r.lo[2];
    v[3] = odd ? __builtin_amdgcn_alignbyte(r.hi, r.lo[3], 2) : r.lo[3];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t keep = (2 * q + 1 < valid ? 0xffff0000u : 0u) | (2 * q < valid ? 0xffffu : 0u);
        v[q] &= keep;
    }
    return v;
}

// Global -> registers: one operand panel for the K step starting at k0.
//   KMAJOR: element (r, k) at X[r*ld + k]; thread loads 8 chunks of 8 k.
//   else:   element (r, k) at X[k*ld + r]; thread loads an 8 (k) x 8 (r) block.
// Chunk i of this thread starts at element e of X with `valid` elements
// inside the matrix (chunk_of).  The raw-buffer path (any alignment) issues
// every chunk's loads first (issue_panel) and assembles the chunks later
// (finish_panel), after the matrix instructions of the current step; the
// other path (operands too large for a raw buffer) loads 16-byte vectors
// when `vec`, else element by element.
template <bool KMAJOR>
__device__ inline void chunk_of(int64_t ld, int64_t rows, int64_t r0, int64_t k0, int64_t K,
                                int tid, int i, int64_t &e, int &valid) {
    if (KMAJOR) {
        const int c = tid + THREADS * i;
        const int row = c >> 3, kc = c & 7;
        const int64_t gr = r0 + row, gk = k0 + kc * 8;
        const int64_t left = K - gk;
        e = gr * ld + gk;
        valid = gr < rows ? int(left < 8 ? left : 8) : 0;
    } else {
        const int rb = tid & 31, kb = tid >> 5;
        const int64_t gk = k0 + kb * 8 + i, gr = r0 + rb * 8;
        const int64_t left = rows - gr;
        e = gk * ld + gr;
        valid = gk < K ? int(left < 8 ? left : 8) : 0;
    }
}

template <bool KMAJOR>
__device__ inline void issue_panel(const UBuf &u, int64_t ld, int64_t rows, int64_t r0,
                                   int64_t k0, int64_t K, int tid, Raw8 raw[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t e;
        int valid;
        chunk_of<KMAJOR>(ld, rows, r0, k0, K, tid, i, e, valid);
        raw[i] = load8u_issue(u, e, valid);
    }
}

template <bool KMAJOR>
__device__ inline void finish_panel(const UBuf &u, const uint16_t *X, int64_t ld, int64_t rows,
                                    int64_t r0, int64_t k0, int64_t K, int tid, const Raw8 raw[8],
                                    u32x4 v[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t e;
        int valid;
        chunk_of<KMAJOR>(ld, rows, r0, k0, K, tid, i, e, valid);
        v[i] = load8u_finish(u, X, e, valid, raw[i]);
    }
}

template <bool KMAJOR>
__device__ inline void load_panel(const uint16_t *X, int64_t ld, int64_t rows, int64_t r0,
                                  int64_t k0, int64_t K, bool vec, int tid, u32x4 v[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t e;
        int valid;
        chunk_of<KMAJOR>(ld, rows, r0, k0, K, tid, i, e, valid);
        // chunk_of's `valid` covers both the row bound and the extent along
        // the contiguous dimension: pass it as the limit
        v[i] = load8(X + e, vec, valid > 0, 0, valid);
    }
}

// 8 x 8 transpose of 16-bit elements: in[i] holds row i (8 elements along r),
// out[j] holds column j (8 elements along k).
__device__ inline void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int q = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int p = 0; p < 4; ++p) out[j][p] = __builtin_amdgcn_perm(in[2 * p + 1][q], in[2 * p][q], sel);
    }
}

// Registers -> LDS panel in the swizzled K-contiguous layout.
template <bool KMAJOR>
__device__ inline void store_panel(u32x4 *s, int tid, const u32x4 v[8]) {
    if (KMAJOR) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + THREADS * i;
            const int row = c >> 3, kc = c & 7;
            s[row * ROW_CHUNKS + (kc ^ swz(row))] = v[i];
        }
    } else {
        const int rb = tid & 31, kb = tid >> 5;
        u32x4 t[8];
        transpose8x8(v, t);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = rb * 8 + j;
            s[row * ROW_CHUNKS + (kb ^ swz(row))] = t[j];
        }
    }
}

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

template <class T, int OUT, bool A_KMAJOR, bool B_KMAJOR, bool UB>
__global__ __launch_bounds__(THREADS, 1) void hgemm_kernel(HgemmArgs p) {
    __shared__ u32x4 smem[2][2][PANEL];  // [buffer][A, B][chunk]: 128 KiB

    const TileCoord t = tile_of(p.grid, blockIdx.x);
    const uint16_t *A = p.A + t.batch * p.sA;
    const uint16_t *B = p.B + t.batch * p.sB;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = lane & 31, lk = lane >> 5;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t steps = (p.K + BK - 1) / BK;
    const int64_t span_a = A_KMAJOR ? (p.M - 1) * p.lda + p.K : (p.K - 1) * p.lda + p.M;
    const int64_t span_b = B_KMAJOR ? (p.N - 1) * p.ldb + p.K : (p.K - 1) * p.ldb + p.N;
    const UBuf ua = make_ubuf(A, UB ? span_a : 0), ub = make_ubuf(B, UB ? span_b : 0);
    u32x4 va[8], vb[8];
    Raw8 ra[8], rb[8];
    if (UB) {
        issue_panel<A_KMAJOR>(ua, p.lda, p.M, m0, 0, p.K, tid, ra);
        issue_panel<B_KMAJOR>(ub, p.ldb, p.N, n0, 0, p.K, tid, rb);
        finish_panel<A_KMAJOR>(ua, A, p.lda, p.M, m0, 0, p.K, tid, ra, va);
        finish_panel<B_KMAJOR>(ub, B, p.ldb, p.N, n0, 0, p.K, tid, rb, vb);
    } else {
        load_panel<A_KMAJOR>(A, p.lda, p.M, m0, 0, p.K, p.vec_a, tid, va);
        load_panel<B_KMAJOR>(B, p.ldb, p.N, n0, 0, p.K, p.vec_b, tid, vb);
    }
    store_panel<A_KMAJOR>(smem[0][0], tid, va);
    store_panel<B_KMAJOR>(smem[0][1], tid, vb);
    __syncthreads();

    for (int64_t s = 0; s < steps; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < steps;
        const int64_t k0 = (s + 1) * BK;
        if (more) {
            if (UB) {
                issue_panel<A_KMAJOR>(ua, p.lda, p.M, m0, k0, p.K, tid, ra);
                issue_panel<B_KMAJOR>(ub, p.ldb, p.N, n0, k0, p.K, tid, rb);
            } else {
                load_panel<A_KMAJOR>(A, p.lda, p.M, m0, k0, p.K, p.vec_a, tid, va);
                load_panel<B_KMAJOR>(B, p.ldb, p.N, n0, k0, p.K, p.vec_b, tid, vb);
            }
        }
        const u32x4 *sa = smem[cur][0];
        const u32x4 *sb = smem[cur][1];
        // Two k16 steps per iteration: a full unroll hoists all fragment reads and spills.
#pragma unroll 2
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int chunk = kk * 2 + lk;
            u32x4 a[4], b[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int ra = wm * 128 + f * 32 + lrow;
                const int rb = wn * 128 + f * 32 + lrow;
                a[f] = sa[ra * ROW_CHUNKS + (chunk ^ swz(ra))];
                b[f] = sb[rb * ROW_CHUNKS + (chunk ^ swz(rb))];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32<T>(a[i], b[j], acc[i][j]);
        }
        if (more) {
            if (UB) {
                finish_panel<A_KMAJOR>(ua, A, p.lda, p.M, m0, k0, p.K, tid, ra, va);
                finish_panel<B_KMAJOR>(ub, B, p.ldb, p.N, n0, k0, p.K, tid, rb, vb);
            }
            store_panel<A_KMAJOR>(smem[cur ^ 1][0], tid, va);
            store_panel<B_KMAJOR>(smem[cur ^ 1][1], tid, vb);
        }
        __syncthreads();
    }

    // Epilogue.  Accumulator register r of the 32 x 32 block (i, j) holds
    // row 8*(r/4) + 4*(lane/32) + r%4 and column lane%32 of that block.  The
    // 16 old values of C a lane needs for a block are loaded before any is
    // used, from element 0 of C where the element lies outside the matrix (a
    // valid address, the value discarded): a load behind each element's
    // bounds test would be waited for before the next one is issued.
    void *C = static_cast<char *>(p.C) + t.batch * p.sC * (OUT == OUT_F32 ? 4 : 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 128 + j * 32 + lrow;
            int64_t off[16];
            bool in[16];
            float old[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
                in[r] = row < p.M && col < p.N;
                off[r] = in[r] ? row * p.ldc + col : 0;
                old[r] = 0.0f;
            }
            if (p.beta != 0.0f) {
#pragma unroll
                for (int r = 0; r < 16; ++r) old[r] = load_c<OUT>(C, off[r]);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (in[r]) {
                    float v = p.alpha * acc[i][j][r];
                    if (p.beta != 0.0f) v = __builtin_fmaf(p.beta, old[r], v);
                    if (p.epi.active()) {
                        const int64_t row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
                        v = epilogue_apply(p.epi, v, t.batch, row, col);
                    }
                    store_c<OUT>(C, off[r], v);
                }
            }
        }
    }
}

template <class T, int OUT, bool AK, bool BKM>
hipError_t launch(HgemmArgs &a, hipStream_t stream) {
    void *args[] = {&a};
    const void *k = a.ubuf_a && a.ubuf_b
                        ? reinterpret_cast<const void *>(&hgemm_kernel<T, OUT, AK, BKM, true>)
                        : reinterpret_cast<const void *>(&hgemm_kernel<T, OUT, AK, BKM, false>);
    return hipLaunchKernel(k, dim3(static_cast<unsigned>(a.grid.count())), dim3(THREADS), args, 0,
                           stream);
}

template <class T, int OUT>
hipError_t launch_layout(const Problem &p, HgemmArgs &a, hipStream_t stream) {
    if (p.a_kmajor)
        return p.b_kmajor ? launch<T, OUT, true, true>(a, stream)
                          : launch<T, OUT, true, false>(a, stream);
    return p.b_kmajor ? launch<T, OUT, false, true>(a, stream)
                      : launch<T, OUT, false, false>(a, stream);
}

}  // namespace

hipError_t launch_hgemm(const Problem &p, hipStream_t stream) {
    HgemmArgs a{};
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
    a.grid = TileGrid{(p.M + BM - 1) / BM, (p.N + BN - 1) / BN, p.batch, 4, 8};
    if (a.grid.count() > 0x7fffffff) return hipErrorInvalidConfiguration;
    a.vec_a = vec16_ok(p.A, p.lda, a.sA, 2);
    a.vec_b = vec16_ok(p.B, p.ldb, a.sB, 2);
    // raw buffer sizes are 31-bit byte counts
    const int64_t span_a = p.a_kmajor ? (p.M - 1) * p.lda + p.K : (p.K - 1) * p.lda + p.M;
    const int64_t span_b = p.b_kmajor ? (p.N - 1) * p.ldb + p.K : (p.K - 1) * p.ldb + p.N;
    a.ubuf_a = 2 * span_a + 4 < (int64_t(1) << 31);
    a.ubuf_b = 2 * span_b + 4 < (int64_t(1) << 31);
    a.epi = p.epi;
    const bool bf = p.in == Elem::BF16;
    if (p.out == Elem::F32)
        return bf ? launch_layout<BF16, OUT_F32>(p, a, stream)
                  : launch_layout<F16, OUT_F32>(p, a, stream);
    return bf ? launch_layout<BF16, OUT_BF16>(p, a, stream)
              : launch_layout<F16, OUT_F16>(p, a, stream);
}

}  // namespace libgemm
