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
//
// The file is compiled once per (input type, order of A) with
// LIBGEMM_HGEMM_PART = 0..3 set, each object holding that part's kernels and
// their launchers, so the parts build in parallel; part 0 also holds the
// host entry points.  Without the macro one object holds everything.
#include "gemm_problem.hpp"
#include "tile_schedule.hpp"

#ifndef LIBGEMM_HGEMM_PART
#define LIBGEMM_HGEMM_PART -1
#endif
#define LIBGEMM_HGEMM_HAS(part) (LIBGEMM_HGEMM_PART < 0 || LIBGEMM_HGEMM_PART == (part))

namespace libgemm {

// Arguments of the kernels, shared by the objects of the parts (named, so
// that the launchers of one part can be called from another).
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

struct StreamK : StreamKSplit {
    float *partials;    // 2 * Gs slots of 256 x 256 floats
};

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int THREADS = 256;
constexpr int ROW_CHUNKS = BK / 8;         // 16-byte chunks per LDS row
constexpr int PANEL = BM * ROW_CHUNKS;     // chunks per operand panel (32 KiB)
static_assert(BM == BN, "both panels share one layout");

constexpr int OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2;


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

// Interior steps.  A panel step is interior when every chunk lies inside the
// matrix and the 20-byte window of its two loads inside the buffer: all 256
// rows exist, the 64 k exist, and where the last row (KMAJOR) or the last k
// (otherwise) is touched, two more elements follow it (a chunk's window ends
// at most 10 elements past its start).  Such a step needs no bounds, masks or
// tail handling: each lane keeps one byte offset per tile (chunk 0 at k = 0,
// from the buffer base) and adds the uniform rest.
template <bool KMAJOR>
__device__ inline bool panel_interior(int64_t rows, int64_t r0, int64_t k0, int64_t K) {
    if (r0 + BM > rows || k0 + BK > K) return false;
    return KMAJOR ? (r0 + BM < rows || k0 + BK + 2 <= K) : (k0 + BK < K || r0 + BM + 2 <= rows);
}

// The lane's byte offset of chunk 0 at k = 0 (meaningful where the panel is
// interior; it may wrap elsewhere and is then not used).
template <bool KMAJOR>
__device__ inline uint32_t lane_offset(const UBuf &u, int64_t ld, int64_t r0, int tid) {
    const int64_t e = KMAJOR ? (r0 + (tid >> 3)) * ld + 8 * (tid & 7)
                             : 8 * (tid >> 5) * ld + r0 + 8 * (tid & 31);
    return u.mis + 2 * static_cast<uint32_t>(e);
}

// KMAJOR: chunk i sits 32*i rows below chunk 0, and the step adds k0, both
// multiples of four bytes, so the dword-aligned offset splits into the lane's
// constant part (voffset) and a uniform part (soffset), and the shift is the
// lane's own.  Otherwise chunk i is i rows of k below chunk 0: the uniform
// part can change the offset's alignment and is added per chunk.
template <bool KMAJOR>
__device__ inline void issue_panel_fast(const UBuf &u, uint32_t lane, int64_t ld, int64_t k0,
                                        Raw8 raw[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t voff, soff;
        if (KMAJOR) {
            voff = lane & ~3u;
            soff = static_cast<uint32_t>(2 * k0 + 64 * ld * i);
        } else {
            voff = (lane + static_cast<uint32_t>(2 * (k0 + i) * ld)) & ~3u;
            soff = 0;
        }
        raw[i].lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(u.rs, voff, soff, 0));
        raw[i].hi = __builtin_amdgcn_raw_buffer_load_b32(u.rs, voff + 16, soff, 0);
    }
}

template <bool KMAJOR>
__device__ inline void finish_panel_fast(uint32_t lane, int64_t ld, int64_t k0, const Raw8 raw[8],
                                         u32x4 v[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // v_alignbyte shifts by the low two bits of its third operand: 0 or 2
        const uint32_t sh = KMAJOR ? lane : lane + static_cast<uint32_t>(2 * (k0 + i) * ld);
        v[i][0] = __builtin_amdgcn_alignbyte(raw[i].lo[1], raw[i].lo[0], sh);
        v[i][1] = __builtin_amdgcn_alignbyte(raw[i].lo[2], raw[i].lo[1], sh);
        v[i][2] = __builtin_amdgcn_alignbyte(raw[i].lo[3], raw[i].lo[2], sh);
        v[i][3] = __builtin_amdgcn_alignbyte(raw[i].hi, raw[i].lo[3], sh);
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

// threadIdx.x behind an empty volatile statement: values derived from it
// are then recomputed where they are used instead of being hoisted out of
// the stream-K kernel's loop over pieces, where they would stay live across
// the k-step loop and push it into spilling.  (In the one-tile kernel it
// changes nothing.)
__device__ inline int opaque_tid() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
}

// Accumulates k steps [kb, ke) (BK = 64 k each) of tile t into acc:
// register-staged double buffering through the two LDS buffers, one barrier
// per step; on return every wave is past the last barrier, so the buffers
// are free.
template <class T, bool A_KMAJOR, bool B_KMAJOR, bool UB>
__device__ __forceinline__ void tile_steps(const HgemmArgs &p, u32x4 (*smem)[2][PANEL],
                                           const TileCoord &t, int64_t kb, int64_t ke,
                                           f32x16 (&acc)[4][4]) {
    const int tid = opaque_tid();
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = lane & 31, lk = lane >> 5;
    const uint16_t *A = p.A + t.batch * p.sA;
    const uint16_t *B = p.B + t.batch * p.sB;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int64_t span_a = A_KMAJOR ? (p.M - 1) * p.lda + p.K : (p.K - 1) * p.lda + p.M;
    const int64_t span_b = B_KMAJOR ? (p.N - 1) * p.ldb + p.K : (p.K - 1) * p.ldb + p.N;
    const UBuf ua = make_ubuf(A, UB ? span_a : 0), ub = make_ubuf(B, UB ? span_b : 0);
    u32x4 va[8], vb[8];
    Raw8 ra[8], rb[8];
    const uint32_t lane_a = UB ? lane_offset<A_KMAJOR>(ua, p.lda, m0, tid) : 0u;
    const uint32_t lane_b = UB ? lane_offset<B_KMAJOR>(ub, p.ldb, n0, tid) : 0u;
    // whether the panels of the step starting at k are interior (uniform)
    auto interior = [&](int64_t k) {
        return panel_interior<A_KMAJOR>(p.M, m0, k, p.K) && panel_interior<B_KMAJOR>(p.N, n0, k, p.K);
    };
    if (UB) {
        if (interior(kb * BK)) {
            issue_panel_fast<A_KMAJOR>(ua, lane_a, p.lda, kb * BK, ra);
            issue_panel_fast<B_KMAJOR>(ub, lane_b, p.ldb, kb * BK, rb);
            finish_panel_fast<A_KMAJOR>(lane_a, p.lda, kb * BK, ra, va);
            finish_panel_fast<B_KMAJOR>(lane_b, p.ldb, kb * BK, rb, vb);
        } else {
            issue_panel<A_KMAJOR>(ua, p.lda, p.M, m0, kb * BK, p.K, tid, ra);
            issue_panel<B_KMAJOR>(ub, p.ldb, p.N, n0, kb * BK, p.K, tid, rb);
            finish_panel<A_KMAJOR>(ua, A, p.lda, p.M, m0, kb * BK, p.K, tid, ra, va);
            finish_panel<B_KMAJOR>(ub, B, p.ldb, p.N, n0, kb * BK, p.K, tid, rb, vb);
        }
    } else {
        load_panel<A_KMAJOR>(A, p.lda, p.M, m0, kb * BK, p.K, p.vec_a, tid, va);
        load_panel<B_KMAJOR>(B, p.ldb, p.N, n0, kb * BK, p.K, p.vec_b, tid, vb);
    }
    store_panel<A_KMAJOR>(smem[0][0], tid, va);
    store_panel<B_KMAJOR>(smem[0][1], tid, vb);
    __syncthreads();

    for (int64_t s = kb; s < ke; ++s) {
        const int cur = (s - kb) & 1;
        const bool more = s + 1 < ke;
        const int64_t k0 = (s + 1) * BK;
        const bool fast = UB && more && interior(k0);
        if (more) {
            if (fast) {
                issue_panel_fast<A_KMAJOR>(ua, lane_a, p.lda, k0, ra);
                issue_panel_fast<B_KMAJOR>(ub, lane_b, p.ldb, k0, rb);
            } else if (UB) {
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
            if (fast) {
                finish_panel_fast<A_KMAJOR>(lane_a, p.lda, k0, ra, va);
                finish_panel_fast<B_KMAJOR>(lane_b, p.ldb, k0, rb, vb);
            } else if (UB) {
                finish_panel<A_KMAJOR>(ua, A, p.lda, p.M, m0, k0, p.K, tid, ra, va);
                finish_panel<B_KMAJOR>(ub, B, p.ldb, p.N, n0, k0, p.K, tid, rb, vb);
            }
            store_panel<A_KMAJOR>(smem[cur ^ 1][0], tid, va);
            store_panel<B_KMAJOR>(smem[cur ^ 1][1], tid, vb);
        }
        __syncthreads();
    }
}

// Epilogue of registers [r0, r0 + NR) of accumulator block (i, j) of the
// thread's wave in tile t, v[q] holding register r0 + q (a vector of at least
// NR floats), for the stream-K fix-up: the same arithmetic as tile_store
// (below), alpha * v (+ beta * C_old, bias, activation) into C.  Accumulator register r of a 32 x 32 block holds row
// 8*(r/4) + 4*(lane/32) + r%4 and column lane%32 of that block.  The old
// values of C are loaded before any is used, from element 0 of C where the
// element lies outside the matrix (a valid address, the value discarded): a
// load behind each element's bounds test would be waited for before the next
// one is issued.
template <int OUT, int NR, class V>
__device__ __forceinline__ void store_regs(const HgemmArgs &p, const TileCoord &t, int i, int j,
                                           int r0, const V &v) {
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int tid = opaque_tid();
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = lane & 31, lk = lane >> 5;
    void *C = static_cast<char *>(p.C) + t.batch * p.sC * (OUT == OUT_F32 ? 4 : 2);
    const int64_t col = n0 + wn * 128 + j * 32 + lrow;
    int64_t off[NR];
    bool in[NR];
    float old[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
        const int r = r0 + q;
        const int64_t row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
        in[q] = row < p.M && col < p.N;
        off[q] = in[q] ? row * p.ldc + col : 0;
        old[q] = 0.0f;
    }
    if (p.beta != 0.0f) {
#pragma unroll
        for (int q = 0; q < NR; ++q) old[q] = load_c<OUT>(C, off[q]);
    }
#pragma unroll
    for (int q = 0; q < NR; ++q) {
        if (in[q]) {
            float x = p.alpha * v[q];
            if (p.beta != 0.0f) x = __builtin_fmaf(p.beta, old[q], x);
            if (p.epi.active()) {
                const int r = r0 + q;
                const int64_t row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
                x = epilogue_apply(p.epi, x, t.batch, row, col);
            }
            store_c<OUT>(C, off[q], x);
        }
    }
}

// Epilogue of tile t: alpha * acc (+ beta * C_old, bias, activation) into C.
template <int OUT>
__device__ __forceinline__ void tile_store(const HgemmArgs &p, const TileCoord &t,
                                           const f32x16 (&acc)[4][4]) {
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int tid = opaque_tid();
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = lane & 31, lk = lane >> 5;
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

template <class T, int OUT, bool A_KMAJOR, bool B_KMAJOR, bool UB>
__global__ __launch_bounds__(THREADS, 1) void hgemm_kernel(HgemmArgs p) {
    __shared__ u32x4 smem[2][2][PANEL];  // [buffer][A, B][chunk]: 128 KiB
    const TileCoord t = tile_of(p.grid, blockIdx.x);
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    tile_steps<T, A_KMAJOR, B_KMAJOR, UB>(p, smem, t, 0, (p.K + BK - 1) / BK, acc);
    tile_store<OUT>(p, t, acc);
}

// Stream-K schedule (the persistent / stream-K tile scheduler of section 12.5
// of "CUDA GEMM 矩阵乘法优化指南", blog.zhenwei.site), in two kernels.
//
// hgemm_streamk_kernel runs one workgroup per compute unit (G of them).  The
// tiles that fill whole waves of G workgroups, in the grouped order of
// tile_of, are computed as in hgemm_kernel, tile w + n*G by workgroup w.  The
// rest, the last partial wave of T_r tiles, is cut into its W = T_r * S
// (tile, k step) iterations, each tile's steps in k order, and workgroup
// w < Gs = min(G, W) takes the contiguous iterations [w*W/Gs, (w+1)*W/Gs).
// A piece that covers a whole tile is stored through the epilogue; any other
// is a partial tile, written to the workspace.  Only the first and the last
// piece of a range can be partial, so workgroup w owns two slots: 2w for the
// piece holding its last iteration, 2w + 1 for the one holding its first.
//
// hgemm_streamk_fixup then finishes each tile that was cut: 64 workgroups per
// tile, each summing one quarter of one 32 x 32 block per wave over the
// tile's pieces in increasing workgroup order (a fixed order, so results do
// not change from run to run) and applying the epilogue.  The kernels
// exchange data only across the launch boundary on one stream: no workgroup
// waits for another.

constexpr int SK_SLOT = BM * BN;  // floats per partial tile

// Slot `slot` of the partial tiles as a raw buffer.  Within a slot, register
// quad q (registers 4q .. 4q+3) of block (i, j) of thread tid is the 16 bytes
// at ((i*4 + j)*4 + q) * THREADS * 16 + tid * 16: every store and load of a
// wave covers 1 KiB of consecutive bytes.
__device__ inline __amdgpu_buffer_rsrc_t slot_rsrc(const StreamK &sk, int64_t slot) {
    return __builtin_amdgcn_make_buffer_rsrc(sk.partials + slot * SK_SLOT, 0, SK_SLOT * 4,
                                             0x00020000);
}

// The schedule's indices are the same in every lane, but 64-bit divisions
// leave them in vector registers, where they would stay live across the
// k-step loop and push it into spilling: they are moved to scalar registers.
__device__ inline int64_t sk_uniform(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(uint64_t(x) >> 32));
    return static_cast<int64_t>((uint64_t(hi) << 32) | lo);
}

template <class T, int OUT, bool A_KMAJOR, bool B_KMAJOR, bool UB>
__global__ __launch_bounds__(THREADS, 1) void hgemm_streamk_kernel(HgemmArgs p, StreamK sk) {
    __shared__ u32x4 smem[2][2][PANEL];
    // Logical workgroup w: the hardware id regrouped per XCD (xcd_remap), so
    // that the workgroups of one die take consecutive tiles and ranges and
    // share their panels in its L2.
    const int64_t G = gridDim.x, S = sk.steps;
    const int64_t w = sk_uniform(xcd_remap(blockIdx.x, G, 8));
    const int64_t n_dp = sk_uniform(sk_whole_tiles(sk, w, G));
    const int64_t begin = sk_uniform(sk_begin(sk, w));
    const int64_t end = sk_uniform(sk_end(sk, w));
    int64_t it = begin;
    for (int64_t item = 0;; ++item) {
        int64_t tile, kb, ke, local = 0;
        if (item < n_dp) {
            tile = w + item * G;
            kb = 0;
            ke = S;
        } else {
            if (it >= end) break;
            local = sk_uniform(it / S);
            const StreamKPiece pc = sk_piece(sk, local, it, end);
            kb = pc.kb;
            ke = pc.ke;
            tile = sk.dp_tiles + local;
            it = local * S + ke;
        }
        TileCoord t = tile_of(p.grid, tile);
        t.batch = sk_uniform(t.batch);
        t.tm = sk_uniform(t.tm);
        t.tn = sk_uniform(t.tn);
        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        tile_steps<T, A_KMAJOR, B_KMAJOR, UB>(p, smem, t, kb, ke, acc);
        if (kb == 0 && ke == S) {
            tile_store<OUT>(p, t, acc);
        } else {
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(sk, sk_slot(sk, w, local, end));
            const int tid = opaque_tid();
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // the whole vector is reinterpreted, then indexed: a bit
                    // cast of one element of it reads element 0 with this
                    // compiler
                    const u32x16 bits = __builtin_bit_cast(u32x16, acc[i][j]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const u32x4 v = {bits[4 * q], bits[4 * q + 1], bits[4 * q + 2],
                                         bits[4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(
                            v, rs, tid * 16, ((i * 4 + j) * 4 + q) * THREADS * 16, 0);
                    }
                }
        }
    }
}

// Workgroup (local tile, piece): piece = (i*4 + j)*4 + q sums register quad q
// of block (i, j) over the pieces of local tile `local` of the cut tiles,
// lowest workgroup first, and stores it.  A tile inside one range was stored
// whole by hgemm_streamk_kernel and its workgroups return at once.
constexpr int SK_BATCH = 8;  // pieces whose loads are in flight together

template <int OUT>
__global__ __launch_bounds__(THREADS) void hgemm_streamk_fixup(HgemmArgs p, StreamK sk) {
    const int64_t S = sk.steps;
    const int64_t local = blockIdx.x / 64;
    const int piece = blockIdx.x % 64;
    const int64_t g0 = sk_owner(sk, local * S), g1 = sk_owner(sk, local * S + S - 1);
    if (g0 == g1) return;
    const int tid = threadIdx.x;
    // every owner but the last holds its last iteration here (slot 2g)
    const int64_t slot1 = sk_slot(sk, g1, local, sk_end(sk, g1));
    f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t g = g0; g <= g1; g += SK_BATCH) {
        u32x4 v[SK_BATCH];
#pragma unroll
        for (int u = 0; u < SK_BATCH; ++u) {
            // past the last piece: an offset beyond the buffer reads zeros
            const int64_t gu = g + u <= g1 ? g + u : g1;
            const uint32_t off = g + u <= g1 ? static_cast<uint32_t>(tid * 16) : 0x80000000u;
            v[u] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(slot_rsrc(sk, gu == g1 ? slot1 : 2 * gu), off,
                                                             piece * THREADS * 16, 0));
        }
#pragma unroll
        for (int u = 0; u < SK_BATCH; ++u) sum += __builtin_bit_cast(f32x4, v[u]);
    }
    const TileCoord t = tile_of(p.grid, sk.dp_tiles + local);
    const int blk = piece >> 2, q = piece & 3;
    store_regs<OUT, 4>(p, t, blk >> 2, blk & 3, 4 * q, sum);
}

// Launchers of one part: input type T, order of A (AK).  The kernels of a
// part are instantiated in its object only.
template <class T, int OUT, bool AK, bool BKM>
hipError_t launch(HgemmArgs &a, hipStream_t stream) {
    void *args[] = {&a};
    const void *k = a.ubuf_a && a.ubuf_b
                        ? reinterpret_cast<const void *>(&hgemm_kernel<T, OUT, AK, BKM, true>)
                        : reinterpret_cast<const void *>(&hgemm_kernel<T, OUT, AK, BKM, false>);
    return hipLaunchKernel(k, dim3(static_cast<unsigned>(a.grid.count())), dim3(THREADS), args, 0,
                           stream);
}

template <class T, int OUT, bool AK>
hipError_t launch_b(const Problem &p, HgemmArgs &a, hipStream_t stream) {
    return p.b_kmajor ? launch<T, OUT, AK, true>(a, stream) : launch<T, OUT, AK, false>(a, stream);
}

template <class T, int OWN, bool AK>
hipError_t launch_part(const Problem &p, HgemmArgs &a, hipStream_t stream) {
    return p.out == Elem::F32 ? launch_b<T, OUT_F32, AK>(p, a, stream)
                              : launch_b<T, OWN, AK>(p, a, stream);
}

// Only the raw-buffer variant exists on this schedule (hgemm_streamk_eligible
// requires operand spans that fit a raw buffer).
template <class T, int OUT, bool AK, bool BKM>
hipError_t launch_sk(HgemmArgs &a, StreamK &sk, int64_t grid, hipStream_t stream) {
    void *args[] = {&a, &sk};
    const void *k = reinterpret_cast<const void *>(&hgemm_streamk_kernel<T, OUT, AK, BKM, true>);
    return hipLaunchKernel(k, dim3(static_cast<unsigned>(grid)), dim3(THREADS), args, 0, stream);
}

template <class T, int OUT, bool AK>
hipError_t launch_sk_b(const Problem &p, HgemmArgs &a, StreamK &sk, int64_t grid,
                       hipStream_t stream) {
    const hipError_t e = p.b_kmajor ? launch_sk<T, OUT, AK, true>(a, sk, grid, stream)
                                    : launch_sk<T, OUT, AK, false>(a, sk, grid, stream);
    if (e != hipSuccess || sk.iters == 0) return e;
    void *args[] = {&a, &sk};
    const int64_t cut = a.grid.count() - sk.dp_tiles;
    return hipLaunchKernel(reinterpret_cast<const void *>(&hgemm_streamk_fixup<OUT>),
                           dim3(static_cast<unsigned>(cut * 64)), dim3(THREADS), args, 0, stream);
}

template <class T, int OWN, bool AK>
hipError_t launch_sk_part(const Problem &p, HgemmArgs &a, StreamK &sk, int64_t grid,
                          hipStream_t stream) {
    return p.out == Elem::F32 ? launch_sk_b<T, OUT_F32, AK>(p, a, sk, grid, stream)
                              : launch_sk_b<T, OWN, AK>(p, a, sk, grid, stream);
}

}  // namespace

// Part k = (input type, order of A): 0 bf16 with A along M, 1 bf16 with A
// along K, 2 and 3 the same for fp16.
template <int PART>
hipError_t hgemm_part(const Problem &p, HgemmArgs &a, hipStream_t stream);
template <int PART>
hipError_t hgemm_streamk_part(const Problem &p, HgemmArgs &a, StreamK &sk, int64_t grid,
                              hipStream_t stream);

#define LIBGEMM_HGEMM_PART_DEF(part, T, OWN, AK)                                              \
    template <>                                                                                \
    hipError_t hgemm_part<part>(const Problem &p, HgemmArgs &a, hipStream_t stream) {          \
        return launch_part<T, OWN, AK>(p, a, stream);                                          \
    }                                                                                          \
    template <>                                                                                \
    hipError_t hgemm_streamk_part<part>(const Problem &p, HgemmArgs &a, StreamK &sk,           \
                                        int64_t grid, hipStream_t stream) {                    \
        return launch_sk_part<T, OWN, AK>(p, a, sk, grid, stream);                             \
    }

#if LIBGEMM_HGEMM_HAS(0)
LIBGEMM_HGEMM_PART_DEF(0, BF16, OUT_BF16, false)
#endif
#if LIBGEMM_HGEMM_HAS(1)
LIBGEMM_HGEMM_PART_DEF(1, BF16, OUT_BF16, true)
#endif
#if LIBGEMM_HGEMM_HAS(2)
LIBGEMM_HGEMM_PART_DEF(2, F16, OUT_F16, false)
#endif
#if LIBGEMM_HGEMM_HAS(3)
LIBGEMM_HGEMM_PART_DEF(3, F16, OUT_F16, true)
#endif

#if LIBGEMM_HGEMM_PART <= 0
namespace {

HgemmArgs make_args(const Problem &p, int32_t xcds) {
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
    a.grid = TileGrid{(p.M + BM - 1) / BM, (p.N + BN - 1) / BN, p.batch, 4, xcds};
    a.vec_a = vec16_ok(p.A, p.lda, a.sA, 2);
    a.vec_b = vec16_ok(p.B, p.ldb, a.sB, 2);
    // raw buffer sizes are 31-bit byte counts
    const int64_t span_a = p.a_kmajor ? (p.M - 1) * p.lda + p.K : (p.K - 1) * p.lda + p.M;
    const int64_t span_b = p.b_kmajor ? (p.N - 1) * p.ldb + p.K : (p.K - 1) * p.ldb + p.N;
    a.ubuf_a = 2 * span_a + 4 < (int64_t(1) << 31);
    a.ubuf_b = 2 * span_b + 4 < (int64_t(1) << 31);
    a.epi = p.epi;
    return a;
}

// Cost of the partial-tile exchange (writing the pieces, the fix-up kernel),
// in k steps of one 256 x 256 tile, measured on MI355X.
constexpr int64_t SK_EXCHANGE_STEPS = 4;

}  // namespace

hipError_t launch_hgemm(const Problem &p, hipStream_t stream) {
    HgemmArgs a = make_args(p, 8);
    if (a.grid.count() > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int part = (p.in == Elem::BF16 ? 0 : 2) + (p.a_kmajor ? 1 : 0);
    switch (part) {
    case 0: return hgemm_part<0>(p, a, stream);
    case 1: return hgemm_part<1>(p, a, stream);
    case 2: return hgemm_part<2>(p, a, stream);
    default: return hgemm_part<3>(p, a, stream);
    }
}

// Step time over partial-tile time for streamk_groups (5.2 us per k step of the general kernel at 4096^3, 0.13 us per partial tile).
#ifndef LIBGEMM_SK_RATIO
#define LIBGEMM_SK_RATIO 40
#endif

// Stream-K pays off when the tiles leave the last wave of workgroups (one
// per compute unit) partly idle, and when the steps it saves there exceed the
// cost of exchanging partial tiles: the last wave then takes
// ceil(T_r * S / G) steps per workgroup instead of S.  The model uses
// HGEMM_STREAMK_MAX_GRID compute units (MI355X has 256).
bool hgemm_streamk_eligible(const Problem &p, bool force) {
    if (p.in != Elem::BF16 && p.in != Elem::F16) return false;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.batch;
    const int64_t steps = (p.K + BK - 1) / BK;
    const int64_t g = HGEMM_STREAMK_MAX_GRID;
    const int64_t cut = tiles % g;
    if (cut == 0 || tiles >= (int64_t(1) << 24) || steps >= (int64_t(1) << 24)) return false;
    const int64_t tail = (cut * steps + g - 1) / g;
    const HgemmArgs a = make_args(p, 1);
    return a.ubuf_a && a.ubuf_b && (force || steps - tail > SK_EXCHANGE_STEPS);
}

namespace {

// The split over HGEMM_STREAMK_MAX_GRID workgroups (one per compute unit of
// MI355X; on a part with fewer units the schedule is still correct).
StreamKSplit hg_streamk_split(const Problem &p) {
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.batch;
    return streamk_split(tiles, (p.K + BK - 1) / BK, HGEMM_STREAMK_MAX_GRID, LIBGEMM_SK_RATIO);
}

}  // namespace

int64_t hgemm_streamk_bytes(const Problem &p) {
    return 2 * hg_streamk_split(p).groups * int64_t(SK_SLOT) * 4;
}

hipError_t launch_hgemm_streamk(const Problem &p, void *workspace, hipStream_t stream) {
    HgemmArgs a = make_args(p, 1);  // the work order itself spreads tiles over the dies
    StreamK sk{};
    static_cast<StreamKSplit &>(sk) = hg_streamk_split(p);
    sk.partials = static_cast<float *>(workspace);
    const int64_t grid = streamk_grid(sk, HGEMM_STREAMK_MAX_GRID);
    if (grid == 0) return hipSuccess;
    const int part = (p.in == Elem::BF16 ? 0 : 2) + (p.a_kmajor ? 1 : 0);
    switch (part) {
    case 0: return hgemm_streamk_part<0>(p, a, sk, grid, stream);
    case 1: return hgemm_streamk_part<1>(p, a, sk, grid, stream);
    case 2: return hgemm_streamk_part<2>(p, a, sk, grid, stream);
    default: return hgemm_streamk_part<3>(p, a, sk, grid, stream);
    }
}

#endif  // LIBGEMM_HGEMM_PART <= 0

}  // namespace libgemm
