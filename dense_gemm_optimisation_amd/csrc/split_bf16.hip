// fp32 operands as sums of two bf16 pieces, for fp32 GEMMs on the bf16
// matrix instructions.
//
// "GPU GEMM 优化完全拆解（三）" (pinghaoyang.com.cn), section on numerical
// precision and why fp32 cuBLAS does not use Tensor Cores: an fp32 operand is
// split into a high and a low part of a narrower matrix format, and three of
// the four cross products are summed (the low x low one is dropped), which
// keeps the result close to fp32 at about three times the narrow format's
// instruction count.  There the narrow format is TF32; the matrix
// instructions here take bf16, so each fp32 value v becomes
//   hi = v rounded to bf16 (to nearest, ties to even; truncated instead if
//        rounding would overflow to infinity),
//   lo = (v - hi) rounded to bf16 (v - hi is exact in fp32),
// and a*b is taken as hi_a*hi_b + hi_a*lo_b + lo_a*hi_b.  Each of those
// products is exact in the fp32 accumulator (8 x 8 significant bits); the
// terms left out are at most 2^-15 |a*b|.
//
// The three products become one bf16 GEMM over K' = 3 Kp (Kp = K rounded up
// to a multiple of 8) by writing K-contiguous copies
//   A' row m    = [hi(A[m, :]) | hi(A[m, :]) | lo(A[m, :])]
//   B' column n = [hi(B[:, n]) | lo(B[:, n]) | hi(B[:, n])]
// each piece zero-padded from K to Kp.  This file writes those copies.

#include <cstdint>

#include "gemm_problem.hpp"

namespace libgemm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 pattern of v, rounded to nearest even; a finite v that would round to
// infinity is truncated instead (the largest bf16 of its sign below it), and
// a NaN stays a (quiet) NaN.
__device__ inline uint32_t bf16_hi(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;      // NaN
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    if ((r & 0x7fffu) == 0x7f80u && (u & 0x7fffffffu) != 0x7f800000u)  // overflowed
        return u >> 16;
    return r;
}

__device__ inline float bf16_value(uint32_t h) { return __builtin_bit_cast(float, h << 16); }

// the low piece: v minus its high piece, rounded to bf16; 0 for a non-finite v
__device__ inline uint32_t bf16_lo(float v, uint32_t hi) {
    if (!__builtin_isfinite(v)) return 0;
    return bf16_hi(v - bf16_value(hi));
}

struct SplitArgs {
    const float *src;
    int64_t ld, stride;   // source element (r, k): src[b*stride + r*ld + k] (kmajor) or src[b*stride + k*ld + r]
    int64_t rows, K, Kp, batch;
    uint32_t lo_pieces;   // bit j set: piece j (of three) holds the low parts
    uint16_t *dst;        // [batch][rows][3 Kp]
};

// The three destination chunks of 8 pieces (hi[e], lo[e]) at row r, k0 of
// batch entry b.
__device__ inline void store_pieces(const SplitArgs &a, int64_t b, int64_t r, int64_t k0,
                                    const uint32_t *hi, const uint32_t *lo) {
    u32x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = hi[2 * e] | (hi[2 * e + 1] << 16);
        l[e] = lo[2 * e] | (lo[2 * e + 1] << 16);
    }
    uint16_t *row = a.dst + (b * a.rows + r) * 3 * a.Kp + k0;
#pragma unroll
    for (int piece = 0; piece < 3; ++piece)
        *reinterpret_cast<u32x4 *>(row + piece * a.Kp) = (a.lo_pieces >> piece) & 1u ? l : h;
}

// K-contiguous source: one thread per 8 consecutive k of one row, which it
// reads once and writes as its three destination chunks; consecutive
// threads take consecutive chunks of a row.  VEC: the rows are 16-byte
// aligned and K is a multiple of 8, so the 8 values are two 16-byte loads.
template <bool VEC>
__global__ __launch_bounds__(256) void split_kmajor_kernel(SplitArgs a) {
    const int64_t cpr = a.Kp / 8;
    const int64_t total = a.batch * a.rows * cpr;
    for (int64_t t = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; t < total;
         t += int64_t(gridDim.x) * blockDim.x) {
        const int64_t c = t % cpr, r = (t / cpr) % a.rows, b = t / (cpr * a.rows);
        const float *s = a.src + b * a.stride + r * a.ld;
        float v[8];
        if (VEC) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(s + c * 8);
            const f32x4 y = *reinterpret_cast<const f32x4 *>(s + c * 8 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = x[e];
                v[4 + e] = y[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = c * 8 + e < a.K ? s[c * 8 + e] : 0.0f;
        }
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hi[e] = bf16_hi(v[e]);
            lo[e] = bf16_lo(v[e], hi[e]);
        }
        store_pieces(a, b, r, c * 8, hi, lo);
    }
}

// Rows-contiguous source: a workgroup takes 64 k x 64 rows, reads it along
// the rows (coalesced), splits each value once, and transposes the pieces
// through LDS so that it writes whole 16-byte chunks along k.
// VEC: the rows are a multiple of 4 and 16-byte aligned quads of them are
// read at once.
constexpr int TT = 64;
template <bool VEC>
__global__ __launch_bounds__(256) void split_rows_kernel(SplitArgs a) {
    __shared__ uint32_t pk[TT][TT + 1];  // (lo << 16) | hi of element (k, r), by [r][k]
    const int64_t tiles_r = (a.rows + TT - 1) / TT, tiles_k = (a.Kp + TT - 1) / TT;
    const int64_t tile = blockIdx.x;
    const int64_t tr = tile % tiles_r, tk = (tile / tiles_r) % tiles_k, b = tile / (tiles_r * tiles_k);
    const int64_t r0 = tr * TT, k0 = tk * TT;
    const float *s = a.src + b * a.stride;
    if (VEC) {
        const int tq = threadIdx.x % 16, ty = threadIdx.x / 16;  // 16 row quads x 16 k
#pragma unroll
        for (int kk = ty; kk < TT; kk += 16) {
            const int64_t k = k0 + kk, r = r0 + 4 * tq;
            f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (k < a.K && r < a.rows) v = *reinterpret_cast<const f32x4 *>(s + k * a.ld + r);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t hi = bf16_hi(v[q]);
                pk[4 * tq + q][kk] = hi | (bf16_lo(v[q], hi) << 16);
            }
        }
    } else {
        const int tx = threadIdx.x % TT, ty = threadIdx.x / TT;  // 64 rows x 4 k
#pragma unroll 4
        for (int kk = ty; kk < TT; kk += 4) {
            const int64_t k = k0 + kk, r = r0 + tx;
            const float v = k < a.K && r < a.rows ? s[k * a.ld + r] : 0.0f;
            const uint32_t hi = bf16_hi(v);
            pk[tx][kk] = hi | (bf16_lo(v, hi) << 16);
        }
    }
    __syncthreads();
    // 64 rows x 8 chunks of 8 k: thread -> (row, chunk), chunk fastest
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = threadIdx.x + i * 256;
        const int rr = idx / 8, cc = idx % 8;
        const int64_t r = r0 + rr, k = k0 + cc * 8;
        if (r >= a.rows || k >= a.Kp) continue;
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t x = pk[rr][cc * 8 + e];
            hi[e] = x & 0xffffu;
            lo[e] = x >> 16;
        }
        store_pieces(a, b, r, k, hi, lo);
    }
}

hipError_t launch_split(const float *src, int64_t ld, int64_t stride, bool kmajor, int64_t rows,
                        int64_t K, int64_t batch, uint32_t lo_pieces, uint16_t *dst,
                        hipStream_t stream) {
    SplitArgs a{};
    a.src = src;
    a.ld = ld;
    a.stride = stride;
    a.rows = rows;
    a.K = K;
    a.Kp = split_kp(K);
    a.batch = batch;
    a.lo_pieces = lo_pieces;
    a.dst = dst;
    void *args[] = {&a};
    if (kmajor) {
        const int64_t total = batch * rows * (a.Kp / 8);
        int64_t blocks = (total + 255) / 256;
        if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
        const bool vec = K % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 && ld % 4 == 0 &&
                         (batch == 1 || stride % 4 == 0);
        return hipLaunchKernel(vec ? reinterpret_cast<const void *>(&split_kmajor_kernel<true>)
                                   : reinterpret_cast<const void *>(&split_kmajor_kernel<false>),
                               dim3(static_cast<unsigned>(blocks)), dim3(256), args, 0, stream);
    }
    const int64_t tiles = batch * ((rows + TT - 1) / TT) * ((a.Kp + TT - 1) / TT);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool vec = rows % 4 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 && ld % 4 == 0 &&
                     (batch == 1 || stride % 4 == 0);
    return hipLaunchKernel(vec ? reinterpret_cast<const void *>(&split_rows_kernel<true>)
                               : reinterpret_cast<const void *>(&split_rows_kernel<false>),
                           dim3(static_cast<unsigned>(tiles)), dim3(256), args, 0, stream);
}

}  // namespace

int64_t split_kp(int64_t K) { return (K + 7) / 8 * 8; }

int64_t split_bytes(int64_t rows, int64_t K, int64_t batch) {
    return (batch * rows * 3 * split_kp(K) * 2 + 255) / 256 * 256;
}

// A' pieces (hi, hi, lo) and B' pieces (hi, lo, hi): piece j of A' meets
// piece j of B' in the K' sum.
hipError_t launch_split_a(const float *A, int64_t lda, int64_t sA, bool kmajor, int64_t M,
                          int64_t K, int64_t batch, uint16_t *dst, hipStream_t stream) {
    return launch_split(A, lda, sA, kmajor, M, K, batch, 0x4u, dst, stream);
}

hipError_t launch_split_b(const float *B, int64_t ldb, int64_t sB, bool kmajor, int64_t N,
                          int64_t K, int64_t batch, uint16_t *dst, hipStream_t stream) {
    return launch_split(B, ldb, sB, kmajor, N, K, batch, 0x2u, dst, stream);
}

}  // namespace libgemm
