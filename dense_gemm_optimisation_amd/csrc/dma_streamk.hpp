// The stream-K pieces shared by the direct-load kernels of 256 x 256 tiles
// (the 16-bit one and the narrow-float one): the partial-tile slots in the
// caller's workspace, the store of a partial tile into its slot and the
// fix-up kernel that adds the pieces of each cut tile and applies the
// epilogue.
//
// Section 12.5 of "CUDA GEMM 矩阵乘法优化指南" (blog.zhenwei.site) names
// persistent kernels and Stream-K; the partition is streamk_schedule.hpp's:
// one workgroup per compute unit (G); the tiles filling whole waves of G are
// computed whole, tile w + n*G by workgroup w; the (tile, k step) iterations
// of the other tiles are split evenly over Gs workgroups; a piece covering a
// whole tile is stored through the epilogue, any other is written to the
// workgroup's slot 2w (the piece holding its last iteration) or 2w + 1 (its
// first), and dma_streamk_fixup adds the pieces of each cut tile in
// increasing workgroup order, so the sum does not depend on the order the
// workgroups ran in.
//
// Both kernels keep a wave's accumulators as FM x FN blocks of 32 x 32 with
// the operands swapped in the matrix instruction (register r of block (i, j)
// of lane l holds row l%32 and column 8*(r/4) + 4*(l/32) + r%4 of the block),
// waves laid out wave = wm*WAVES_N + wn; the slot layout and the fix-up
// follow that layout.
#pragma once

#include "dma_tile.hpp"

namespace libgemm {
namespace {

using namespace dmatile;

typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

struct DmaStreamK : StreamKSplit {
    float *partials;    // 2 * Gs slots of 256 x 256 floats
};

constexpr int SK_SLOT = BM * BN;  // floats per partial tile

// Slot `slot` as a raw buffer.  Register quad q of block (i, j) of thread
// tid is the 16 bytes at ((i*FN + j)*4 + q) * threads * 16 + tid * 16.
__device__ inline __amdgpu_buffer_rsrc_t slot_rsrc(const DmaStreamK &sk, int64_t slot) {
    return __builtin_amdgcn_make_buffer_rsrc(sk.partials + slot * SK_SLOT, 0, SK_SLOT * 4,
                                             0x00020000);
}

// Writes a piece's accumulators (unscaled) to slot `slot`.
template <int FM, int FN, int THREADS>
__device__ __forceinline__ void store_partial(const DmaStreamK &sk, int64_t slot,
                                              const f32x16 (&acc)[FM][FN]) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(sk, slot);
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            // the whole vector is reinterpreted, then indexed
            const u32x16 bits = __builtin_bit_cast(u32x16, acc[i][j]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 v = {bits[4 * q], bits[4 * q + 1], bits[4 * q + 2], bits[4 * q + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(
                    v, rs, tid * 16, ((i * FN + j) * 4 + q) * THREADS * 16, 0);
            }
        }
}

// Workgroup (local tile, piece), piece = (i*FN + j)*4 + q: sums register
// quad q of block (i, j) over the pieces of cut tile `local`, lowest
// workgroup first, and stores it; a quad is four consecutive columns of one
// row.  p is the 256 x 256 tile grid of the main kernel, with C's pointer,
// leading dimension and stride, the scalars and the epilogue.
template <int OUT, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void dma_streamk_fixup(DmaArgs p,
                                                                          DmaStreamK sk) {
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FN = WTN / 32;
    constexpr int THREADS = WAVES_M * WAVES_N * 64;
    constexpr int PIECES = (BM / WAVES_M / 32) * FN * 4;
    constexpr int BATCH = 8;  // pieces whose loads are in flight together
    const int64_t S = sk.steps;
    const int64_t local = blockIdx.x / PIECES;
    const int piece = blockIdx.x % PIECES;
    const int64_t g0 = sk_owner(sk, local * S), g1 = sk_owner(sk, local * S + S - 1);
    if (g0 == g1) return;
    const int tid = threadIdx.x;
    // Every owner but the last ends its range inside this tile, so its piece
    // is the one holding its last iteration, in slot 2g; only the last
    // owner's range may go on into the next tile.
    const int64_t slot1 = sk_slot(sk, g1, local, sk_end(sk, g1));
    f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t g = g0; g <= g1; g += BATCH) {
        u32x4 v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            // past the last piece: an offset beyond the buffer reads zeros
            const int64_t gu = g + u <= g1 ? g + u : g1;
            const uint32_t off = g + u <= g1 ? static_cast<uint32_t>(tid * 16) : 0x80000000u;
            v[u] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(slot_rsrc(sk, gu == g1 ? slot1 : 2 * gu), off,
                                                             piece * THREADS * 16, 0));
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) sum += __builtin_bit_cast(f32x4, v[u]);
    }
    const TileCoord t = tile_of(p.grid, sk.dp_tiles + local);
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int blk = piece >> 2, q = piece & 3;
    const int i = blk / FN, j = blk % FN;
    const int64_t row = t.tm * BM + wm * WTM + i * 32 + (lane & 31);
    const int64_t col0 = t.tn * BN + wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);
    if (row >= p.M) return;
    constexpr int ESZ = OUT == OUT_F32 ? 4 : 2;
    char *Cb = static_cast<char *>(p.C) + t.batch * p.sC * ESZ;
    // the lane's four columns as one aligned vector access when they are
    // all inside C and their address allows it (one 16- or 8-byte store
    // instead of four)
    char *quad = Cb + (row * p.ldc + col0) * ESZ;
    if (col0 + 3 < p.N && reinterpret_cast<uintptr_t>(quad) % (4 * ESZ) == 0) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = p.alpha * sum[e];
        if (OUT == OUT_F32) {
            if (p.beta != 0.0f) {
                const f32x4 o = *reinterpret_cast<const f32x4 *>(quad);
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(p.beta, o[e], x[e]);
            }
        } else if (p.beta != 0.0f) {
            const u32x2 o = *reinterpret_cast<const u32x2 *>(quad);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint16_t b = uint16_t(o[e / 2] >> (16 * (e % 2)));
                const float v = OUT == OUT_BF16 ? __builtin_bit_cast(float, uint32_t(b) << 16)
                                                : static_cast<float>(__builtin_bit_cast(_Float16, b));
                x[e] = __builtin_fmaf(p.beta, v, x[e]);
            }
        }
        if (p.epi.active())
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = epilogue_apply(p.epi, x[e], t.batch, row, col0 + e);
        if (OUT == OUT_F32) {
            *reinterpret_cast<f32x4 *>(quad) = x;
        } else {
            u32x2 w;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint16_t lo, hi;
                if (OUT == OUT_BF16) {
                    lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2 * h]));
                    hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2 * h + 1]));
                } else {
                    lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x[2 * h]));
                    hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x[2 * h + 1]));
                }
                w[h] = uint32_t(lo) | (uint32_t(hi) << 16);
            }
            *reinterpret_cast<u32x2 *>(quad) = w;
        }
        return;
    }
    float old[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t off = row * p.ldc + (col0 + e < p.N ? col0 + e : 0);
        old[e] = 0.0f;
        if (p.beta != 0.0f) {
            if (OUT == OUT_F32) {
                old[e] = reinterpret_cast<const float *>(Cb)[off];
            } else {
                const uint16_t b = reinterpret_cast<const uint16_t *>(Cb)[off];
                old[e] = OUT == OUT_BF16 ? __builtin_bit_cast(float, uint32_t(b) << 16)
                                         : static_cast<float>(__builtin_bit_cast(_Float16, b));
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t col = col0 + e;
        if (col >= p.N) continue;
        float x = p.alpha * sum[e];
        if (p.beta != 0.0f) x = __builtin_fmaf(p.beta, old[e], x);
        if (p.epi.active()) x = epilogue_apply(p.epi, x, t.batch, row, col);
        const int64_t off = row * p.ldc + col;
        if (OUT == OUT_F32)
            reinterpret_cast<float *>(Cb)[off] = x;
        else if (OUT == OUT_BF16)
            reinterpret_cast<uint16_t *>(Cb)[off] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
        else
            reinterpret_cast<uint16_t *>(Cb)[off] =
                __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    }
}

// The fix-up launch after a stream-K main kernel over grid `tiles` whose
// split is sk: one workgroup per (cut tile, piece); nothing when no tile was
// cut.
template <int OUT, int WAVES_M, int WAVES_N>
hipError_t launch_dma_streamk_fixup(DmaArgs &a, DmaStreamK &sk, int64_t tiles,
                                    hipStream_t stream) {
    if (sk.iters == 0) return hipSuccess;
    constexpr int PIECES = (BM / WAVES_M / 32) * (BN / WAVES_N / 32) * 4;
    const int64_t cut = tiles - sk.dp_tiles;
    void *args[] = {&a, &sk};
    return hipLaunchKernel(reinterpret_cast<const void *>(&dma_streamk_fixup<OUT, WAVES_M, WAVES_N>),
                           dim3(static_cast<unsigned>(cut * PIECES)), dim3(WAVES_M * WAVES_N * 64),
                           args, 0, stream);
}

}  // namespace
}  // namespace libgemm
