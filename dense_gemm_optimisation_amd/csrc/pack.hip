// Copy of an operand into a zero-padded, 16-byte aligned layout, so that a
// problem whose operands are not aligned can run on the direct-load kernels.
//
// The source is `outer` rows of `inner` contiguous elements (leading
// dimension ld, `batch` slices `stride` elements apart); the destination is
// `outer_p` >= outer rows of `inner_p` >= inner elements, inner_p a multiple
// of 16 bytes, slices outer_p * inner_p apart (or one slice when the source
// stride is 0: a shared operand stays shared).  Rows and columns beyond the
// source extent are zero, which is the zero fill at matrix edges that
// section 5.2 of "CUDA GEMM 矩阵乘法优化指南" (blog.zhenwei.site) does with
// predicated loads, done once per operand instead of on every tile.
//
// One thread writes one 16-byte chunk at a time.  The source chunk may start at any
// element boundary: the kernel reads the 4-byte aligned words that cover it
// with buffer loads (the buffer's range check keeps every read inside the
// operand) and shifts them into place; the last chunk of a slice is read
// element by element, so no read depends on how the range check treats a
// load that straddles the end of the buffer.
#include <cstdint>

#include <hip/hip_runtime.h>

#include "gemm_problem.hpp"

namespace libgemm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PackArgs {
    const char *src;
    char *dst;
    int64_t outer, inner, ld, stride;  // source extent, elements
    int64_t batch;
    uint32_t outer_p;                  // destination rows of one slice
    uint32_t chunks_per_row;           // inner_p * esize / 16
};

// Grid: x covers the chunks of one slice (workgroups bx of gx, a
// grid-stride loop past them), y the slices (a loop past gridDim.y).  A
// slice has fewer than 2^31 chunks (its source extent is below 2^31 bytes),
// so the index arithmetic inside a slice is 32-bit.
template <int ESIZE>
__device__ __forceinline__ void pack_run(const PackArgs &a, uint32_t bx, uint32_t gx) {
    constexpr int PER = 16 / ESIZE;  // elements per chunk
    const uint32_t per_slice = a.outer_p * a.chunks_per_row;
    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y)
    for (uint32_t r = bx * 256u + threadIdx.x; r < per_slice; r += gx * 256u) {
        const int64_t g = b * per_slice + r;  // destination chunk
        const uint32_t o = r / a.chunks_per_row;
        const int64_t e0 = int64_t(r - o * a.chunks_per_row) * PER;
        u32x4 out = {0u, 0u, 0u, 0u};
        if (o < a.outer && e0 < a.inner) {
            const char *slice = a.src + b * a.stride * ESIZE;
            // the slice as a raw buffer from its first 4-byte boundary
            const uintptr_t base = reinterpret_cast<uintptr_t>(slice);
            const uintptr_t base4 = base & ~uintptr_t(3);
            const int64_t span = (a.outer - 1) * a.ld + a.inner;  // elements of the slice
            const int64_t bytes = span * ESIZE + int64_t(base - base4);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                reinterpret_cast<void *>(base4), 0, static_cast<int>(bytes), 0x00020000);
            const int64_t off = (o * a.ld + e0) * ESIZE + int64_t(base - base4);  // byte offset
            const int64_t off4 = off & ~int64_t(3);
            const int nvalid = a.inner - e0 < PER ? int(a.inner - e0) : PER;
            if (off4 + 20 <= bytes) {
                const u32x4 w = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(off4), 0, 0));
                if (off == off4) {
                    out = w;
                } else {
                    // 16-bit elements at a 2-byte offset: one more word, then
                    // each output word takes the high half of one word and the
                    // low half of the next
                    const uint32_t w4 = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(off4 + 16), 0, 0);
                    out[0] = __builtin_amdgcn_alignbyte(w[1], w[0], 2);
                    out[1] = __builtin_amdgcn_alignbyte(w[2], w[1], 2);
                    out[2] = __builtin_amdgcn_alignbyte(w[3], w[2], 2);
                    out[3] = __builtin_amdgcn_alignbyte(w4, w[3], 2);
                }
            } else {
                // end of the slice: element by element, all inside it
                uint32_t e[PER];
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    e[i] = 0u;
                    if (i < nvalid) {
                        if (ESIZE == 2)
                            e[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, static_cast<int>(off + 2 * i), 0, 0);
                        else
                            e[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(off + 4 * i), 0, 0);
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    out[q] = ESIZE == 2 ? (e[2 * q] & 0xffffu) | (e[2 * q + 1] << 16) : e[q];
            }
            // elements past the end of the row are zero
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                if (i >= nvalid) {
                    if (ESIZE == 2)
                        out[i / 2] &= (i & 1) ? 0x0000ffffu : 0xffff0000u;
                    else
                        out[i] = 0u;
                }
            }
        }
        *reinterpret_cast<u32x4 *>(a.dst + g * 16) = out;
    }
}

template <int ESIZE>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
    pack_run<ESIZE>(a, blockIdx.x, gridDim.x);
}

// Both operands in one launch: workgroups [0, na) copy a, the rest b, so
// the two copies overlap instead of running one after the other.
template <int ESIZE>
__global__ __launch_bounds__(256) void pack2_kernel(PackArgs a, PackArgs b, uint32_t na) {
    if (blockIdx.x < na)
        pack_run<ESIZE>(a, blockIdx.x, na);
    else
        pack_run<ESIZE>(b, blockIdx.x - na, gridDim.x - na);
}

// The kernel arguments of spec s with destination dst, and the x workgroups
// and y slices a launch of it takes (0 workgroups when there is nothing to
// copy); false when a slice has 2^31 chunks or more.
bool pack_args(const PackSpec &s, void *dst, PackArgs &a, int64_t &bx, int64_t &by) {
    a = PackArgs{};
    a.src = static_cast<const char *>(s.src);
    a.dst = static_cast<char *>(dst);
    a.outer = s.outer;
    a.inner = s.inner;
    a.ld = s.ld;
    a.stride = s.stride;
    a.batch = s.stride == 0 && s.batch > 1 ? 1 : s.batch;
    const int64_t cpr = s.inner_p * s.esize / 16;
    const int64_t per_slice = s.outer_p * cpr;
    bx = by = 0;
    if (per_slice == 0 || a.batch == 0) return true;
    if (per_slice >= (int64_t(1) << 31)) return false;
    a.outer_p = static_cast<uint32_t>(s.outer_p);
    a.chunks_per_row = static_cast<uint32_t>(cpr);
    // enough workgroups to fill the chip several times over; the loops cover the rest
    bx = (per_slice + 255) / 256 < 8192 ? (per_slice + 255) / 256 : 8192;
    by = a.batch < 1024 ? a.batch : 1024;
    return true;
}

}  // namespace

int64_t packed_bytes(const PackSpec &s) {
    return (s.stride == 0 && s.batch > 1 ? 1 : s.batch) * s.outer_p * s.inner_p * s.esize;
}

hipError_t launch_pack(const PackSpec &s, void *dst, hipStream_t stream) {
    PackArgs a;
    int64_t bx, by;
    if (!pack_args(s, dst, a, bx, by)) return hipErrorInvalidValue;
    if (bx == 0) return hipSuccess;
    void *args[] = {&a};
    const void *k = s.esize == 2 ? reinterpret_cast<const void *>(&pack_kernel<2>)
                                 : reinterpret_cast<const void *>(&pack_kernel<4>);
    return hipLaunchKernel(k, dim3(static_cast<unsigned>(bx), static_cast<unsigned>(by)), dim3(256),
                           args, 0, stream);
}

// Copies of two operands of one element size, in one launch when both have
// something to copy.
hipError_t launch_pack2(const PackSpec &sa, void *dst_a, const PackSpec &sb, void *dst_b,
                        hipStream_t stream) {
    PackArgs a, b;
    int64_t ax, ay, bx, by;
    if (!pack_args(sa, dst_a, a, ax, ay) || !pack_args(sb, dst_b, b, bx, by))
        return hipErrorInvalidValue;
    if (ax == 0 || bx == 0 || sa.esize != sb.esize) {
        const hipError_t e = launch_pack(sa, dst_a, stream);
        return e != hipSuccess ? e : launch_pack(sb, dst_b, stream);
    }
    uint32_t na = static_cast<uint32_t>(ax);
    void *args[] = {&a, &b, &na};
    const void *k = sa.esize == 2 ? reinterpret_cast<const void *>(&pack2_kernel<2>)
                                  : reinterpret_cast<const void *>(&pack2_kernel<4>);
    return hipLaunchKernel(k, dim3(static_cast<unsigned>(ax + bx), static_cast<unsigned>(ay > by ? ay : by)),
                           dim3(256), args, 0, stream);
}

}  // namespace libgemm
