// C <- beta * C for the calls whose product term vanishes (alpha == 0 or
// K == 0), where A and B are not read, followed by the fused epilogue (bias,
// activation) when one is requested.  With beta == 0, C is written without
// being read, so NaN or Inf already in C does not propagate.
#include "gemm_problem.hpp"

namespace libgemm {
namespace {

struct ScaleArgs {
    int64_t M, N, batch;
    float beta;
    void *C;
    int64_t ldc, sC;
    int out;  // Elem of C
    Epilogue epi;
};

__device__ inline bool out_is_8bit(int out) {
    return out == static_cast<int>(Elem::E4M3) || out == static_cast<int>(Elem::E5M2);
}

// (8-bit outputs are quantised results and are never read: beta is 0 for them)
__device__ inline float load_elem(const void *c, int64_t i, int out) {
    if (out == static_cast<int>(Elem::F32)) return static_cast<const float *>(c)[i];
    const uint16_t bits = static_cast<const uint16_t *>(c)[i];
    if (out == static_cast<int>(Elem::BF16)) return __builtin_bit_cast(float, uint32_t(bits) << 16);
    return static_cast<float>(__builtin_bit_cast(_Float16, bits));
}

__device__ inline void store_elem(void *c, int64_t i, int out, float v) {
    if (out == static_cast<int>(Elem::F32)) {
        static_cast<float *>(c)[i] = v;
    } else if (out == static_cast<int>(Elem::BF16)) {
        static_cast<uint16_t *>(c)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    } else {
        static_cast<uint16_t *>(c)[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
}

__global__ __launch_bounds__(256) void scale_kernel(ScaleArgs a) {
    const int64_t total = a.M * a.N * a.batch;
    const int64_t step = int64_t(gridDim.x) * blockDim.x;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += step) {
        const int64_t b = e / (a.M * a.N);
        const int64_t r = e - b * a.M * a.N;
        const int64_t i = r / a.N, j = r - (r / a.N) * a.N;
        const int64_t off = b * a.sC + i * a.ldc + j;
        float v = a.beta == 0.0f ? 0.0f : a.beta * load_elem(a.C, off, a.out);
        if (a.epi.active()) v = epilogue_apply(a.epi, v, b, i, j);
        if (out_is_8bit(a.out))
            static_cast<uint8_t *>(a.C)[off] = uint8_t(epilogue_f8x2(a.epi, v, 0.0f));
        else
            store_elem(a.C, off, a.out, v);
    }
}

}  // namespace

hipError_t launch_scale(const Problem &p, hipStream_t stream) {
    ScaleArgs a{p.M, p.N, p.batch, p.beta, p.C, p.ldc, p.batch > 1 ? p.sC : 0,
                static_cast<int>(p.out), p.epi};
    const int64_t total = p.M * p.N * p.batch;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(&scale_kernel),
                           dim3(static_cast<unsigned>(blocks)), dim3(256), args, 0, stream);
}

}  // namespace libgemm
