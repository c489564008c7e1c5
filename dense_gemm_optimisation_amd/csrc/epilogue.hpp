// Fused epilogue shared by the kernels: D = act(alpha*acc + beta*C_old + bias).
//
// The pages fold "GEMM + bias + activation" into the GEMM kernel ("第4章：经典
// 算子实现 —— GEMM", aiinfra.vidrealm.tech, section 7.2) and apply such
// element-wise work to the accumulators just before they are stored ("GPU
// GEMM 优化完全拆解（三）", pinghaoyang.com.cn, section on mainloop and
// epilogue).  The bias is one value per column of the caller's C; when the
// host computes a column-major C as the row-major C^T, that becomes one
// value per row of the kernel's C, which `per_row` says.  The activation is
// ReLU, max(x, 0), or GELU, x * Phi(x) with Phi the standard normal
// distribution function (see epilogue_gelu).
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace libgemm {

enum Activation : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2 };

struct Epilogue {
    const void *bias = nullptr;  // nullptr: no bias
    int64_t bias_stride = 0;     // elements between the bias vectors of batch entries
    int per_row = 0;             // bias indexed by the kernel's row (else its column)
    int bias_type = 0;           // element type of the bias: 0 fp32, 1 bf16, 2 fp16
    int act = ACT_NONE;
    // 8-bit (quantised) output: the value is multiplied by out_scale and
    // stored as OCP E4M3 (out_e5m2 = 0) or E5M2, rounded to nearest even and
    // saturated (magnitudes beyond the largest finite value, infinities
    // included, store that value; NaN stores a NaN).
    float out_scale = 1.0f;
    int out_e5m2 = 0;

    __host__ __device__ bool active() const { return bias != nullptr || act != ACT_NONE; }
};

#if defined(__HIPCC__)
__device__ inline float epilogue_bias(const Epilogue &e, int64_t batch, int64_t i) {
    const int64_t o = batch * e.bias_stride + i;
    if (e.bias_type == 0) return static_cast<const float *>(e.bias)[o];
    const uint16_t b = static_cast<const uint16_t *>(e.bias)[o];
    if (e.bias_type == 1) return __builtin_bit_cast(float, uint32_t(b) << 16);
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// GELU(x) = x * Phi(x).  Phi comes from the complementary error function,
// Phi(x) = 1 - erfc(z)/2 for x >= 0 and erfc(z)/2 for x < 0 with
// z = |x|/sqrt 2, and erfc(z) for z >= 0 from the rational approximation of
// Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erfc(z) ~ (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2) with
// t = 1 / (1 + p z), absolute error at most 1.5e-7.  It is a handful of
// instructions; a general-purpose error function inlined into the kernels
// raises their register pressure enough to make the main loops spill.
__device__ inline float epilogue_gelu(float x) {
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * z);  // v_rcp_f32, 1 ulp
    const float poly =
        t * (0.254829592f +
             t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float half_erfc = 0.5f * poly * __expf(-z * z);
    return x * (x >= 0.0f ? 1.0f - half_erfc : half_erfc);
}

__device__ inline float epilogue_act(int act, float v) {
    if (act == ACT_RELU) return v > 0.0f ? v : 0.0f;
    if (act == ACT_GELU) return epilogue_gelu(v);
    return v;
}

// v is alpha*acc + beta*C_old of element (row, col) of batch entry `batch`
// of the kernel's (row-major) C.
__device__ inline float epilogue_apply(const Epilogue &e, float v, int64_t batch, int64_t row,
                                       int64_t col) {
    if (e.bias != nullptr) v += epilogue_bias(e, batch, e.per_row ? row : col);
    return epilogue_act(e.act, v);
}

// Quantisation of the epilogue's values for an 8-bit output: the epilogue
// section of "GPU GEMM 优化完全拆解（三）" (pinghaoyang.com.cn) does the
// quantisation scaling in the write-back.  v * out_scale is clamped to the
// format's largest finite magnitude (448 for E4M3, 57344 for E5M2; a NaN
// passes through) and converted by the matrix cores' companion instruction,
// which rounds to nearest even: two values into bytes 0 and 1 of the result.
__device__ inline uint32_t epilogue_f8x2(const Epilogue &e, float v0, float v1) {
    const float maxf = e.out_e5m2 ? 57344.0f : 448.0f;
    auto clamp = [&](float x) {
        x *= e.out_scale;
        return x > maxf ? maxf : (x < -maxf ? -maxf : x);
    };
    const float a = clamp(v0), b = clamp(v1);
    const int r = e.out_e5m2 ? __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false)
                             : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return static_cast<uint32_t>(r) & 0xffffu;
}

// The bias of element `i` of the vector (a row or a column index of the
// kernel's C), or 0 outside [0, n) or without a bias: kernels load the
// values a lane needs before the stores, so the loads overlap.
__device__ inline float epilogue_bias_or_zero(const Epilogue &e, int64_t batch, int64_t i,
                                              int64_t n) {
    return (e.bias != nullptr && i < n) ? epilogue_bias(e, batch, i) : 0.0f;
}
#endif

}  // namespace libgemm
