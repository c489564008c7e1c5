/*
 * libgemm — dense general matrix multiply on AMD Instinct MI355X (gfx950).
 *
 *   C <- alpha * op(A) * op(B) + beta * C
 *
 * with op(A) an M x K matrix, op(B) a K x N matrix and C an M x N matrix.
 * This is the GEMM of "CUDA GEMM 矩阵乘法优化指南" (blog.zhenwei.site),
 * section 2.1 (C = alpha x A x B + beta x C, A M x K, B K x N, C M x N).
 * The scalars and the argument order (dimensions, alpha, A and its leading
 * dimension, B and its leading dimension, beta, C and its leading dimension)
 * follow the BLAS call shown in section 7.1 of "第4章：经典算子实现 —— GEMM"
 * (aiinfra.vidrealm.tech), with per-operand storage orders in place of the
 * column-major-only convention of that library.
 *
 * Entry points
 *   gemm_f32   fp32 inputs, fp32 output, fp32 arithmetic (on the matrix cores).
 *   gemm_f32_valu  the same product on the vector ALUs (register-tiled).
 *   gemm_f32_bf16x3  fp32 inputs and output, computed as three bf16 products
 *              of split operands on the bf16 matrix cores (a caller
 *              workspace holds the split copies; accuracy below).
 *   gemm_bf16  bf16 inputs, fp32 accumulation on the matrix cores, output in
 *              bf16 (c_dtype = GEMM_DTYPE_SAME) or fp32 (GEMM_DTYPE_F32).
 *   gemm_f16   the same for IEEE fp16 inputs.
 *   gemm_f32_bias_act, gemm_bf16_bias_act, gemm_f16_bias_act
 *              the same products with a fused epilogue: a per-column bias
 *              and an activation applied before the store (see below).
 *   gemm_bf16_quant, gemm_f16_quant  the fused epilogue followed by a
 *              scale and a saturating store as 8-bit floats (E4M3/E5M2).
 *   gemm_f8    8-bit float inputs (OCP E4M3 or E5M2, each operand in its own
 *              format), fp32 accumulation, output in fp32, bf16 or fp16.
 *   gemm_mx    block-scaled inputs (MXFP8, MXFP6, MXFP4: one E8M0 scale per
 *              32 elements along K), fp32 accumulation, output in fp32,
 *              bf16 or fp16.
 *   gemm_f32_ws, gemm_bf16_ws, gemm_f16_ws, gemm_f8_ws, gemm_mx_ws
 *              the products with a caller-provided workspace, which lets
 *              the library copy unaligned operands into aligned ones and
 *              run the stream-K schedule (see below); gemm_workspace_size
 *              gives the bytes it needs.
 *   gemm_bf16_noalloc  gemm_bf16_ws on the library's own scratch memory.
 *   gemm_kernel_name, gemm_f8_kernel_name, gemm_mx_kernel_name,
 *   gemm_kernel_name_ws, gemm_f8_kernel_name_ws, gemm_mx_kernel_name_ws,
 *   gemm_kernel_name_bf16x3, gemm_kernel_name_quant
 *              which kernel
 *              a GEMM call with the
 *              given arguments would launch (host only; for tests and
 *              profiling).
 *   gemm_test_switches  kernel-choice overrides for testing.
 *
 * Layout
 *   Each matrix has its own order.  Element (i, k) of A is at
 *   A[i*lda + k] when orderA == GEMM_ROW_MAJOR and at A[k*lda + i] when
 *   GEMM_COL_MAJOR; element (k, j) of B and (i, j) of C likewise.  A leading
 *   dimension must be at least max(1, extent of the contiguous dimension).
 *   Every pointer must be a multiple of its element size; any leading
 *   dimension is accepted.  16-byte aligned A and B (bases, leading
 *   dimensions and strides multiples of 16 bytes) take the fast direct-load
 *   path, anything else a slower exact path (or, with a workspace, aligned
 *   copies made first); C is read and written in 16-byte chunks at any
 *   leading dimension.
 *
 * Batch
 *   `batch` independent problems; problem b uses A + b*strideA, B + b*strideB
 *   and C + b*strideC (strides in elements, >= 0).  A stride of 0 for A or B
 *   shares one matrix across the batch.  C slices must not overlap each
 *   other (strideC at least the span of one C matrix when batch > 1).
 *
 * Scalars and semantics
 *   alpha and beta are fp32 for every element type; the epilogue computes
 *   alpha*acc + beta*C_old in fp32 and rounds to the output type
 *   round-to-nearest-even.  beta == 0: C is written without being read (NaN
 *   in C does not propagate).  alpha == 0 or K == 0: C <- beta*C and A, B are
 *   not read.  M == 0, N == 0 or batch == 0: nothing is done.
 *
 * Ownership and synchronisation
 *   The caller owns every buffer; A, B and C are device pointers valid on
 *   `stream`.  The library allocates nothing, retains no pointer and keeps no
 *   state between calls.  A call only enqueues work on `stream` (a hipStream_t;
 *   0 means the null stream) and returns; results are visible after the
 *   stream is synchronised.  C must not overlap A or B.
 *
 * Errors
 *   Every argument is validated before any HIP call; an invalid call launches
 *   nothing, changes no memory and returns a negative status.  Nothing is
 *   printed and no exception crosses this interface.
 *     GEMM_ERR_INVALID_ARG  negative dimension, batch or stride; leading
 *                           dimension too small; null pointer for a matrix
 *                           that must be read or written; a pointer that is
 *                           not a multiple of its element size; order or dtype out
 *                           of range; C slices overlapping each other; C
 *                           overlapping A or B (checked on the address ranges
 *                           the operands span).
 *     GEMM_ERR_UNSUPPORTED  a combination this build does not provide.
 *     GEMM_ERR_HIP          the kernel launch reported a HIP error.
 */
#ifndef LIBGEMM_H
#define LIBGEMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gemm_order_t {
    GEMM_ROW_MAJOR = 0,
    GEMM_COL_MAJOR = 1
} gemm_order_t;

typedef enum gemm_dtype_t {
    GEMM_DTYPE_SAME = 0, /* output in the input type (bf16 or fp16) */
    GEMM_DTYPE_F32 = 1   /* output in fp32 */
} gemm_dtype_t;

typedef enum gemm_input_t {
    GEMM_INPUT_F32 = 0,
    GEMM_INPUT_BF16 = 1,
    GEMM_INPUT_F16 = 2
} gemm_input_t;

/* OCP 8-bit floating-point formats of gemm_f8's operands. */
typedef enum gemm_f8_format_t {
    GEMM_F8_E4M3 = 0, /* 1 sign, 4 exponent (bias 7), 3 fraction bits; no
                         infinities, S.1111.111 is NaN, largest finite 448 */
    GEMM_F8_E5M2 = 1  /* 1 sign, 5 exponent (bias 15), 2 fraction bits;
                         IEEE-style infinities and NaNs, largest finite 57344 */
} gemm_f8_format_t;

/* Element formats of gemm_mx's operands (the OCP microscaling element
 * types).  None of the 6- and 4-bit ones has infinities or NaNs. */
typedef enum gemm_mx_format_t {
    GEMM_MX_E4M3 = 0, /* MXFP8: as GEMM_F8_E4M3 */
    GEMM_MX_E5M2 = 1, /* MXFP8: as GEMM_F8_E5M2 */
    GEMM_MX_E2M3 = 2, /* MXFP6: 1 sign, 2 exponent (bias 1), 3 fraction bits; largest 7.5 */
    GEMM_MX_E3M2 = 3, /* MXFP6: 1 sign, 3 exponent (bias 3), 2 fraction bits; largest 28 */
    GEMM_MX_E2M1 = 4  /* MXFP4: 1 sign, 2 exponent (bias 1), 1 fraction bit;
                         0, 0.5, 1, 1.5, 2, 3, 4, 6 */
} gemm_mx_format_t;

/* Element type of the C of gemm_f8 and gemm_mx. */
typedef enum gemm_output_t {
    GEMM_OUTPUT_F32 = 0,
    GEMM_OUTPUT_BF16 = 1,
    GEMM_OUTPUT_F16 = 2
} gemm_output_t;

typedef enum gemm_activation_t {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1, /* max(x, 0) */
    GEMM_ACT_GELU = 2  /* x * Phi(x), Phi the standard normal distribution function */
} gemm_activation_t;

typedef enum gemm_status_t {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = -1,
    GEMM_ERR_UNSUPPORTED = -2,
    GEMM_ERR_HIP = -3,
    GEMM_ERR_SCRATCH = -4 /* gemm_bf16_noalloc only: the call would need more
                             than GEMM_NOALLOC_SCRATCH_BYTES of scratch */
} gemm_status_t;

/* fp32 SGEMM.  A, B, C point to float; see the header comment for layout,
 * batch, semantics and errors. */
gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K, float alpha,
                       const float *A, int64_t lda, gemm_order_t orderA,
                       const float *B, int64_t ldb, gemm_order_t orderB,
                       float beta, float *C, int64_t ldc, gemm_order_t orderC,
                       int64_t batch, int64_t strideA, int64_t strideB,
                       int64_t strideC, hipStream_t stream);

/* bf16 HGEMM with fp32 accumulation.  A and B hold bf16 bit patterns
 * (uint16_t); C holds bf16 patterns (c_dtype = GEMM_DTYPE_SAME) or float
 * (GEMM_DTYPE_F32).  The hgemm sm120 article (wingedge777.com) computes this
 * product with fp16/bf16 operands and fp32 accumulation on matrix units. */
gemm_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha,
                        const uint16_t *A, int64_t lda, gemm_order_t orderA,
                        const uint16_t *B, int64_t ldb, gemm_order_t orderB,
                        float beta, void *C, int64_t ldc, gemm_order_t orderC,
                        gemm_dtype_t c_dtype, int64_t batch, int64_t strideA,
                        int64_t strideB, int64_t strideC, hipStream_t stream);

/* IEEE fp16 HGEMM with fp32 accumulation; as gemm_bf16. */
gemm_status_t gemm_f16(int64_t M, int64_t N, int64_t K, float alpha,
                       const uint16_t *A, int64_t lda, gemm_order_t orderA,
                       const uint16_t *B, int64_t ldb, gemm_order_t orderB,
                       float beta, void *C, int64_t ldc, gemm_order_t orderC,
                       gemm_dtype_t c_dtype, int64_t batch, int64_t strideA,
                       int64_t strideB, int64_t strideC, hipStream_t stream);

/* Fused epilogue: C <- act(alpha * op(A) * op(B) + beta * C + bias), with
 * the bias one value per column j of C (bias[j], added to every row) and
 * act applied to each element after the bias, in fp32, before the rounding
 * to the output type.  The pages fold "GEMM + bias + activation" into one
 * kernel ("第4章：经典算子实现 —— GEMM", aiinfra.vidrealm.tech, section 7.2)
 * and apply element-wise operations such as ReLU to the accumulators before
 * the store ("GPU GEMM 优化完全拆解（三）", pinghaoyang.com.cn, section on
 * mainloop and epilogue).
 *   bias        device vector of N elements of the input type (float for
 *               gemm_f32_bias_act, bf16/fp16 bit patterns otherwise), or
 *               NULL for no bias.  It must not overlap C.
 *   strideBias  elements between the bias vectors of consecutive batch
 *               entries (>= 0; 0 shares one vector).
 *   act         GEMM_ACT_NONE, GEMM_ACT_RELU or GEMM_ACT_GELU.  GELU is
 *               x * Phi(x); Phi is evaluated in fp32 through the rational
 *               approximation 7.1.26 of Abramowitz and Stegun for erfc
 *               (absolute error at most 1.5e-7 in Phi).
 * All other arguments, the layouts, batch rules, ownership and errors are
 * those of gemm_f32 / gemm_bf16 / gemm_f16; an act out of range, a negative
 * strideBias or a bias overlapping C is GEMM_ERR_INVALID_ARG.  With
 * alpha == 0 or K == 0 the result is act(beta * C + bias). */
gemm_status_t gemm_f32_bias_act(int64_t M, int64_t N, int64_t K, float alpha,
                                const float *A, int64_t lda, gemm_order_t orderA,
                                const float *B, int64_t ldb, gemm_order_t orderB,
                                float beta, float *C, int64_t ldc,
                                gemm_order_t orderC, int64_t batch,
                                int64_t strideA, int64_t strideB,
                                int64_t strideC, const float *bias,
                                int64_t strideBias, gemm_activation_t act,
                                hipStream_t stream);

gemm_status_t gemm_bf16_bias_act(int64_t M, int64_t N, int64_t K, float alpha,
                                 const uint16_t *A, int64_t lda,
                                 gemm_order_t orderA, const uint16_t *B,
                                 int64_t ldb, gemm_order_t orderB, float beta,
                                 void *C, int64_t ldc, gemm_order_t orderC,
                                 gemm_dtype_t c_dtype, int64_t batch,
                                 int64_t strideA, int64_t strideB,
                                 int64_t strideC, const uint16_t *bias,
                                 int64_t strideBias, gemm_activation_t act,
                                 hipStream_t stream);

gemm_status_t gemm_f16_bias_act(int64_t M, int64_t N, int64_t K, float alpha,
                                const uint16_t *A, int64_t lda,
                                gemm_order_t orderA, const uint16_t *B,
                                int64_t ldb, gemm_order_t orderB, float beta,
                                void *C, int64_t ldc, gemm_order_t orderC,
                                gemm_dtype_t c_dtype, int64_t batch,
                                int64_t strideA, int64_t strideB,
                                int64_t strideC, const uint16_t *bias,
                                int64_t strideBias, gemm_activation_t act,
                                hipStream_t stream);

/* Quantised output: the fused epilogue above, then scaled and stored as
 * 8-bit floats.  The pages do quantisation scaling in the epilogue's
 * write-back ("GPU GEMM 优化完全拆解（三）", pinghaoyang.com.cn, section on
 * mainloop and epilogue) and list quantised (INT8/INT4/FP8) GEMMs among the
 * uses of a customisable epilogue ("第4章：经典算子实现 —— GEMM",
 * aiinfra.vidrealm.tech, section 7.2).  For each element of C:
 *   C <- Q(c_scale * act(alpha * op(A) * op(B) + bias))
 * computed in fp32, where Q rounds to the nearest value of c_format (OCP
 * E4M3 or E5M2, ties to even) and saturates: magnitudes beyond the largest
 * finite value (448, resp. 57344), infinities included, store that value
 * with their sign; a NaN stores a NaN pattern.  C holds one byte per element
 * (uint8_t, its leading dimension and strides in elements); C is never read
 * (there is no beta).  bias, strideBias and act are as for the _bias_act
 * calls (bias of the input type, or NULL).  The product runs on the 16-bit
 * direct-load kernel: operands it cannot read whole 16-byte chunks of (base,
 * leading dimension or stride not 16-byte aligned, contiguous extent not a
 * multiple of 8, a slice of 1 GiB or more) give GEMM_ERR_UNSUPPORTED before
 * anything is launched.  With alpha == 0 or K == 0 the result is
 * Q(c_scale * act(bias)).  A c_format out of range is GEMM_ERR_INVALID_ARG;
 * all other arguments, layouts, batch rules, ownership and errors are those of
 * gemm_bf16 / gemm_f16. */
gemm_status_t gemm_bf16_quant(int64_t M, int64_t N, int64_t K, float alpha,
                              const uint16_t *A, int64_t lda, gemm_order_t orderA,
                              const uint16_t *B, int64_t ldb, gemm_order_t orderB,
                              uint8_t *C, int64_t ldc, gemm_order_t orderC,
                              gemm_f8_format_t c_format, float c_scale, int64_t batch,
                              int64_t strideA, int64_t strideB, int64_t strideC,
                              const uint16_t *bias, int64_t strideBias,
                              gemm_activation_t act, hipStream_t stream);

gemm_status_t gemm_f16_quant(int64_t M, int64_t N, int64_t K, float alpha,
                             const uint16_t *A, int64_t lda, gemm_order_t orderA,
                             const uint16_t *B, int64_t ldb, gemm_order_t orderB,
                             uint8_t *C, int64_t ldc, gemm_order_t orderC,
                             gemm_f8_format_t c_format, float c_scale, int64_t batch,
                             int64_t strideA, int64_t strideB, int64_t strideC,
                             const uint16_t *bias, int64_t strideBias,
                             gemm_activation_t act, hipStream_t stream);

/* 8-bit float GEMM: C <- alpha * op(A) * op(B) + beta * C with A and B
 * holding E4M3 or E5M2 bit patterns (formatA, formatB; the two may differ),
 * and C of type typeC (float, or bf16 / fp16 bit patterns).  The pages list
 * E4M3 and E5M2 as the 8-bit floating formats below fp16/bf16 for matrix
 * units ("CUDA GEMM 矩阵乘法优化指南", blog.zhenwei.site, section 13.2).
 * Accuracy: the products are formed exactly, but gfx950's 8-bit matrix
 * instruction adds them at reduced precision: within each group of 8
 * consecutive k, a product smaller than 2^-13 of the group's largest is
 * cut off below that point (groups combine at fp32 precision).  The result
 * therefore lies within about 1e-3 * sum_k |alpha A_ik B_kj| (plus
 * |beta C_ij| rounding) of the exact value, rather than within fp32
 * rounding of it; products of small integers are exact.  The epilogue is
 * that of gemm_bf16 (alpha*acc + beta*C_old in fp32, rounded to
 * nearest-even into typeC).  NaN and, for E5M2, infinite inputs propagate
 * as in IEEE arithmetic.  Any per-tensor
 * scale factors of the 8-bit data are folded into alpha by the caller.
 * Layout, batch (strides in elements, i.e. bytes for A and B), ownership
 * and errors are those of gemm_bf16.  A format or typeC out of range is
 * GEMM_ERR_INVALID_ARG.  The fast path needs row-major A, column-major B
 * (both contiguous along K), 16-byte aligned A and B, lda, ldb, strideA,
 * strideB and K multiples of 16; every other call is exact on a slower
 * general kernel. */
gemm_status_t gemm_f8(int64_t M, int64_t N, int64_t K, float alpha,
                      const uint8_t *A, int64_t lda, gemm_order_t orderA,
                      gemm_f8_format_t formatA, const uint8_t *B, int64_t ldb,
                      gemm_order_t orderB, gemm_f8_format_t formatB,
                      float beta, void *C, int64_t ldc, gemm_order_t orderC,
                      gemm_output_t typeC, int64_t batch, int64_t strideA,
                      int64_t strideB, int64_t strideC, hipStream_t stream);

/* Block-scaled GEMM: C <- alpha * A * B + beta * C, where every 32
 * consecutive elements along K of a row of A (a column of B) share one
 * E8M0 scale, a power of two 2^(e - 127) (e = 255 is NaN): the block-scale
 * quantisation of MXFP8/MXFP6/MXFP4 ("CUDA GEMM 矩阵乘法优化指南",
 * blog.zhenwei.site, section 13.2).  The value of A(i, k) is
 * 2^(scaleA[i*ldsa + k/32] - 127) times its element; products are exact and
 * accumulate in fp32 (with the same reduced-precision additions as gemm_f8:
 * the matrix instruction is the same), then alpha * acc + beta * C in fp32,
 * rounded to typeC to nearest-even.
 *   A        M x K, contiguous along K: row i is elements i*lda .. i*lda+K-1
 *            of a packed element stream (8-bit formats one byte each; 6-bit
 *            ones four elements in three bytes, 4-bit ones two per byte, the
 *            stream little-endian: element n occupies bits w*n .. w*n+w-1,
 *            bit b being bit b%8 of byte b/8).  Device memory, 16-byte
 *            aligned; lda a multiple of 64 elements, at least K.
 *   B        K x N, contiguous along K: column j is elements j*ldb ..
 *            j*ldb+K-1 of its stream; the same rules.
 *   scaleA   E8M0 bytes, row i of A's at scaleA + i*ldsa; 4-byte aligned,
 *            ldsa a multiple of 4 and at least 4*ceil(K/128).  The kernel
 *            reads a row's scales sixteen blocks at a time, so it may read
 *            bytes past the row's ceil(K/32) (into the row's padding or the
 *            next row) but never past the slice's M*ldsa bytes; such bytes
 *            are never used.  scaleB likewise for B's columns (N*ldsb).
 *   formatA, formatB  element formats of one width: both 8-bit (E4M3/E5M2,
 *            in any combination), both 6-bit (E2M3/E3M2) or both E2M1;
 *            a mixed-width pair is GEMM_ERR_UNSUPPORTED.
 *   K        a multiple of 64 (two scale blocks).
 *   C        typeC (fp32, or bf16/fp16 bit patterns), orderC, ldc as for
 *            gemm_f8; a column-major C is computed as C^T = B^T A^T.
 *   batch    strideA and strideB in elements (multiples of 64),
 *            strideScaleA and strideScaleB in bytes (multiples of 4),
 *            strideC in elements; 0 shares an operand or its scales.
 * alpha == 0 or K == 0 gives beta * C without reading A, B or the scales.
 * Any other layout rule broken, a format or typeC out of range, or C
 * overlapping an operand or a scale array is GEMM_ERR_INVALID_ARG, before
 * any HIP call; a slice of A, B or a scale array of 2^30 bytes or more is
 * GEMM_ERR_UNSUPPORTED.  Ownership and synchronisation as for gemm_bf16. */
gemm_status_t gemm_mx(int64_t M, int64_t N, int64_t K, float alpha,
                      const void *A, int64_t lda, gemm_mx_format_t formatA,
                      const uint8_t *scaleA, int64_t ldsa,
                      const void *B, int64_t ldb, gemm_mx_format_t formatB,
                      const uint8_t *scaleB, int64_t ldsb,
                      float beta, void *C, int64_t ldc, gemm_order_t orderC,
                      gemm_output_t typeC, int64_t batch, int64_t strideA,
                      int64_t strideB, int64_t strideScaleA,
                      int64_t strideScaleB, int64_t strideC, hipStream_t stream);

/* Workspace entry points.  gemm_f32_ws / gemm_bf16_ws / gemm_f16_ws take the
 * arguments of gemm_f32 / gemm_bf16 / gemm_f16 plus a device workspace, and
 * compute the same product.  For fp32 both kernels (the general one and the
 * direct-load one; 128 x 128 tiles, four workgroups per compute unit) have
 * the same schedule, with the same workspace.
 * With at least gemm_workspace_size() bytes, a problem on either 16-bit
 * kernel (the general one for operands that are not 16-byte aligned, the
 * direct-load one for aligned operands with 64 tiles or more) whose
 * 256 x 256 tiles leave the last wave of workgroups partly idle runs on the
 * stream-K schedule ("CUDA GEMM 矩阵乘法优化指南", blog.zhenwei.site, section
 * 12.5, persistent kernels and Stream-K): the tiles that fill whole waves of
 * one workgroup per compute unit are computed whole, and the k steps of the
 * remaining tiles are split evenly over a number of workgroups that balances
 * the tail against the exchange; the pieces of a tile that was cut are
 * written to the workspace and added, in a fixed order, by a second kernel on
 * the same stream, which also applies the epilogue.  It is chosen when the
 * steps saved in the last wave outweigh that exchange (about four k steps of
 * one tile on the general 16-bit kernel, eight on the fp32 kernels; on the
 * 16-bit direct-load one about 0.14 k steps per partial tile plus two).  The
 * testing switch
 * GEMM_TEST_FORCE_STREAMK chooses it wherever it can run.
 * Operands that are not 16-byte aligned (base, leading dimension, stride or
 * contiguous extent), in a problem of at least 64 tiles of 256 x 256
 * (bf16/fp16) or 160 tiles of 128 x 128 (fp32), are first copied into the
 * workspace in the same order, zero-padded to whole 16-byte chunks along
 * their contiguous dimension (K padded to a multiple of 8, resp. 4, with zero
 * rows or columns), and the direct-load kernel (or its stream-K schedule, by
 * the same cost model) runs on the copies, with the caller's M,
 * N and C.  The zero padding adds nothing to any result.  This is chosen
 * whenever the copies and any partial tiles fit the workspace; otherwise the
 * general kernel runs on the caller's operands as described above.  When the
 * last column of tiles of the (row-major-C) problem holds at most 32 columns
 * of C, those columns run after the rest as a problem of their own on the
 * copies, on the split-K kernel, instead of taking a wave of tiles.
 * A 16-bit problem of at most 16 rows of C (of K-contiguous A) with an
 * N-contiguous B, N >= 256 and K >= 1024 is split along K across
 * workgroups ("GPU GEMM 优化完全拆解（三）", pinghaoyang.com.cn, the
 * rasterization and split-K section): each workgroup multiplies 128 columns
 * of B over one slice of K (about 512 workgroups in all) and writes fp32
 * partial sums, split * batch * M * ceil(N / 128) * 128 * 4 bytes of the
 * workspace; a second kernel on the same stream adds each element's slices
 * in one fixed order and applies the epilogue.
 * Results are deterministic run to run; they may differ in rounding from
 * gemm_bf16 (the partial sums are grouped differently), within the same
 * accuracy.  Every other call ignores the workspace and behaves exactly like
 * gemm_bf16.
 *   workspace        device memory, 256-byte aligned, not overlapping A, B or
 *                    C; owned by the caller and clobbered by the call (it
 *                    holds operand copies and partial tiles while the
 *                    kernels run on `stream`; calls that share a workspace
 *                    must be ordered on one stream).  NULL only with
 *                    workspace_bytes = 0.
 *   workspace_bytes  its size; smaller than gemm_workspace_size() (0
 *                    included) means the workspace is not used.
 * A misaligned, overlapping or NULL (with bytes > 0) workspace is
 * GEMM_ERR_INVALID_ARG; everything else is as for gemm_bf16. */
size_t gemm_workspace_size(void);

gemm_status_t gemm_f32_ws(int64_t M, int64_t N, int64_t K, float alpha,
                          const float *A, int64_t lda, gemm_order_t orderA,
                          const float *B, int64_t ldb, gemm_order_t orderB,
                          float beta, float *C, int64_t ldc, gemm_order_t orderC,
                          int64_t batch, int64_t strideA, int64_t strideB,
                          int64_t strideC, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

gemm_status_t gemm_bf16_ws(int64_t M, int64_t N, int64_t K, float alpha,
                           const uint16_t *A, int64_t lda, gemm_order_t orderA,
                           const uint16_t *B, int64_t ldb, gemm_order_t orderB,
                           float beta, void *C, int64_t ldc,
                           gemm_order_t orderC, gemm_dtype_t c_dtype,
                           int64_t batch, int64_t strideA, int64_t strideB,
                           int64_t strideC, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

gemm_status_t gemm_f16_ws(int64_t M, int64_t N, int64_t K, float alpha,
                          const uint16_t *A, int64_t lda, gemm_order_t orderA,
                          const uint16_t *B, int64_t ldb, gemm_order_t orderB,
                          float beta, void *C, int64_t ldc, gemm_order_t orderC,
                          gemm_dtype_t c_dtype, int64_t batch, int64_t strideA,
                          int64_t strideB, int64_t strideC, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* 8-bit and block-scaled workspace entry points.  gemm_f8_ws takes the
 * arguments of gemm_f8, gemm_mx_ws those of gemm_mx, each plus a workspace
 * under the rules of gemm_bf16_ws, and computes the same product.  With at
 * least gemm_workspace_size() bytes, a call on the direct-load kernel
 * (gemm_f8's fast path; every gemm_mx call that multiplies) whose 256 x 256
 * tiles leave the last wave of one workgroup per compute unit partly idle
 * runs on the stream-K schedule described for gemm_bf16_ws ("CUDA GEMM 矩阵
 * 乘法优化指南", blog.zhenwei.site, section 12.5), a k step being 128 k,
 * when the cost model of the 16-bit direct-load kernel (about 0.14 k steps
 * per partial tile plus two) says it pays; GEMM_TEST_FORCE_STREAMK chooses
 * it wherever tiles are left over.  The pieces of a cut tile start and end
 * at multiples of 128 k and are added in a fixed order, so results are
 * deterministic and within the accuracy stated for gemm_f8 and gemm_mx
 * (products of small integers stay exact).  Every other call ignores the
 * workspace.  A misaligned or NULL (with bytes > 0) workspace, or one that
 * overlaps A, B, C or (gemm_mx_ws) a scale array, is GEMM_ERR_INVALID_ARG;
 * everything else is as for gemm_f8 / gemm_mx. */
gemm_status_t gemm_f8_ws(int64_t M, int64_t N, int64_t K, float alpha,
                         const uint8_t *A, int64_t lda, gemm_order_t orderA,
                         gemm_f8_format_t formatA, const uint8_t *B, int64_t ldb,
                         gemm_order_t orderB, gemm_f8_format_t formatB,
                         float beta, void *C, int64_t ldc, gemm_order_t orderC,
                         gemm_output_t typeC, int64_t batch, int64_t strideA,
                         int64_t strideB, int64_t strideC, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

gemm_status_t gemm_mx_ws(int64_t M, int64_t N, int64_t K, float alpha,
                         const void *A, int64_t lda, gemm_mx_format_t formatA,
                         const uint8_t *scaleA, int64_t ldsa,
                         const void *B, int64_t ldb, gemm_mx_format_t formatB,
                         const uint8_t *scaleB, int64_t ldsb,
                         float beta, void *C, int64_t ldc, gemm_order_t orderC,
                         gemm_output_t typeC, int64_t batch, int64_t strideA,
                         int64_t strideB, int64_t strideScaleA,
                         int64_t strideScaleB, int64_t strideC, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Allocation-free variant of gemm_bf16_ws, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 * It takes the arguments of gemm_bf16 and computes exactly what gemm_bf16_ws
 * computes with a workspace of gemm_workspace_size() bytes: the same kernels,
 * the same schedule, bit-identical results.  In place of a caller's
 * workspace it uses a scratch array of GEMM_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that the library holds on every GPU it runs on, from the time its code is
 * loaded there until the process ends; it calls no allocating routine.
 *   Limit: a call whose schedule would use more scratch than that returns
 *          GEMM_ERR_SCRATCH before any HIP call and launches nothing.  Only
 *          the stream-K schedule of the general kernel can need more (up to
 *          128 MiB of partial tiles: unaligned operands, fewer than 64 tiles
 *          of 256 x 256, a long K); gemm_bf16 computes those calls without
 *          scratch.  Copies of unaligned operands and the direct-load
 *          kernel's partial tiles stay within the limit at the workload
 *          sizes tested (4095 x 4097 x 1001: 17 MB; 4096 x 4352 x 4096: 59 MB).
 *   Set-up: the first call on a device looks up the scratch's address there
 *          (hipGetSymbolAddress, with that device current for the lookup;
 *          the caller's current device is restored) and keeps it.  Make one
 *          call on each device before capturing calls into a graph.  The
 *          device is the one `stream` belongs to.
 *   Sharing: every call on one GPU uses that GPU's scratch, which keeps the
 *          last call's contents.  Nothing in it needs to start at zero: each
 *          byte a kernel reads was written earlier in the same call.  Calls
 *          that may run at the same time on one GPU (on different streams,
 *          or from several host threads) race on the scratch and give wrong
 *          results; order them, for example on one stream.
 * Errors are those of gemm_bf16, plus GEMM_ERR_SCRATCH. */
#define GEMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

gemm_status_t gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K, float alpha,
                                const uint16_t *A, int64_t lda, gemm_order_t orderA,
                                const uint16_t *B, int64_t ldb, gemm_order_t orderB,
                                float beta, void *C, int64_t ldc, gemm_order_t orderC,
                                gemm_dtype_t c_dtype, int64_t batch, int64_t strideA,
                                int64_t strideB, int64_t strideC, hipStream_t stream);

/* fp32 SGEMM on the vector ALUs: the register-tiled design of section 7 of
 * "CUDA GEMM 矩阵乘法优化指南" (blog.zhenwei.site) -- LDS-staged 128 x 256 x 16
 * tiles, an 8 x 16 tile of fused multiply-adds per thread -- instead of the
 * matrix-core kernels gemm_f32 uses.  Arguments, semantics and errors are
 * those of gemm_f32. */
gemm_status_t gemm_f32_valu(int64_t M, int64_t N, int64_t K, float alpha,
                            const float *A, int64_t lda, gemm_order_t orderA,
                            const float *B, int64_t ldb, gemm_order_t orderB,
                            float beta, float *C, int64_t ldc, gemm_order_t orderC,
                            int64_t batch, int64_t strideA, int64_t strideB,
                            int64_t strideC, hipStream_t stream);

/* fp32 GEMM on the bf16 matrix instructions, by splitting each operand into
 * two bf16 pieces ("GPU GEMM 优化完全拆解（三）", pinghaoyang.com.cn, the
 * section on numerical precision and why fp32 cuBLAS does not use Tensor
 * Cores, describes the split into a high and a low part and three products
 * for TF32; bf16 plays that part here).  Each element v of A and B becomes
 * hi = v rounded to bf16 (nearest, ties to even; truncated if that would
 * overflow) and lo = (v - hi) rounded to bf16, and a*b is summed as
 * hi*hi + hi*lo + lo*hi in fp32.  The terms left out are at most 2^-15 |a*b|,
 * so each element of C is within (2^-15 + the fp32 accumulation error of 3K
 * terms) * sum_k |A_ik| |B_kj| of the exact result; alpha, beta, C and the
 * orders are applied exactly as in gemm_f32 (beta = 0: C is not read).
 * Non-finite elements of A or B give non-finite results in the elements
 * they reach (NaN where an infinity meets a zero piece); subnormal low
 * pieces may be flushed, an error below 2^-126 per product.
 *   workspace        device memory of at least
 *                    gemm_f32_bf16x3_workspace_size(M, N, K, batch) bytes,
 *                    256-byte aligned, not overlapping A, B or C; it receives
 *                    the bf16 copies (A: M x 3Kp per batch entry, B: N x 3Kp,
 *                    Kp = K rounded up to a multiple of 8; one copy of an
 *                    operand whose batch stride is 0), written on `stream`
 *                    before the product runs.  Calls that share it must be
 *                    ordered (for example, on one stream).
 *   workspace_bytes  its size.
 * A workspace that is NULL, misaligned, too small or overlapping is
 * GEMM_ERR_INVALID_ARG.  When nothing is multiplied (M, N or batch = 0,
 * K = 0 or alpha = 0) the call is gemm_f32's and the workspace is not used.
 * Everything else is as for gemm_f32. */
size_t gemm_f32_bf16x3_workspace_size(int64_t M, int64_t N, int64_t K, int64_t batch);

gemm_status_t gemm_f32_bf16x3(int64_t M, int64_t N, int64_t K, float alpha,
                              const float *A, int64_t lda, gemm_order_t orderA,
                              const float *B, int64_t ldb, gemm_order_t orderB,
                              float beta, float *C, int64_t ldc, gemm_order_t orderC,
                              int64_t batch, int64_t strideA, int64_t strideB,
                              int64_t strideC, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Testing aid: process-wide overrides of the kernel choice, so that tests
 * can run every kernel on problems the normal choice sends elsewhere.  Not
 * for production use.  The set holds until the next call; 0 (the initial
 * state) clears every override.  Returns the previous set.  Every GEMM entry
 * point and kernel-name query reads the set at each call.
 *   GEMM_TEST_FORCE_GENERAL  every call on the general kernel of its type
 *                            (no direct-load, split-K, skinny or stream-K
 *                            kernel, no operand copies)
 *   GEMM_TEST_NO_SPLITK      few-tile and skinny problems on the main kernels
 *   GEMM_TEST_FORCE_STREAMK  workspace calls take the stream-K schedule
 *                            wherever it can run, whatever its cost model says
 *   GEMM_TEST_F32_VALU       fp32 calls on the vector-ALU kernel */
typedef enum gemm_test_switch_t {
    GEMM_TEST_FORCE_GENERAL = 1,
    GEMM_TEST_NO_SPLITK = 2,
    GEMM_TEST_FORCE_STREAMK = 4,
    GEMM_TEST_F32_VALU = 8
} gemm_test_switch_t;

int gemm_test_switches(int flags);

/* Static, human-readable name of a status code (never NULL). */
const char *gemm_status_string(gemm_status_t status);

/* Version of this interface; bumped on any incompatible change. */
int gemm_abi_version(void);

/* The kernel that gemm_f32 (in = GEMM_INPUT_F32; c_dtype is then ignored),
 * gemm_bf16 or gemm_f16 would launch for the same arguments, as a static
 * string: "sgemm_mfma_dma", "sgemm_mfma", "sgemm_splitk", "sgemm_valu",
 * "hgemm_mfma_dma", "hgemm_mfma", "hgemm_splitk", "gemm_skinny" or "scale";
 * "" when the call would return without launching anything (M, N or batch
 * is 0); NULL when the arguments are invalid (the GEMM call would return an
 * error status).  The choice depends on the shape, the orders, the
 * alignment of the pointers, leading dimensions and strides, and the testing
 * switches (gemm_test_switches), exactly as in the GEMM calls.  Pointers are compared
 * and tested for alignment but never dereferenced; no HIP call is made, so
 * this works without a GPU. */
const char *gemm_kernel_name(gemm_input_t in, int64_t M, int64_t N, int64_t K,
                             float alpha, const void *A, int64_t lda,
                             gemm_order_t orderA, const void *B, int64_t ldb,
                             gemm_order_t orderB, float beta, const void *C,
                             int64_t ldc, gemm_order_t orderC,
                             gemm_dtype_t c_dtype, int64_t batch,
                             int64_t strideA, int64_t strideB, int64_t strideC);

/* The kernel that gemm_f8 would launch for the same arguments:
 * "f8gemm_mfma_dma", "f8gemm_mfma" or "scale"; "" and NULL as for
 * gemm_kernel_name (of the testing switches, only GEMM_TEST_FORCE_GENERAL
 * applies here). */
const char *gemm_f8_kernel_name(int64_t M, int64_t N, int64_t K, float alpha,
                                const uint8_t *A, int64_t lda,
                                gemm_order_t orderA, gemm_f8_format_t formatA,
                                const uint8_t *B, int64_t ldb,
                                gemm_order_t orderB, gemm_f8_format_t formatB,
                                float beta, const void *C, int64_t ldc,
                                gemm_order_t orderC, gemm_output_t typeC,
                                int64_t batch, int64_t strideA,
                                int64_t strideB, int64_t strideC);

/* The kernel gemm_mx would launch: "mxgemm_mfma_dma", "scale" when only
 * beta * C is computed, "" when nothing is done, NULL for an invalid call
 * (any status other than GEMM_OK).  Host only; no pointer is dereferenced. */
const char *gemm_mx_kernel_name(int64_t M, int64_t N, int64_t K, float alpha,
                                const void *A, int64_t lda,
                                gemm_mx_format_t formatA,
                                const uint8_t *scaleA, int64_t ldsa,
                                const void *B, int64_t ldb,
                                gemm_mx_format_t formatB,
                                const uint8_t *scaleB, int64_t ldsb,
                                float beta, const void *C, int64_t ldc,
                                gemm_order_t orderC, gemm_output_t typeC,
                                int64_t batch, int64_t strideA, int64_t strideB,
                                int64_t strideScaleA, int64_t strideScaleB,
                                int64_t strideC);

/* The kernel gemm_f8_ws would launch: the names of gemm_f8_kernel_name, or
 * "f8gemm_mfma_dma_streamk" for the stream-K schedule; "" and NULL as for
 * gemm_kernel_name, whose testing switches apply, GEMM_TEST_FORCE_STREAMK
 * included.  The workspace is only checked, never dereferenced. */
const char *gemm_f8_kernel_name_ws(int64_t M, int64_t N, int64_t K, float alpha,
                                   const uint8_t *A, int64_t lda,
                                   gemm_order_t orderA, gemm_f8_format_t formatA,
                                   const uint8_t *B, int64_t ldb,
                                   gemm_order_t orderB, gemm_f8_format_t formatB,
                                   float beta, const void *C, int64_t ldc,
                                   gemm_order_t orderC, gemm_output_t typeC,
                                   int64_t batch, int64_t strideA,
                                   int64_t strideB, int64_t strideC,
                                   const void *workspace, size_t workspace_bytes);

/* The kernel gemm_mx_ws would launch: the names of gemm_mx_kernel_name, or
 * "mxgemm_mfma_dma_streamk" for the stream-K schedule (GEMM_TEST_FORCE_STREAMK
 * and GEMM_TEST_FORCE_GENERAL, which keeps one workgroup per tile, apply).
 * Host only; no pointer is dereferenced. */
const char *gemm_mx_kernel_name_ws(int64_t M, int64_t N, int64_t K, float alpha,
                                   const void *A, int64_t lda,
                                   gemm_mx_format_t formatA,
                                   const uint8_t *scaleA, int64_t ldsa,
                                   const void *B, int64_t ldb,
                                   gemm_mx_format_t formatB,
                                   const uint8_t *scaleB, int64_t ldsb,
                                   float beta, const void *C, int64_t ldc,
                                   gemm_order_t orderC, gemm_output_t typeC,
                                   int64_t batch, int64_t strideA, int64_t strideB,
                                   int64_t strideScaleA, int64_t strideScaleB,
                                   int64_t strideC, const void *workspace,
                                   size_t workspace_bytes);

/* The kernel gemm_f32_ws (in = GEMM_INPUT_F32; c_dtype is then ignored),
 * gemm_bf16_ws (GEMM_INPUT_BF16) or gemm_f16_ws (GEMM_INPUT_F16) would
 * launch: the names of gemm_kernel_name, or "hgemm_mfma_streamk",
 * "hgemm_mfma_dma_streamk", "sgemm_mfma_streamk" or "sgemm_mfma_dma_streamk"
 * for the stream-K schedules, "hgemm_mfma_dma_packed",
 * "hgemm_mfma_dma_streamk_packed", "sgemm_mfma_dma_packed" or
 * "sgemm_mfma_dma_streamk_packed" when the operands are first copied into
 * the workspace, "gemm_skinny_splitk" for the skinny split-K; "" and NULL as for gemm_kernel_name, whose testing switches
 * apply, GEMM_TEST_FORCE_STREAMK included.  The workspace is only
 * checked, never dereferenced. */
const char *gemm_kernel_name_ws(gemm_input_t in, int64_t M, int64_t N, int64_t K,
                                float alpha, const void *A, int64_t lda,
                                gemm_order_t orderA, const void *B, int64_t ldb,
                                gemm_order_t orderB, float beta, const void *C,
                                int64_t ldc, gemm_order_t orderC,
                                gemm_dtype_t c_dtype, int64_t batch,
                                int64_t strideA, int64_t strideB, int64_t strideC,
                                const void *workspace, size_t workspace_bytes);

/* The kernel gemm_bf16_quant (in = GEMM_INPUT_BF16) or gemm_f16_quant
 * (GEMM_INPUT_F16) would launch: "hgemm_mfma_dma", "scale" when nothing is
 * multiplied, "" for an empty problem, NULL for invalid arguments or a
 * problem the call would reject as GEMM_ERR_UNSUPPORTED.  No HIP call. */
const char *gemm_kernel_name_quant(gemm_input_t in, int64_t M, int64_t N, int64_t K,
                                   float alpha, const void *A, int64_t lda,
                                   gemm_order_t orderA, const void *B, int64_t ldb,
                                   gemm_order_t orderB, const void *C, int64_t ldc,
                                   gemm_order_t orderC, gemm_f8_format_t c_format,
                                   int64_t batch, int64_t strideA, int64_t strideB,
                                   int64_t strideC);

/* The bf16 kernel gemm_f32_bf16x3 would run on the split copies (one of the
 * names of gemm_kernel_name for 16-bit inputs), "scale" or "" when nothing is
 * multiplied, NULL when the arguments or the workspace are invalid.  The
 * workspace is only checked, never dereferenced; no HIP call is made. */
const char *gemm_kernel_name_bf16x3(int64_t M, int64_t N, int64_t K, float alpha,
                                    const void *A, int64_t lda, gemm_order_t orderA,
                                    const void *B, int64_t ldb, gemm_order_t orderB,
                                    float beta, const void *C, int64_t ldc,
                                    gemm_order_t orderC, int64_t batch, int64_t strideA,
                                    int64_t strideB, int64_t strideC, const void *workspace,
                                    size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_H */
