/*
 * CPU oracle for the dense general matrix multiply C = alpha*A*B + beta*C.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library: it is a separate, plain C
 * program that anyone can check against the definition by eye.
 *
 * What it follows:
 *   - "CUDA GEMM 矩阵乘法优化指南" (blog.zhenwei.site), section 2.1: the GEMM
 *     definition C = alpha x A x B + beta x C with A of size M x K, B of size
 *     K x N and C of size M x N, each output element taking K multiply-adds.
 *   - the CUDA SGEMM optimisation article at m.lqnn.cn, section 1.2: the
 *     kernel result is checked against a CPU computation in double precision.
 *
 * Every output element is the textbook dot product, accumulated in double, in
 * increasing k order, one rounded double multiply and one rounded double add
 * per step (the file is compiled with -ffp-contract=off so nothing is fused).
 * Inputs are decoded from their stored bit patterns exactly into double.
 * Alongside the result the oracle returns the magnitude scale of the terms,
 *   den = |alpha| * sum_k |A_ik * B_kj| + |beta| * |C0_ij|,
 * which the tests use to normalise the error of a GPU result.
 *
 * The fused epilogue (optional): the pages fold "GEMM + bias + activation"
 * into one kernel ("第4章：经典算子实现 —— GEMM", aiinfra.vidrealm.tech,
 * section 7.2, on CUTLASS) and apply element-wise operations such as ReLU on
 * the accumulators before the store ("GPU GEMM 优化完全拆解（三）",
 * pinghaoyang.com.cn, section on mainloop and epilogue).  Here
 *   D_ij = act(alpha * sum_k A_ik B_kj + beta * C0_ij + bias_j),
 * bias_j the j-th element of a vector of N input-type values (one per
 * column of C, the b-th batch entry sBias elements after the previous one),
 * act one of identity, ReLU max(x, 0), or GELU x * Phi(x) with Phi the
 * standard normal distribution function, 0.5 * (1 + erf(x / sqrt 2)).  den
 * gains |bias_j|; it stays the scale of the terms before the activation.
 *
 * 8-bit inputs: the pages list the 8-bit floating formats E4M3 and E5M2 for
 * matrix units ("CUDA GEMM 矩阵乘法优化指南", blog.zhenwei.site, section
 * 13.2).  They are the OCP formats: E4M3 has no infinities and one NaN
 * pattern per sign (S.1111.111), largest finite 448; E5M2 follows the IEEE
 * rules (infinities at exponent 31 with a zero fraction, NaNs otherwise).
 * Both have subnormals.  A and B may be in different 8-bit formats.
 *
 * Block-scaled (MX) inputs: the pages list the microscaling formats MXFP8,
 * MXFP6 and MXFP4, in which every 32 consecutive elements share one E8M0
 * scale factor, an 8-bit exponent with no sign or fraction ("CUDA GEMM
 * 矩阵乘法优化指南", blog.zhenwei.site, section 13.2, on block-scale
 * quantisation).  The value of element k of a row is its scale times its own
 * value: X[k] = 2^(e(k/32) - 127) * x[k], the E8M0 pattern 255 being NaN.
 * Element formats: E4M3 and E5M2 as above; E2M3 (1 sign, 2 exponent bits,
 * bias 1, 3 fraction bits, largest 7.5) and E3M2 (1 sign, 3 exponent bits,
 * bias 3, 2 fraction bits, largest 28), both with subnormals and no
 * infinities or NaNs; E2M1 (1 sign, 2 exponent bits, bias 1, 1 fraction bit:
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6).  orc_mx_gemm below computes
 *   C_ij = alpha * sum_k XA(i,k) XB(k,j) + beta * C0_ij,
 * each product of two decoded, scaled elements formed in double and added
 * in increasing k order, as for the other types.
 *
 * Readings taken where the pages are silent:
 *   - beta == 0: C0 is not read (BLAS convention), so NaN in C0 does not leak.
 *   - alpha == 0 or K == 0: the product term is skipped and A, B are not read.
 *   - 16-bit results are rounded from double to the target format directly,
 *     round-to-nearest-even, never through float (no double rounding).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F16 2
#define ORC_E4M3 3 /* OCP 8-bit float: 1 sign, 4 exponent (bias 7), 3 fraction bits */
#define ORC_E5M2 4 /* OCP 8-bit float: 1 sign, 5 exponent (bias 15), 2 fraction bits */
/* Element and scale formats of the block-scaled (MX) inputs; orc_decode takes
 * them one value per byte (low bits), orc_mx_gemm packed (see mx_load). */
#define ORC_E2M3 5 /* 6-bit float: 1 sign, 2 exponent (bias 1), 3 fraction bits */
#define ORC_E3M2 6 /* 6-bit float: 1 sign, 3 exponent (bias 3), 2 fraction bits */
#define ORC_E2M1 7 /* 4-bit float: 1 sign, 2 exponent (bias 1), 1 fraction bit */
#define ORC_E8M0 8 /* scale: 2^(e - 127), 255 is NaN */

#define ORC_ROW 0
#define ORC_COL 1

#define ORC_ACT_NONE 0
#define ORC_ACT_RELU 1
#define ORC_ACT_GELU 2

/* ---------------------------------------------------------------- decoding */

static double decode_f32(uint32_t bits) {
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* bf16 is the top half of an IEEE binary32 pattern. */
static double decode_bf16(uint16_t bits) { return decode_f32((uint32_t)bits << 16); }

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t bits) {
    int sign = bits >> 15;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);             /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* E4M3: value (1 + m/8) * 2^(e-7), subnormal m/8 * 2^-6; S.1111.111 is NaN. */
static double decode_e4m3(uint8_t bits) {
    int sign = bits >> 7;
    int e = (bits >> 3) & 0xf;
    int m = bits & 0x7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);           /* m/8 * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* E5M2: value (1 + m/4) * 2^(e-15), subnormal m/4 * 2^-14; e == 31 is Inf/NaN. */
static double decode_e5m2(uint8_t bits) {
    int sign = bits >> 7;
    int e = (bits >> 2) & 0x1f;
    int m = bits & 0x3;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -16);          /* m/4 * 2^-14 */
    else
        v = ldexp((double)(4 + m), e - 17); /* (1 + m/4) * 2^(e-15) */
    return sign ? -v : v;
}

/*
 * A small float with no infinities or NaNs: sign bit s (above the others),
 * ebits exponent bits with bias `bias`, mbits fraction bits.  Normal values
 * (1 + m/2^mbits) * 2^(e - bias), subnormals (e == 0) m/2^mbits * 2^(1 - bias).
 */
static double decode_small(unsigned bits, int ebits, int mbits, int bias) {
    const unsigned m = bits & ((1u << mbits) - 1);
    const unsigned e = (bits >> mbits) & ((1u << ebits) - 1);
    const int s = (bits >> (ebits + mbits)) & 1;
    double v = e == 0 ? ldexp((double)m, 1 - bias - mbits)
                      : ldexp(1.0 + ldexp((double)m, -mbits), (int)e - bias);
    return s ? -v : v;
}

static double decode_e2m3(uint8_t bits) { return decode_small(bits & 0x3f, 2, 3, 1); }
static double decode_e3m2(uint8_t bits) { return decode_small(bits & 0x3f, 3, 2, 3); }
static double decode_e2m1(uint8_t bits) { return decode_small(bits & 0x0f, 2, 1, 1); }

/* E8M0: 2^(e - 127); the all-ones pattern is NaN. */
static double decode_e8m0(uint8_t bits) { return bits == 255 ? NAN : ldexp(1.0, (int)bits - 127); }

static double load(int type, const void *base, int64_t idx) {
    switch (type) {
    case ORC_F32: {
        uint32_t b;
        memcpy(&b, (const char *)base + 4 * idx, 4);
        return decode_f32(b);
    }
    case ORC_BF16:
        return decode_bf16(((const uint16_t *)base)[idx]);
    case ORC_E4M3:
        return decode_e4m3(((const uint8_t *)base)[idx]);
    case ORC_E5M2:
        return decode_e5m2(((const uint8_t *)base)[idx]);
    case ORC_E2M3:
        return decode_e2m3(((const uint8_t *)base)[idx]);
    case ORC_E3M2:
        return decode_e3m2(((const uint8_t *)base)[idx]);
    case ORC_E2M1:
        return decode_e2m1(((const uint8_t *)base)[idx]);
    case ORC_E8M0:
        return decode_e8m0(((const uint8_t *)base)[idx]);
    default:
        return decode_f16(((const uint16_t *)base)[idx]);
    }
}

/* Offset of element (r, c) of a matrix stored with leading dimension ld. */
static int64_t offset(int order, int64_t r, int64_t c, int64_t ld) {
    return order == ORC_ROW ? r * ld + c : c * ld + r;
}

/* ---------------------------------------------------------------- rounding */

/*
 * Round x to the nearest value of a binary format with p significand bits
 * (counting the implicit one), minimum normal exponent emin and maximum
 * exponent emax; ties go to even; results beyond the largest finite value
 * become infinity.  Within one binade the representable values are the
 * multiples of q = 2^(e - p + 1); below the normal range the spacing stays at
 * 2^(emin - p + 1).  x / q and r * q are exact (q is a power of two), and
 * nearbyint rounds to nearest-even in the default floating-point mode.
 */
static double round_to_format(double x, int p, int emin, int emax) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e2;
    frexp(x, &e2);          /* x = f * 2^e2 with 0.5 <= |f| < 1 */
    int e = e2 - 1;         /* x = 1.xxx * 2^e */
    if (e < emin) e = emin; /* subnormal range keeps the smallest spacing */
    double q = ldexp(1.0, e - (p - 1));
    double r = nearbyint(x / q) * q;
    double maxfinite = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxfinite) r = copysign(INFINITY, x);
    return r;
}

static uint16_t encode_bf16(double r) {
    /* r is already a bf16 value, hence exactly a binary32 value. */
    if (isnan(r)) return 0x7fc0;
    float f = (float)r;
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)(b >> 16);
}

static uint16_t encode_f16(double r) {
    if (isnan(r)) return 0x7e00;
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (isinf(a)) return sign | 0x7c00;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int e = e2 - 1;
    if (e < -14) /* subnormal: a = m * 2^-24 */
        return sign | (uint16_t)ldexp(a, 24);
    uint16_t m = (uint16_t)(ldexp(a, 10 - e) - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | m;
}

/*
 * 8-bit float outputs (the quantised epilogue: the epilogue section of "GPU
 * GEMM 优化完全拆解（三）" folds quantisation scaling into the write-back).
 * Round x to E4M3 or E5M2 by round_to_format, saturating: magnitudes beyond
 * the largest finite value (448 for E4M3, whose all-ones pattern is NaN;
 * 57344 for E5M2), infinities included, become that value with x's sign; a
 * NaN becomes the canonical NaN (0x7f, resp. 0x7e).
 */
static uint8_t encode_f8(double x, int e5m2) {
    const int p = e5m2 ? 3 : 4, emin = e5m2 ? -14 : -6, bias = e5m2 ? 15 : 7;
    const double maxfinite = e5m2 ? 57344.0 : 448.0;
    if (isnan(x)) return e5m2 ? 0x7e : 0x7f;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    /* at most maxfinite, a value of the format, rounds to at most maxfinite */
    double r = a > maxfinite ? maxfinite : round_to_format(a, p, emin, e5m2 ? 15 : 8);
    if (r == 0.0) return sign;
    int e2;
    frexp(r, &e2);
    int e = e2 - 1;
    if (e < emin) /* subnormal: r = m * 2^(emin - p + 1) */
        return sign | (uint8_t)ldexp(r, -(emin - p + 1));
    uint8_t m = (uint8_t)(ldexp(r, p - 1 - e) - ldexp(1.0, p - 1));
    return sign | (uint8_t)((e + bias) << (p - 1)) | m;
}

/* ---------------------------------------------------------------- exports */

int orc_version(void) { return 5; }

void orc_decode(int type, const void *src, double *dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = load(type, src, i);
}

/* Round doubles to the stored bit patterns of `type` (uint32 for f32). */
void orc_round(int type, const double *src, void *dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        switch (type) {
        case ORC_F32: {
            double r = round_to_format(src[i], 24, -126, 127);
            float f = (float)r; /* exact: r is a binary32 value or inf */
            if (isnan(src[i])) f = NAN;
            memcpy((char *)dst + 4 * i, &f, 4);
            break;
        }
        case ORC_BF16:
            ((uint16_t *)dst)[i] = encode_bf16(round_to_format(src[i], 8, -126, 127));
            break;
        case ORC_E4M3:
        case ORC_E5M2:
            ((uint8_t *)dst)[i] = encode_f8(src[i], type == ORC_E5M2);
            break;
        default:
            ((uint16_t *)dst)[i] = encode_f16(round_to_format(src[i], 11, -14, 15));
            break;
        }
    }
}

struct problem {
    int in_type, c_type;
    int b_type; /* type of B (and of the bias: in_type) */
    int64_t M, N, K;
    double alpha, beta;
    const void *A, *B, *C0;
    int64_t lda, ldb, ldc;
    int oA, oB, oC;
    int64_t sA, sB, sC;
    const void *bias; /* NULL: no bias */
    int64_t sBias;
    int act;
};

/*
 * One output element (b, i, j): the definition of section 2.1 of the
 * zhenwei.site guide, written out.  A(b,i,k) is element (i, k) of the b-th
 * M x K matrix, which starts sA elements after the previous one; likewise
 * B(b,k,j) and C0(b,i,j).
 */
static void finish(const struct problem *P, int64_t b, int64_t i, int64_t j, double s,
                   double t, double *ref, double *den);

static void element(const struct problem *P, int64_t b, int64_t i, int64_t j,
                    double *ref, double *den) {
    double s = 0.0, t = 0.0;
    if (P->alpha != 0.0) {
        const int64_t a0 = b * P->sA, b0 = b * P->sB;
        for (int64_t k = 0; k < P->K; ++k) {
            double a = load(P->in_type, P->A, a0 + offset(P->oA, i, k, P->lda));
            double x = load(P->b_type, P->B, b0 + offset(P->oB, k, j, P->ldb));
            double p = a * x;
            s = s + p;
            t = t + fabs(p);
        }
    }
    finish(P, b, i, j, s, t, ref, den);
}

/*
 * The rest of the definition once the dot product s (and the sum of the
 * absolute values of its terms, t) is known: alpha * s + beta * C0, the bias
 * and the activation.
 */
static void finish(const struct problem *P, int64_t b, int64_t i, int64_t j, double s,
                   double t, double *ref, double *den) {
    double r = P->alpha * s;
    double d = fabs(P->alpha) * t;
    if (P->beta != 0.0) {
        double c0 = load(P->c_type, P->C0, b * P->sC + offset(P->oC, i, j, P->ldc));
        r = r + P->beta * c0;
        d = d + fabs(P->beta) * fabs(c0);
    }
    if (P->bias != NULL) {
        double bj = load(P->in_type, P->bias, b * P->sBias + j);
        r = r + bj;
        d = d + fabs(bj);
    }
    if (P->act == ORC_ACT_RELU)
        r = r > 0.0 ? r : 0.0;
    else if (P->act == ORC_ACT_GELU)
        r = r * 0.5 * (1.0 + erf(r / sqrt(2.0)));
    *ref = r;
    *den = d;
}

#define PROBLEM_ARGS                                                                   \
    int in_type, int c_type, int64_t M, int64_t N, int64_t K, double alpha,            \
        const void *A, int64_t lda, int oA, const void *B, int64_t ldb, int oB,        \
        double beta, const void *C0, int64_t ldc, int oC, int64_t sA, int64_t sB,      \
        int64_t sC, const void *bias, int64_t sBias, int act, int b_type

#define PROBLEM_INIT                                                                   \
    struct problem P = {in_type, c_type, b_type, M,     N,  K,  alpha, beta, A,     \
                        B,       C0,     lda,    ldb,   ldc, oA, oB,    oC,   sA,    \
                        sB,      sC,     bias,   sBias, act}

/*
 * All batch*M*N elements; ref and den are dense [batch][M][N].
 *
 * The same arithmetic as element(), in another loop order: the slice of B is
 * decoded into doubles once, and each block of ROWS rows of C keeps one
 * running sum per element while k goes up, so every element still receives
 * its products one at a time in increasing k order, each a rounded double
 * multiply followed by a rounded double add (the file is built with
 * -ffp-contract=off).  Only the order in which different elements advance
 * changes, which no element's value depends on: the result equals element()
 * bit for bit (a CPU test compares the two on every element).
 */
#define ROWS 16
void orc_gemm(PROBLEM_ARGS, int64_t batch, double *ref, double *den) {
    PROBLEM_INIT;
    double *bd = alpha == 0.0 || K == 0 || N == 0
                     ? NULL
                     : (double *)malloc((size_t)K * (size_t)N * sizeof(double));
    if (bd == NULL) {  /* no product term, or no room for the decoded slice */
        const int64_t total = batch * M * N;
#pragma omp parallel for schedule(dynamic, 64)
        for (int64_t e = 0; e < total; ++e) {
            int64_t b = e / (M * N), i = (e / N) % M, j = e % N;
            element(&P, b, i, j, &ref[e], &den[e]);
        }
        return;
    }
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t b0 = b * sB, a0 = b * sA;
        if (b == 0 || sB != 0) {
#pragma omp parallel for schedule(static)
            for (int64_t k = 0; k < K; ++k)
                for (int64_t j = 0; j < N; ++j)
                    bd[k * N + j] = load(b_type, B, b0 + offset(oB, k, j, ldb));
        }
        const int64_t blocks = (M + ROWS - 1) / ROWS;
#pragma omp parallel
        {
            double *s = (double *)malloc((size_t)ROWS * (size_t)N * 2 * sizeof(double));
            double *t = s + (size_t)ROWS * (size_t)N;
#pragma omp for schedule(dynamic, 1)
            for (int64_t blk = 0; blk < blocks; ++blk) {
                const int64_t i0 = blk * ROWS;
                const int64_t rows = M - i0 < ROWS ? M - i0 : ROWS;
                if (s == NULL) {  /* no room for the running sums: the element loop */
                    for (int64_t r = 0; r < rows; ++r)
                        for (int64_t j = 0; j < N; ++j) {
                            const int64_t e = (b * M + i0 + r) * N + j;
                            element(&P, b, i0 + r, j, &ref[e], &den[e]);
                        }
                    continue;
                }
                for (int64_t e = 0; e < rows * N; ++e) s[e] = 0.0, t[e] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double *x = bd + k * N;
                    for (int64_t r = 0; r < rows; ++r) {
                        const double a = load(in_type, A, a0 + offset(oA, i0 + r, k, lda));
                        double *sr = s + r * N, *tr = t + r * N;
                        for (int64_t j = 0; j < N; ++j) {
                            const double p = a * x[j];
                            sr[j] = sr[j] + p;
                            tr[j] = tr[j] + fabs(p);
                        }
                    }
                }
                for (int64_t r = 0; r < rows; ++r)
                    for (int64_t j = 0; j < N; ++j) {
                        const int64_t e = (b * M + i0 + r) * N + j;
                        finish(&P, b, i0 + r, j, s[r * N + j], t[r * N + j], &ref[e], &den[e]);
                    }
            }
            free(s);
        }
    }
    free(bd);
}

/* Only the listed elements; idx holds count triples (b, i, j). */
void orc_gemm_at(PROBLEM_ARGS, int64_t count, const int64_t *idx, double *ref,
                 double *den) {
    PROBLEM_INIT;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t e = 0; e < count; ++e)
        element(&P, idx[3 * e], idx[3 * e + 1], idx[3 * e + 2], &ref[e], &den[e]);
}

/* ---------------------------------------------------------------- MX */

/*
 * Element idx of a packed MX operand in format fmt.  Storage: the elements
 * of a row follow one another as one little-endian bit stream, 8, 6 or 4
 * bits each: element idx occupies bits [w*idx, w*idx + w) of the stream,
 * bit n of the stream being bit n % 8 of byte n / 8.  (E4M3/E5M2: one byte
 * each; E2M3/E3M2: four elements in three bytes; E2M1: two per byte, the
 * lower index in the low half.)
 */
static int mx_width(int fmt) {
    return fmt == ORC_E2M1 ? 4 : (fmt == ORC_E2M3 || fmt == ORC_E3M2) ? 6 : 8;
}

static double mx_load(int fmt, const uint8_t *base, int64_t idx) {
    const int w = mx_width(fmt);
    const int64_t bit = idx * w;
    /* the (at most two) bytes that hold the element, low byte first */
    unsigned v = base[bit / 8];
    if (bit % 8 + w > 8) v |= (unsigned)base[bit / 8 + 1] << 8;
    v = (v >> (bit % 8)) & ((1u << w) - 1);
    switch (fmt) {
    case ORC_E4M3: return decode_e4m3((uint8_t)v);
    case ORC_E5M2: return decode_e5m2((uint8_t)v);
    case ORC_E2M3: return decode_e2m3((uint8_t)v);
    case ORC_E3M2: return decode_e3m2((uint8_t)v);
    default: return decode_e2m1((uint8_t)v);
    }
}

struct mx_problem {
    int fa, fb, c_type;
    int64_t M, N, K;
    double alpha, beta;
    const uint8_t *A, *SA, *B, *SB;
    const void *C0;
    int64_t lda, ldsa, ldb, ldsb, ldc;
    int oC;
    int64_t sA, sB, sSA, sSB, sC;
};

/*
 * Output element (b, i, j): A(i, k) is element b*sA + i*lda + k of A's
 * stream with scale SA[b*sSA + i*ldsa + k/32]; B(k, j) is element
 * b*sB + j*ldb + k of B's (K contiguous along each column of B) with scale
 * SB[b*sSB + j*ldsb + k/32].  Each side is decoded and scaled exactly, their
 * product formed in double and added in increasing k.
 */
static void mx_element(const struct mx_problem *P, int64_t b, int64_t i, int64_t j,
                       double *ref, double *den) {
    double s = 0.0, t = 0.0;
    if (P->alpha != 0.0) {
        for (int64_t k = 0; k < P->K; ++k) {
            const double xa = decode_e8m0(P->SA[b * P->sSA + i * P->ldsa + k / 32]) *
                              mx_load(P->fa, P->A, b * P->sA + i * P->lda + k);
            const double xb = decode_e8m0(P->SB[b * P->sSB + j * P->ldsb + k / 32]) *
                              mx_load(P->fb, P->B, b * P->sB + j * P->ldb + k);
            const double p = xa * xb;
            s = s + p;
            t = t + fabs(p);
        }
    }
    double r = P->alpha * s;
    double d = fabs(P->alpha) * t;
    if (P->beta != 0.0) {
        const double c0 = load(P->c_type, P->C0, b * P->sC + offset(P->oC, i, j, P->ldc));
        r = r + P->beta * c0;
        d = d + fabs(P->beta) * fabs(c0);
    }
    *ref = r;
    *den = d;
}

#define MX_ARGS                                                                           \
    int fa, int fb, int c_type, int64_t M, int64_t N, int64_t K, double alpha,            \
        const uint8_t *A, int64_t lda, const uint8_t *SA, int64_t ldsa, const uint8_t *B, \
        int64_t ldb, const uint8_t *SB, int64_t ldsb, double beta, const void *C0,        \
        int64_t ldc, int oC, int64_t sA, int64_t sB, int64_t sSA, int64_t sSB, int64_t sC

#define MX_INIT                                                                           \
    struct mx_problem P = {fa, fb,  c_type, M,   N,   K,  alpha, beta, A,   SA,  B,  SB,   \
                           C0, lda, ldsa,   ldb, ldsb, ldc, oC,   sA,   sB,  sSA, sSB, sC}

/* All batch*M*N elements; ref and den are dense [batch][M][N]. */
void orc_mx_gemm(MX_ARGS, int64_t batch, double *ref, double *den) {
    MX_INIT;
    const int64_t total = batch * M * N;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t e = 0; e < total; ++e)
        mx_element(&P, e / (M * N), (e / N) % M, e % N, &ref[e], &den[e]);
}

/* Only the listed elements; idx holds count triples (b, i, j). */
void orc_mx_gemm_at(MX_ARGS, int64_t count, const int64_t *idx, double *ref, double *den) {
    MX_INIT;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t e = 0; e < count; ++e)
        mx_element(&P, idx[3 * e], idx[3 * e + 1], idx[3 * e + 2], &ref[e], &den[e]);
}

/* Element idx of a packed MX operand, decoded (unscaled). */
double orc_mx_element(int fmt, const uint8_t *base, int64_t idx) { return mx_load(fmt, base, idx); }

#ifdef _OPENMP
#include <omp.h>
int orc_max_threads(void) { return omp_get_max_threads(); }
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int orc_max_threads(void) { return 1; }
void orc_set_threads(int n) { (void)n; }
#endif
