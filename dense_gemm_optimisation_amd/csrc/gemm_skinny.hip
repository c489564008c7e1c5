// GEMM with at most 16 rows of C (a skinny M: the batch of tokens in a
// decoding step, as in a 16 x 4096 x 4096 product), fp32, bf16 or fp16.
//
// Such a product is bound by reading B from HBM: A is a few KiB per k-slice
// and stays in L2, C is tiny.  Reaching HBM bandwidth takes enough bytes of B
// in flight to cover the memory latency on every compute unit, so the kernel
// is built around that rather than around tiles of C:
//
//   * a workgroup owns 16 columns of C (all M <= 16 rows), so N = 4096 gives
//     256 workgroups, one per compute unit; its 8 waves split K into
//     contiguous slices (split-K inside the workgroup, the sliced-K idea of
//     the rasterization and split-K section of "GPU GEMM 优化完全拆解（三）",
//     pinghaoyang.com.cn), so the partial sums are added in a fixed order
//     with no memory outside the kernel;
//   * each wave moves its slice of B into its own 16 KiB of LDS with direct
//     global -> LDS loads (16 bytes per lane), four 4 KiB chunks per round,
//     all issued before any is waited for: 128 KiB of B in flight per
//     compute unit.  Loads outside B or past the slice read as zero;
//   * A's fragments for the round go straight from global memory (L2) into
//     registers, one 16-byte load per lane per matrix-instruction step;
//   * the product is formed with the 16 x 16 matrix instructions
//     (v_mfma_f32_16x16x32_{bf16,f16}, v_mfma_f32_16x16x4_f32), operands
//     swapped (C^T = B^T A^T) so a lane ends with four consecutive columns of
//     one row.  A B chunk contiguous along N is stored [k][16 n] and read
//     with transposing LDS reads (16-bit types) or one float per k (fp32); a
//     chunk contiguous along K is stored [16 n][k] with its 16-byte chunks
//     XOR-swizzled by row and read 16 bytes at a time;
//   * the eight partials are summed through LDS in wave order; the epilogue
//     computes alpha*sum + beta*C_old in fp32 (C_old not read when
//     beta == 0) and rounds to the output type to nearest-even.
#include "gemm_problem.hpp"
#include "lds_dma.hpp"
#include "tile_schedule.hpp"

namespace libgemm {
namespace {

using dma::OOB;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int WAVES = 8;
constexpr int TN = 16;       // columns of C per workgroup; rows: M <= 16
constexpr int CHUNK = 4096;  // bytes of B per chunk
constexpr int RING = 4;      // chunks per wave per round
constexpr int OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2;

struct F32 {};
struct BF16 {};
struct F16 {};

// Element size in bytes of each input type.
template <class T>
struct Kind {
    static constexpr int SIZE = 2;
};
template <>
struct Kind<F32> {
    static constexpr int SIZE = 4;
};

struct SkinnyArgs {
    int64_t M, N, K;
    float alpha, beta;
    const void *A;
    const void *B;
    void *C;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;
    int64_t tiles_n;
    int64_t kper;  // k per wave slice, a multiple of the k per chunk
    Epilogue epi;
};

template <class T>
__device__ inline f4 mfma_step(u32x4 b, u32x4 a, f4 acc);
template <>
__device__ inline f4 mfma_step<BF16>(u32x4 b, u32x4 a, f4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                   __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
}
template <>
__device__ inline f4 mfma_step<F16>(u32x4 b, u32x4 a, f4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b),
                                                  __builtin_bit_cast(f16x8, a), acc, 0, 0, 0);
}
// fp32: the lane's four k values feed four instructions (k = 4*group + e).
// (Each element is copied to a scalar before the bit cast: a bit cast of a
// vector element expression reads element 0 with this compiler.)
template <>
__device__ inline f4 mfma_step<F32>(u32x4 b, u32x4 a, f4 acc) {
    const f4 bf = __builtin_bit_cast(f4, b), af = __builtin_bit_cast(f4, a);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float be = bf[e], ae = af[e];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(be, ae, acc, 0, 0, 0);
    }
    return acc;
}

template <class T, bool B_KMAJOR>
struct Chunk {
    static constexpr int SIZE = Kind<T>::SIZE;
    static constexpr int PER16 = 16 / SIZE;               // elements per 16 bytes
    static constexpr int CK = CHUNK / (TN * SIZE);        // k per chunk (128 or 64)
    static constexpr int STEP_K = 4 * PER16;              // k per step (32 or 16)
    static constexpr int STEPS = CK / STEP_K;             // steps per chunk (4)
    static constexpr int ROW = TN * SIZE;                 // bytes per k row, N-contiguous
    static_assert(STEPS == 4 && CHUNK / 1024 == 4, "chunk shape");

    // The four direct loads of the chunk of k values [k0, k0 + CK) (k < kend
    // valid) into LDS at `lds`.  Lane L of load b fills 16-byte piece
    // P = 64b + L of the chunk.
    __device__ static void issue(dma::u32x4 rs, uint32_t lds, int64_t n0, int64_t N, int64_t ld,
                                 int64_t k0, int64_t kend, int lane) {
#pragma unroll
        for (int b = 0; b < CHUNK / 1024; ++b) {
            const int P = 64 * b + lane;
            uint32_t v;
            if (B_KMAJOR) {  // [16 n][CK k]: 16 pieces per n row, swizzled by row
                const int n = P >> 4, c = (P & 15) ^ n;
                const int64_t gn = n0 + n, gk = k0 + c * PER16;
                v = (gn < N && gk < kend) ? uint32_t((gn * ld + gk) * SIZE) : OOB;
            } else {  // [CK k][16 n]: ROW / 16 pieces per k row
                constexpr int PPR = ROW / 16;
                const int krow = P / PPR, q = P % PPR;
                const int64_t gk = k0 + krow, gn = n0 + q * PER16;
                v = (gk < kend && gn < N) ? uint32_t((gk * ld + gn) * SIZE) : OOB;
            }
            dma::direct_load16(rs, lds + b * 1024, v);
        }
    }

    // B operand of step s for lane (j = lane % 16, G = lane / 16): column
    // n0 + j, the PER16 values of k = s*STEP_K + G*PER16 + 0.. in order.
    __device__ static u32x4 frag(const LDS char *chunk, int s, int lane) {
        const int j = lane & 15, G = lane >> 4;
        if (B_KMAJOR) {
            const int c = s * 4 + G;
            return *reinterpret_cast<const LDS u32x4 *>(chunk + j * (CK * SIZE) + ((c ^ j) << 4));
        } else if (SIZE == 4) {
            u32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = *reinterpret_cast<const LDS uint32_t *>(
                    chunk + (s * STEP_K + G * PER16 + e) * ROW + j * 4);
            return out;
        } else {
            // transposing reads: within each 16-lane group, lane i addresses k
            // row (i >> 2) and columns 4*(i & 3) .. +3 of a 4 x 16 block and
            // lane j receives column j of the block's four rows
            u32x4 out;
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const int krow = s * STEP_K + G * PER16 + 4 * e2 + (j >> 2);
                const LDS s16x4 *p =
                    reinterpret_cast<const LDS s16x4 *>(chunk + krow * ROW + (4 * (j & 3)) * 2);
                const u32x2 v = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<LDS s16x4 *>(p)));
                out[2 * e2] = v[0];
                out[2 * e2 + 1] = v[1];
            }
            return out;
        }
    }
};

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

template <class T, int OUT, bool B_KMAJOR>
__global__ __launch_bounds__(WAVES * 64, 1) void skinny_kernel(SkinnyArgs p) {
    using CB = Chunk<T, B_KMAJOR>;
    constexpr int SIZE = CB::SIZE, CK = CB::CK, STEP_K = CB::STEP_K;
    constexpr int RK = RING * CK;  // k per round
    __shared__ __attribute__((aligned(1024))) char smem[WAVES * RING * CHUNK];

    // consecutive column blocks (which share cache lines of B when it is
    // N-contiguous) go to one XCD
    const int64_t id = xcd_remap(blockIdx.x, gridDim.x, 8);
    const int64_t batch = dma::uniform(id / p.tiles_n);
    const int64_t n0 = dma::uniform((id - batch * p.tiles_n) * TN);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, G = lane >> 4;

    const char *A = static_cast<const char *>(p.A) + batch * p.sA * SIZE;
    const char *B = static_cast<const char *>(p.B) + batch * p.sB * SIZE;
    const int64_t span_a = (p.M - 1) * p.lda + p.K;
    const int64_t span_b = B_KMAJOR ? (p.N - 1) * p.ldb + p.K : (p.K - 1) * p.ldb + p.N;
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(A), 0, static_cast<int>(span_a * SIZE), 0x00020000);
    const dma::u32x4 rsb = dma::raw_buffer(
        static_cast<uint64_t>(dma::uniform(reinterpret_cast<int64_t>(B))), uint32_t(span_b * SIZE));

    // this wave's slice of K
    const int64_t kw0 = wave * p.kper;
    const int64_t kw1 = kw0 + p.kper < p.K ? kw0 + p.kper : p.K;
    LDS char *mine = (LDS char *)smem + wave * RING * CHUNK;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(mine));

    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t r0 = kw0; r0 < kw1; r0 += RK) {
        // every chunk of B of the round, then A's fragments for it
#pragma unroll
        for (int c = 0; c < RING; ++c)
            CB::issue(rsb, lds0 + c * CHUNK, n0, p.N, p.ldb, r0 + c * CK, kw1, lane);
        u32x4 a[RING * CB::STEPS];
#pragma unroll
        for (int t = 0; t < RING * CB::STEPS; ++t) {
            const int64_t k = r0 + t * STEP_K + G * CB::PER16;
            const int v = (j < p.M && k < kw1) ? static_cast<int>((j * p.lda + k) * SIZE)
                                               : static_cast<int>(OOB);
            a[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsa, v, 0, 0));
        }
        dma::wait_vmcnt<0>();
#pragma unroll
        for (int c = 0; c < RING; ++c)
#pragma unroll
            for (int s = 0; s < CB::STEPS; ++s)
                acc = mfma_step<T>(CB::frag(mine + c * CHUNK, s, lane), a[c * CB::STEPS + s], acc);
        // the next round's loads overwrite these chunks
        dma::wait_lgkmcnt0();
    }

    // Sum of the eight partials through LDS, in wave order.  Partial w,
    // register r, lane l is at red[(w * 4 + r) * 64 + l]; it is element
    // (l % 16, n0 + 4*(l / 16) + r) of C (C^T blocks).
    __syncthreads();  // every wave is done with its chunks
    LDS float *red = (LDS float *)smem;
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    if (tid < 4 * 64) {
        const int r = tid >> 6, l = tid & 63;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[(w * 4 + r) * 64 + l];
        const int64_t m = l & 15, n = n0 + 4 * (l >> 4) + r;
        if (m < p.M && n < p.N) {
            char *Cb = static_cast<char *>(p.C) + batch * p.sC * (OUT == OUT_F32 ? 4 : 2);
            const int64_t off = m * p.ldc + n;
            float v = p.alpha * s;
            if (p.beta != 0.0f) v = __builtin_fmaf(p.beta, load_c<OUT>(Cb, off), v);
            if (p.epi.active()) v = epilogue_apply(p.epi, v, batch, m, n);
            store_c<OUT>(Cb, off, v);
        }
    }
}

template <class T, int OUT>
hipError_t launch(const Problem &p, SkinnyArgs &a, int64_t blocks, hipStream_t stream) {
    void *args[] = {&a};
    const void *fn = p.b_kmajor ? reinterpret_cast<const void *>(&skinny_kernel<T, OUT, true>)
                                : reinterpret_cast<const void *>(&skinny_kernel<T, OUT, false>);
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(WAVES * 64), args, 0,
                           stream);
}

// ---- split-K across workgroups (workspace entry points), N-contiguous B
//
// With B contiguous along N, the kernel above gives each workgroup 16 columns
// of B: 32 bytes (16-bit) of every 128-byte line, the other three quarters
// fetched by three other compute units, and the request rate per compute
// unit, not HBM, sets its speed.  Here a workgroup of 8 waves owns 128 columns
// (256 contiguous bytes of every row of a 16-bit B) and one slice of K, so
// every line it fetches is all useful and each row gives two consecutive
// lines (measured: 32-byte pieces of a row reach 1.6 TB/s, 128-byte ones 2.5,
// 256-byte ones above 3); the K slices are split over enough
// workgroups to give every compute unit several ("Split-K", in the
// rasterization and split-K section of "GPU GEMM 优化完全拆解（三）",
// pinghaoyang.com.cn).  Each workgroup moves its slice of B into 32 KiB of
// LDS with direct loads, 16-byte chunks XOR-swizzled by row for the
// transposing reads, and each wave computes one 16 x 16 block of C^T over the
// slice; the partial blocks go to the workspace, and skinny_sk_reduce adds
// the slices of every element in increasing slice order (deterministic) and
// applies the epilogue.
constexpr int SK_NB = 128;             // columns of C per workgroup
constexpr int SK_WAVES = 8;            // one 16-column block each
constexpr int SK_TILE = 32768;         // bytes of B per round: 128 k rows of 128 columns
constexpr int SK_ATILE = 4096;         // bytes of A per round: 16 rows of 128 k
constexpr int SK_STAGE = SK_TILE + SK_ATILE;
constexpr int SK_STAGES = 2;           // rounds in flight

struct SkinnySkArgs {
    int64_t M, N, K;
    const void *A;
    const void *B;
    int64_t lda, ldb, sA, sB;
    int64_t nblk, split, kslice, batch;
    float *part;       // [split][batch][M][nblk * SK_NB] fp32
};

// 16-bit inputs.  Each round moves 128 k rows of the workgroup's 128 columns
// of B and the same 128 k of A's 16 rows into one slot of a two-slot LDS ring,
// with direct loads; the next round's loads are in flight while this one is
// multiplied.  A sits in LDS beside B because every wave needs the same A
// fragments, and reading them from global memory at each step would put an
// L2 round trip in front of every matrix instruction.
template <class T>
__global__ __launch_bounds__(SK_WAVES * 64) void skinny_sk_kernel(SkinnySkArgs p) {
    constexpr int SIZE = Kind<T>::SIZE;
    static_assert(SIZE == 2, "16-bit inputs");
    constexpr int ROW = SK_NB * SIZE;          // 256 bytes of B per k row
    constexpr int CPR = ROW / 16;              // 16 chunks of 16 bytes per row
    constexpr int R = SK_TILE / ROW;           // 128 k rows per round
    constexpr int AROW = R * SIZE;             // 256 bytes of A per row per round
    constexpr int ACPR = AROW / 16;            // 16 chunks per A row
    static_assert(16 * AROW == SK_ATILE && ACPR == 16, "A tile shape");
    constexpr int STEP_K = 32;                 // k per matrix-instruction step
    constexpr int LOADS = SK_TILE / 1024 / SK_WAVES;  // B loads per wave per round (4)
    constexpr int ALOADS = SK_ATILE / 1024;           // waves 0..3 load one A piece each
    __shared__ __attribute__((aligned(1024))) char smem[SK_STAGES * SK_STAGE];

    const int64_t id = blockIdx.x;
    const int64_t nb = id % p.nblk;
    const int64_t q = dma::uniform((id / p.nblk) % p.split);
    const int64_t batch = dma::uniform(id / (p.nblk * p.split));
    const int64_t n0 = dma::uniform(nb * SK_NB);
    const int64_t kb = q * p.kslice;
    const int64_t ke = kb + p.kslice < p.K ? kb + p.kslice : p.K;
    const int64_t rounds = (ke - kb + R - 1) / R;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, G = lane >> 4;

    const char *A = static_cast<const char *>(p.A) + batch * p.sA * SIZE;
    const char *B = static_cast<const char *>(p.B) + batch * p.sB * SIZE;
    const int64_t span_a = (p.M - 1) * p.lda + p.K;
    const int64_t span_b = (p.K - 1) * p.ldb + p.N;
    const dma::u32x4 rsa = dma::raw_buffer(
        static_cast<uint64_t>(dma::uniform(reinterpret_cast<int64_t>(A))), uint32_t(span_a * SIZE));
    const dma::u32x4 rsb = dma::raw_buffer(
        static_cast<uint64_t>(dma::uniform(reinterpret_cast<int64_t>(B))), uint32_t(span_b * SIZE));
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS char *)smem));

    // Round r into slot r % SK_STAGES.  B piece P is k row P / CPR, physical
    // chunk P % CPR, which holds logical chunk (P % CPR) ^ (row % CPR); A
    // piece P is row P / ACPR with its chunks swizzled by the row the same
    // way.  Waves 0..3 issue their A piece first, so every wave's loads
    // complete round by round.
    auto issue = [&](int64_t r) {
        const int64_t kr = kb + r * R;
        const uint32_t slot = lds0 + static_cast<uint32_t>(r % SK_STAGES) * SK_STAGE;
        if (wave < ALOADS) {
            const int P = wave * 64 + lane;
            const int row = P / ACPR;
            const int64_t gk = kr + ((P % ACPR) ^ row) * 8;
            const uint32_t v = (row < p.M && gk < ke) ? uint32_t((row * p.lda + gk) * SIZE) : OOB;
            dma::direct_load16(rsa, slot + SK_TILE + wave * 1024, v);
        }
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int P = (wave * LOADS + i) * 64 + lane;
            const int row = P / CPR;
            const int lc = (P % CPR) ^ (row % CPR);
            const int64_t gk = kr + row, gn = n0 + lc * 8;
            const uint32_t v = (gk < ke && gn < p.N) ? uint32_t((gk * p.ldb + gn) * SIZE) : OOB;
            dma::direct_load16(rsb, slot + (wave * LOADS + i) * 1024, v);
        }
    };

    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t r = 0; r < SK_STAGES - 1 && r < rounds; ++r) issue(r);
    for (int64_t r = 0; r < rounds; ++r) {
        if (r + SK_STAGES - 1 < rounds) {
            issue(r + SK_STAGES - 1);
            // the loads issued after round r's: one round's worth
            if (wave < ALOADS) dma::wait_vmcnt<(SK_STAGES - 1) * (LOADS + 1)>();
            else dma::wait_vmcnt<(SK_STAGES - 1) * LOADS>();
        } else {
            dma::wait_vmcnt<0>();
        }
        __syncthreads();
        const LDS char *tile = (const LDS char *)smem + (r % SK_STAGES) * SK_STAGE;
        const LDS char *atile = tile + SK_TILE;
        const int64_t rows = ke - kb - r * R < R ? ke - kb - r * R : R;
        const int steps = static_cast<int>((rows + STEP_K - 1) / STEP_K);
        for (int st = 0; st < steps; ++st) {
            // A: row j, logical chunk 4 * st + G (k = 32 st + 8 G .. +7)
            const u32x4 a = *reinterpret_cast<const LDS u32x4 *>(atile + j * AROW + (((4 * st + G) ^ j) << 4));
            // B: transposing reads, as in Chunk::frag, on the tile's 16
            // columns 16 * wave .. +15
            u32x4 b;
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const int krow = st * STEP_K + G * 8 + 4 * e2 + (j >> 2);
                const int byte = (wave * 16 + 4 * (j & 3)) * 2;
                const int pc = (byte >> 4) ^ (krow % CPR);
                const LDS s16x4 *ptr = reinterpret_cast<const LDS s16x4 *>(
                    tile + krow * ROW + (pc << 4) + (byte & 15));
                const u32x2 v = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<LDS s16x4 *>(ptr)));
                b[2 * e2] = v[0];
                b[2 * e2 + 1] = v[1];
            }
            acc = mfma_step<T>(b, a, acc);
        }
        __syncthreads();  // the round after next overwrites this slot
    }
    // lane l holds C^T block element (row l % 16, columns 4*(l / 16) + r)
    const int64_t m = lane & 15;
    if (m < p.M) {
        const int64_t Np = p.nblk * SK_NB;
        float *dst = p.part + ((q * p.batch + batch) * p.M + m) * Np + n0 + wave * 16 + 4 * G;
        *reinterpret_cast<f4 *>(dst) = acc;
    }
}

// A workgroup of four waves covers 64 groups of four consecutive columns of
// one row of C; wave g adds slice quarter g (slices in increasing order) and
// wave 0 then adds the four quarters in order, so every element's sum has
// one fixed order, and applies alpha, beta * C_old and the epilogue.
template <int OUT>
__global__ __launch_bounds__(256) void skinny_sk_reduce(SkinnySkArgs p, float alpha, float beta,
                                                       void *C, int64_t ldc, int64_t sC, Epilogue epi) {
    __shared__ f4 quarter[4][64];
    const int64_t Np = p.nblk * SK_NB;
    const int64_t quads = Np / 4;
    const int64_t total = p.batch * p.M * quads;
    const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int64_t t = blockIdx.x * int64_t(64) + lane;
    const bool live = t < total;
    const int64_t tt = live ? t : 0;
    const int64_t n = (tt % quads) * 4;
    const int64_t m = (tt / quads) % p.M;
    const int64_t batch = tt / (quads * p.M);
    const int64_t per = (p.split + 3) / 4;
    const int64_t q0 = g * per, q1 = q0 + per < p.split ? q0 + per : p.split;
    const float *src = p.part + (batch * p.M + m) * Np + n;
    const int64_t qstride = p.batch * p.M * Np;
    f4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live) {
        int64_t q = q0;
        for (; q + 4 <= q1; q += 4) {
            f4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const f4 *>(src + (q + u) * qstride);
#pragma unroll
            for (int u = 0; u < 4; ++u) s += v[u];
        }
        for (; q < q1; ++q) s += *reinterpret_cast<const f4 *>(src + q * qstride);
    }
    quarter[g][lane] = s;
    __syncthreads();
    if (g != 0 || !live) return;
    s = ((quarter[0][lane] + quarter[1][lane]) + quarter[2][lane]) + quarter[3][lane];
    char *Cb = static_cast<char *>(C) + batch * sC * (OUT == OUT_F32 ? 4 : 2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (n + e >= p.N) continue;
        const int64_t off = m * ldc + n + e;
        float v = alpha * s[e];
        if (beta != 0.0f) v = __builtin_fmaf(beta, load_c<OUT>(Cb, off), v);
        if (epi.active()) v = epilogue_apply(epi, v, batch, m, n + e);
        store_c<OUT>(Cb, off, v);
    }
}

// The split: about SK_GRID workgroups in all, slices a whole number of
// instruction steps.  More slices keep more loads in flight but write more
// partial sums (split * M * N * 4 bytes, written once and read once).
#ifndef LIBGEMM_SKINNY_SK_GRID
#define LIBGEMM_SKINNY_SK_GRID 512
#endif
constexpr int64_t SK_GRID = LIBGEMM_SKINNY_SK_GRID;

SkinnySkArgs sk_args(const Problem &p) {
    SkinnySkArgs a{};
    const int esz = elem_bytes(p.in);
    const int64_t step = 64 / esz;  // k per instruction step
    a.M = p.M;
    a.N = p.N;
    a.K = p.K;
    a.A = p.A;
    a.B = p.B;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.sA = p.batch > 1 ? p.sA : 0;
    a.sB = p.batch > 1 ? p.sB : 0;
    a.batch = p.batch;
    a.nblk = (p.N + SK_NB - 1) / SK_NB;
    int64_t split = SK_GRID / (a.nblk * p.batch);
    const int64_t max_split = (p.K + step - 1) / step;
    split = split < 1 ? 1 : (split > max_split ? max_split : split);
    a.kslice = ((p.K + split - 1) / split + step - 1) / step * step;
    a.split = (p.K + a.kslice - 1) / a.kslice;
    return a;
}

template <class T, int OUT>
hipError_t launch_sk(const Problem &p, SkinnySkArgs &a, hipStream_t stream) {
    void *args[] = {&a};
    const int64_t blocks = a.nblk * a.split * a.batch;
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&skinny_sk_kernel<T>),
                                   dim3(static_cast<unsigned>(blocks)), dim3(SK_WAVES * 64), args, 0,
                                   stream);
    if (e != hipSuccess) return e;
    const int64_t outs = a.batch * a.M * (a.nblk * SK_NB / 4);
    float alpha = p.alpha, beta = p.beta;
    void *C = p.C;
    int64_t ldc = p.ldc, sC = p.batch > 1 ? p.sC : 0;
    Epilogue epi = p.epi;
    void *rargs[] = {&a, &alpha, &beta, &C, &ldc, &sC, &epi};
    return hipLaunchKernel(reinterpret_cast<const void *>(&skinny_sk_reduce<OUT>),
                           dim3(static_cast<unsigned>((outs + 63) / 64)), dim3(256), rargs, 0, stream);
}

}  // namespace

// At most 16 rows of C, A contiguous along K, a K worth splitting eight
// ways, and operands the direct loads can read whole 16-byte chunks of (the
// same conditions as the main kernels' direct-load paths).  For fp32 the
// kernel's 16-column blocks read half cache lines of an N-contiguous B,
// where the fp32 split-K kernel's 32-column blocks read whole ones; measured
// on MI355X that kernel is faster there, and also once N is large enough to
// give it 256 or more workgroups, so fp32 takes this path only for a
// K-contiguous B and N below 8192.
#ifndef LIBGEMM_SKINNY_MAX_M
#define LIBGEMM_SKINNY_MAX_M 16
#endif

bool skinny_eligible(const Problem &p) {
    if (p.M > LIBGEMM_SKINNY_MAX_M || !p.a_kmajor || p.K < 256) return false;
    if (p.in == Elem::F32) return p.b_kmajor && p.N < 8192 && sgemm_dma_eligible(p);
    return hgemm_dma_eligible(p);
}

hipError_t launch_skinny(const Problem &p, hipStream_t stream) {
    SkinnyArgs a{};
    a.M = p.M;
    a.N = p.N;
    a.K = p.K;
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.A = p.A;
    a.B = p.B;
    a.C = p.C;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.sA = p.batch > 1 ? p.sA : 0;
    a.sB = p.batch > 1 ? p.sB : 0;
    a.sC = p.batch > 1 ? p.sC : 0;
    a.tiles_n = (p.N + TN - 1) / TN;
    const int64_t ck = CHUNK / (TN * elem_bytes(p.in));
    a.kper = ((p.K + WAVES * ck - 1) / (WAVES * ck)) * ck;
    a.epi = p.epi;
    const int64_t blocks = a.tiles_n * p.batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (p.in == Elem::F32) return launch<F32, OUT_F32>(p, a, blocks, stream);
    const bool bf = p.in == Elem::BF16;
    if (p.out == Elem::F32)
        return bf ? launch<BF16, OUT_F32>(p, a, blocks, stream)
                  : launch<F16, OUT_F32>(p, a, blocks, stream);
    return bf ? launch<BF16, OUT_BF16>(p, a, blocks, stream)
              : launch<F16, OUT_F16>(p, a, blocks, stream);
}

// Split-K across workgroups for at most 16 rows of C and an N-contiguous B
// (workspace entry points): the same operand conditions as skinny_eligible,
// 16-bit inputs, and a problem big enough for the split to matter.
bool skinny_sk_eligible(const Problem &p) {
    if (p.in == Elem::F32 || p.b_kmajor || !skinny_eligible(p)) return false;
    if (p.N < 256 || p.K < 1024) return false;
    const SkinnySkArgs a = sk_args(p);
    return a.nblk * a.split * a.batch <= 0x7fffffff && a.batch * a.M * a.nblk * SK_NB / 4 <= 0x7fffffff;
}

int64_t skinny_sk_bytes(const Problem &p) {
    const SkinnySkArgs a = sk_args(p);
    return a.split * a.batch * p.M * a.nblk * SK_NB * 4;
}

hipError_t launch_skinny_sk(const Problem &p, void *workspace, hipStream_t stream) {
    SkinnySkArgs a = sk_args(p);
    a.part = static_cast<float *>(workspace);
    const bool bf = p.in == Elem::BF16;
    if (p.out == Elem::F32)
        return bf ? launch_sk<BF16, OUT_F32>(p, a, stream) : launch_sk<F16, OUT_F32>(p, a, stream);
    return bf ? launch_sk<BF16, OUT_BF16>(p, a, stream) : launch_sk<F16, OUT_F16>(p, a, stream);
}

}  // namespace libgemm
