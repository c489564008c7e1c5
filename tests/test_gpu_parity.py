"""GPU parity: libgemm's HIP kernels against the CPU oracle, element by element.

Small and medium problems compare every element; full-size workloads compare
whole rows and columns, tile-boundary elements and random samples.  Every run
also checks the canary guard bands and ld/batch padding around C and that A
and B are unchanged (see parity.py for the tolerances).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from dense_gemm_optimisation_amd import binding
from workloads import COL, ROW, Problem

from parity import log, run

pytestmark = pytest.mark.gpu

DT = ["f32", "bf16", "f16"]


def P(name, dt, M, N, K, c_dtype=None, **kw):
    return Problem(name, dt, c_dtype or dt, M, N, K, **kw)


def check(p, kernel=None, **kw):
    """Run p against the oracle; with `kernel`, also require that the library
    launched that kernel (so a test of a fast path cannot silently fall back
    to another one)."""
    res, out = run(p, **kw)
    assert res.ok, res.why
    if kernel is not None:
        assert res.kernel == kernel, f"{p.name} ran on {res.kernel!r}, expected {kernel!r}"
    return res, out


# ------------------------------------------------------------------ shapes and edges

SHAPES = [(1, 1, 1), (1, 7, 3), (2, 3, 5), (7, 9, 13), (31, 33, 17), (64, 64, 64),
          (127, 129, 65), (128, 128, 128), (129, 127, 200), (255, 257, 63), (256, 256, 256),
          (300, 290, 130), (513, 130, 77), (70, 600, 33), (33, 70, 1000)]


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(dt, shape):
    M, N, K = shape
    check(P(f"shape-{dt}", dt, M, N, K, alpha=1.0, beta=0.0), seed=M * 7 + N * 3 + K)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (37, 45, 29), (256, 256, 64), (300, 290, 130)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp32_output(dt, shape):
    M, N, K = shape
    check(P(f"f32out-{dt}", dt, M, N, K, c_dtype="f32", alpha=0.75, beta=-1.5), seed=5)


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("orders", [(a, b, c) for a in (ROW, COL) for b in (ROW, COL)
                                    for c in (ROW, COL)], ids=lambda o: "%d%d%d" % o)
def test_layouts_with_padded_ld(dt, orders):
    oa, ob, oc = orders
    M, N, K = 261, 199, 150
    lda = (K if oa == ROW else M) + 13
    ldb = (N if ob == ROW else K) + 8
    ldc = (N if oc == ROW else M) + 5
    check(P(f"layout-{dt}", dt, M, N, K, alpha=1.25, beta=0.5, order_a=oa, order_b=ob,
            order_c=oc, lda=lda, ldb=ldb, ldc=ldc), seed=11)


@pytest.mark.parametrize("dt", DT)
def test_misaligned_bases_and_odd_ld(dt):
    p = P(f"misaligned-{dt}", dt, 190, 211, 97, alpha=1.0, beta=1.0, lda=99, ldb=213, ldc=215)
    check(p, seed=12, base_offset=(1, 3, 1))


@pytest.mark.parametrize("dt", DT)
def test_aligned_ld_but_ragged_k(dt):
    # 16-byte aligned rows, but K not a multiple of the vector width or tile
    check(P(f"raggedk-{dt}", dt, 300, 260, 1001, lda=1008, ldb=264, ldc=264), seed=13)


# ------------------------------------------------------------------ alpha / beta semantics

@pytest.mark.parametrize("dt", DT)
def test_beta_zero_ignores_nan_in_c(dt):
    nan = np.float32(np.nan) if dt == "f32" else (0x7FC0 if dt == "bf16" else 0x7E00)
    res, _ = check(P(f"beta0nan-{dt}", dt, 140, 150, 70, alpha=1.0, beta=0.0), seed=14,
                   c_init=nan)


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("case", ["alpha0", "k0", "alpha0_beta0"])
def test_scale_only_paths(dt, case):
    kw = dict(alpha=0.0, beta=-2.0) if case == "alpha0" else \
        dict(alpha=1.5, beta=0.5) if case == "k0" else dict(alpha=0.0, beta=0.0)
    K = 0 if case == "k0" else 33
    p = P(f"{case}-{dt}", dt, 77, 65, K, **kw)
    if case == "alpha0_beta0":
        nan = np.float32(np.nan) if dt == "f32" else (0x7FC0 if dt == "bf16" else 0x7E00)
        check(p, seed=15, c_init=nan)
    else:
        check(p, seed=15)


# ------------------------------------------------------------------ exact results

def _int_host(p, rng, lo=-8, hi=8):
    def mk(n, dt):
        v = rng.integers(lo, hi + 1, n).astype(np.float32)
        return v if dt == "f32" else workloads.to_16bit(v, dt)
    return (mk(p.buffer_elems("a"), p.in_dtype), mk(p.buffer_elems("b"), p.in_dtype),
            mk(p.buffer_elems("c"), p.c_dtype))


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("shape", [(256, 256, 1001), (300, 517, 260), (64, 4096, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_integer_inputs_bit_exact(dt, shape):
    # every product and partial sum of small integers is exact in fp32, so
    # the result must equal the oracle's correctly rounded value bit for bit
    M, N, K = shape
    p = P(f"int-{dt}", dt, M, N, K, alpha=2.0, beta=1.0)
    host = _int_host(p, np.random.default_rng(16))
    res, out = check(p, host=host)
    assert res.max_err == 0.0 and res.max_ulp == 0


@pytest.mark.parametrize("dt", DT)
def test_identity_and_permutation_bit_exact(dt):
    M, N = 300, 257
    rng = np.random.default_rng(17)
    perm = rng.permutation(M)
    Pm = np.zeros((M, M), np.float32)
    Pm[np.arange(M), perm] = 1.0
    for name, a in (("identity", np.eye(M, dtype=np.float32)), ("permutation", Pm)):
        p = P(f"{name}-{dt}", dt, M, N, M)
        a_st = a.ravel() if dt == "f32" else workloads.to_16bit(a.ravel(), dt)
        _, b, c = workloads.generate(p, seed=18)
        res, out = check(p, host=(a_st, b, c))
        if dt != "f32":
            assert res.max_ulp == 0


@pytest.mark.parametrize("dt", DT)
def test_all_ones_closed_form(dt):
    M, N, K = 200, 300, 700
    p = P(f"ones-{dt}", dt, M, N, K, alpha=0.5, beta=-1.0)
    one = np.ones(1, np.float32)
    mk = (lambda n: np.ones(n, np.float32)) if dt == "f32" else \
        (lambda n: workloads.to_16bit(np.ones(n, np.float32), dt))
    c0 = np.random.default_rng(19).integers(-4, 5, M * N).astype(np.float32)
    c0s = c0 if dt == "f32" else workloads.to_16bit(c0, dt)
    res, out = check(p, host=(mk(M * K), mk(K * N), c0s))
    assert res.max_err == 0.0 and res.max_ulp == 0
    del one


# ------------------------------------------------------------------ batches

@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("bcast", ["none", "a", "b"])
def test_batched_strided(dt, bcast):
    M, N, K, batch = 130, 260, 90, 3
    kw = {}
    if bcast == "a":
        kw["stride_a"] = 0
    if bcast == "b":
        kw["stride_b"] = 0
    p = P(f"batch-{bcast}-{dt}", dt, M, N, K, batch=batch, beta=1.0, stride_c=M * N + 17, **kw)
    res, out = check(p, seed=20)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_batch_slice_equals_single_call(dt):
    M, N, K, batch = 257, 129, 140, 3
    pb = P(f"batch-vs-single-{dt}", dt, M, N, K, batch=batch)
    a, b, c = workloads.generate(pb, seed=21)
    _, out_b = check(pb, host=(a, b, c))
    from parity import GUARD
    for i in range(batch):
        ps = P(f"single{i}-{dt}", dt, M, N, K)
        sl = lambda x, s, n: x[i * s:i * s + n]
        host = (sl(a, pb.stride_a, M * K), sl(b, pb.stride_b, K * N), sl(c, pb.stride_c, M * N))
        _, out_s = check(ps, host=host)
        assert np.array_equal(out_s[GUARD:GUARD + M * N],
                              out_b[GUARD + i * pb.stride_c:GUARD + i * pb.stride_c + M * N])


@pytest.mark.parametrize("dt", DT)
def test_repeat_runs_bit_identical(dt):
    check(P(f"determinism-{dt}", dt, 520, 700, 300, beta=0.5), seed=22, repeat=3)


# ------------------------------------------------------------------ the workloads

SMALL_CONFIGS = ["f32_256"]
FULL_CONFIGS = ["f32_4096", "bf16_4096", "f16_4096", "f32_edge", "bf16_edge", "bf16_tail", "bf16_skinny",
                "bf16_attn_qk", "bf16_attn_pv", "bf16_qkv", "bf16_ffn_up", "bf16_ffn_down",
                "bf16_ffn_up_gelu", "bf16_ffn_up_gelu_e4m3", "fp8_4096", "fp8_tail"]


@pytest.mark.parametrize("name", SMALL_CONFIGS)
def test_small_config_every_element(name):
    check(workloads.config(name))


@pytest.mark.parametrize("name", FULL_CONFIGS)
def test_full_config_sampled(name):
    check(workloads.config(name), sample="auto")


@pytest.mark.parametrize("name", ["f32_4096", "bf16_4096", "f16_4096"])
def test_headline_config_every_element(name):
    # the 4096^3 headline problems compared element by element (16.8 M each),
    # on the kernel the benchmark times
    res, _ = check(workloads.config(name))
    assert res.checked == 4096 * 4096
    log(f"{name}: every element checked, max_err={res.max_err:.3e} max_ulp={res.max_ulp} "
        f"strict_fail={res.strict_fail} exempt={res.exempt}")


@pytest.mark.parametrize("name", ["bf16_4096", "bf16_edge", "bf16_attn_pv"])
def test_full_config_fp32_output(name):
    p = workloads.config(name)
    check(p.with_(name=p.name + "-f32out", c_dtype="f32"), sample="auto")


# ------------------------------------------------------------------ fast (direct-load) path

DMA_SHAPES = [(8, 8, 8), (256, 256, 64), (264, 520, 72), (512, 256, 128), (1000, 1032, 1000),
              (24, 4096, 512), (2048, 264, 136)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", DMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_direct_load_path_ragged_aligned(switches, dt, shape, orders):
    # extents multiples of 8 but not of the 256 x 256 x 64 tile: the direct
    # loads' range check and the last-stage k mask produce the edge zeros
    # (few-tile shapes kept off the split-K kernel)
    switches(binding.TEST_NO_SPLITK)
    M, N, K = shape
    oa, ob = orders
    check(P(f"dma-{dt}", dt, M, N, K, alpha=0.5, beta=1.0, order_a=oa, order_b=ob),
          kernel="hgemm_mfma_dma", seed=M + N + K)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_direct_load_path_fp32_out_and_col_major_c(dt):
    check(P(f"dma-f32out-{dt}", dt, 520, 264, 200, c_dtype="f32", beta=-1.0),
          kernel="hgemm_mfma_dma", seed=31)
    check(P(f"dma-colC-{dt}", dt, 520, 264, 200, order_c=COL, beta=0.25),
          kernel="hgemm_mfma_dma", seed=32)


def test_general_kernel_forced_on_aligned_problem(switches):
    # the same aligned problem through the general kernel (register-staged)
    switches(binding.TEST_FORCE_GENERAL)
    check(P("forced-general-bf16", "bf16", 512, 768, 320, beta=1.0), kernel="hgemm_mfma", seed=33)


# ------------------------------------------------------------------ fp32 kernels

F32_DMA_SHAPES = [(4, 4, 4), (128, 128, 16), (132, 260, 20), (260, 132, 1000), (1000, 1028, 1004),
                  (24, 4096, 512), (2048, 132, 68)]


@pytest.mark.parametrize("shape", F32_DMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_f32_direct_load_path_ragged_aligned(switches, shape, orders):
    # extents multiples of 4 but not of the 128 x 128 x 16 tile: the direct
    # loads' range check and the last-stage k mask produce the edge zeros
    # (few-tile shapes kept off the split-K kernel)
    switches(binding.TEST_NO_SPLITK)
    M, N, K = shape
    oa, ob = orders
    check(P("dma-f32", "f32", M, N, K, alpha=0.5, beta=1.0, order_a=oa, order_b=ob),
          kernel="sgemm_mfma_dma", seed=M + N + K)


def test_f32_direct_load_path_batch_and_col_major_c(switches):
    switches(binding.TEST_NO_SPLITK)
    check(P("dma-f32-batch", "f32", 260, 132, 200, beta=-1.0, batch=3), kernel="sgemm_mfma_dma",
          seed=51)
    check(P("dma-f32-colC", "f32", 260, 132, 200, order_c=COL, beta=0.25), kernel="sgemm_mfma_dma",
          seed=52)
    p = P("dma-f32-int", "f32", 264, 136, 4096, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="sgemm_mfma_dma", host=_int_host(p, np.random.default_rng(53)))
    assert res.max_err == 0.0


@pytest.mark.parametrize("env", ["force_general", "f32_valu"])
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_f32_other_kernels_forced_on_aligned_problem(switches, env, orders):
    # the aligned problem the direct-load kernel would take, through the
    # register-staged matrix-core kernel and through the vector-ALU kernel
    switches({"force_general": binding.TEST_FORCE_GENERAL, "f32_valu": binding.TEST_F32_VALU}[env])
    oa, ob = orders
    want = {"force_general": "sgemm_mfma", "f32_valu": "sgemm_valu"}[env]
    check(P(f"forced-{env}", "f32", 520, 392, 300, beta=1.0, order_a=oa, order_b=ob), kernel=want,
          seed=54)


# ------------------------------------------------------------------ vector-ALU fp32 kernel (register tiles)

# The register-tiled vector-ALU kernel (128 x 256 x 16 block tiles, 8 x 16
# outputs per thread) on the shapes, layouts and edges the matrix-core fp32
# kernels are held to; the switch routes every fp32 call to it.
VALU_SHAPES = [(1, 1, 1), (7, 9, 13), (31, 33, 17), (127, 129, 65), (129, 255, 200),
               (255, 257, 63), (300, 290, 130), (513, 130, 77), (33, 70, 1000)]


@pytest.mark.parametrize("shape", VALU_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (COL, COL)], ids=lambda o: "%d%d" % o)
def test_valu_kernel_shapes(switches, shape, orders):
    switches(binding.TEST_F32_VALU)
    M, N, K = shape
    oa, ob = orders
    check(P("valu", "f32", M, N, K, alpha=0.75, beta=0.5, order_a=oa, order_b=ob),
          kernel="sgemm_valu", seed=M + N + K + 11)


def test_valu_kernel_misaligned_batches_col_major_c_and_integers(switches):
    switches(binding.TEST_F32_VALU)
    check(P("valu-misaligned", "f32", 190, 211, 97, beta=1.0, lda=99, ldb=213, ldc=215),
          kernel="sgemm_valu", seed=120, base_offset=(1, 3, 1))
    for bcast in ("none", "a", "b"):
        kw = {"stride_a": 0} if bcast == "a" else {"stride_b": 0} if bcast == "b" else {}
        check(P(f"valu-batch-{bcast}", "f32", 130, 260, 90, batch=3, beta=1.0,
                stride_c=130 * 260 + 17, **kw), kernel="sgemm_valu", seed=121)
    check(P("valu-colC", "f32", 300, 290, 130, order_c=COL, ldc=303, beta=0.5),
          kernel="sgemm_valu", seed=122)
    p = P("valu-int", "f32", 300, 517, 260, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="sgemm_valu", host=_int_host(p, np.random.default_rng(123)))
    assert res.max_err == 0.0


@pytest.mark.parametrize("name", ["f32_4096", "f32_edge"])
def test_valu_kernel_full_configs_sampled(switches, name):
    switches(binding.TEST_F32_VALU)
    check(workloads.config(name), kernel="sgemm_valu", sample="auto")


def test_valu_entry_point():
    # gemm_f32_valu itself, without the switch, on the 4096^3 headline problem
    p = workloads.config("f32_4096_valu")
    res, _ = check(p, sample="auto")
    assert res.ok


# ------------------------------------------------------------------ skinny path (at most 16 rows of C)

SKINNY_SHAPES = [(1, 520, 256), (5, 4096, 1000), (16, 4096, 4096), (16, 16, 8200), (11, 264, 2056)]


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("shape", SKINNY_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ob", [ROW, COL], ids=["Brow", "Bcol"])
def test_skinny_path(dt, shape, ob):
    # M <= 16 with a row-major A: B streamed through LDS in 16-column blocks,
    # K split eight ways (slices ragged against K, rows past M zero); fp32
    # takes this path only with a K-contiguous B (else split-K)
    M, N, K = shape
    want = "sgemm_splitk" if (dt == "f32" and ob == ROW) else "gemm_skinny"
    check(P(f"skinny-{dt}", dt, M, N, K, alpha=0.75, beta=-0.5, order_b=ob), kernel=want,
          seed=M + 7 * N + K, sample="auto" if M * N * K > 100_000_000 else None)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_skinny_fp32_output_and_batch(dt):
    check(P(f"skinny-f32out-{dt}", dt, 16, 520, 2048, c_dtype="f32", beta=1.0, batch=3),
          kernel="gemm_skinny", seed=71)


@pytest.mark.parametrize("dt", DT)
def test_skinny_column_major_c_and_integers(dt):
    # column-major C with 12 columns is computed as the 12-row C^T = B^T A^T,
    # which is skinny when B is column-major (A^T of the swapped problem is
    # then K-contiguous)
    # (the swapped problem's B is A^T, K-contiguous since A is row-major, so
    # fp32 takes the skinny kernel here too)
    check(P(f"skinny-colC-{dt}", dt, 520, 12, 2048, order_b=COL, order_c=COL, beta=0.5),
          kernel="gemm_skinny", seed=72)
    p = P(f"skinny-int-{dt}", dt, 16, 264, 4096, alpha=2.0, beta=1.0,
          order_b=COL if dt == "f32" else ROW)
    res, _ = check(p, kernel="gemm_skinny", host=_int_host(p, np.random.default_rng(73)))
    assert res.max_err == 0.0


# ------------------------------------------------------------------ fused epilogue (bias, activation)

RELU, GELU = 1, 2
EPI_CASES = [
    # (input type, output type, M, N, K, extra problem fields, kernel)
    ("f32", "f32", 520, 264, 200, {}, "sgemm_mfma_dma"),
    ("f32", "f32", 190, 211, 97, {}, "sgemm_mfma"),
    ("f32", "f32", 64, 136, 512, {}, "sgemm_splitk"),
    ("f32", "f32", 8, 136, 512, dict(order_b=COL), "gemm_skinny"),
    ("bf16", "bf16", 520, 264, 200, {}, "hgemm_mfma_dma"),
    ("bf16", "f32", 520, 264, 200, {}, "hgemm_mfma_dma"),
    ("f16", "f16", 520, 264, 200, dict(order_a=COL, order_b=COL), "hgemm_mfma_dma"),
    ("bf16", "bf16", 190, 211, 97, {}, "hgemm_mfma"),
    ("bf16", "bf16", 64, 136, 1024, {}, "hgemm_splitk"),
    ("f16", "f32", 8, 136, 512, {}, "gemm_skinny"),
]


@pytest.mark.parametrize("case", EPI_CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[6]}")
@pytest.mark.parametrize("act", [0, RELU, GELU], ids=["bias", "bias-relu", "bias-gelu"])
def test_fused_bias_and_activation(case, act):
    dt, ct, M, N, K, extra, kernel = case
    check(P(f"epi-{dt}-{kernel}-{act}", dt, M, N, K, c_dtype=ct, alpha=0.75, beta=0.5,
            bias=True, act=act, **extra), kernel=kernel, seed=M + N + act)


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("act", [RELU, GELU], ids=["relu", "gelu"])
def test_fused_activation_without_bias(dt, act):
    check(P(f"epi-nobias-{dt}", dt, 264, 520, 136, act=act), seed=81 + act)


@pytest.mark.parametrize("dt", DT)
def test_fused_epilogue_col_major_c_and_batches(dt):
    # column-major C: the library computes C^T, where the bias runs along rows
    check(P(f"epi-colC-{dt}", dt, 520, 264, 200, order_c=COL, beta=0.5, bias=True, act=RELU),
          seed=82)
    # one bias vector per batch entry, and one shared by all
    check(P(f"epi-batch-{dt}", dt, 264, 136, 200, batch=3, bias=True, act=GELU), seed=83)
    check(P(f"epi-batch-shared-{dt}", dt, 264, 136, 200, batch=3, bias=True, stride_bias=0,
            act=GELU), seed=84)


@pytest.mark.parametrize("dt", DT)
def test_fused_epilogue_without_product_term(dt):
    # alpha == 0 and K == 0: C <- act(beta*C + bias), A and B not read
    check(P(f"epi-alpha0-{dt}", dt, 130, 70, 40, alpha=0.0, beta=0.5, bias=True, act=RELU),
          kernel="scale", seed=85)
    check(P(f"epi-k0-{dt}", dt, 130, 70, 0, beta=-1.5, bias=True, act=GELU), kernel="scale",
          seed=86)


def test_fused_epilogue_on_vector_alu_kernel(switches):
    switches(binding.TEST_F32_VALU)
    check(P("epi-valu", "f32", 520, 264, 200, beta=0.5, bias=True, act=GELU),
          kernel="sgemm_valu", seed=87)


@pytest.mark.parametrize("dt", DT)
def test_fused_relu_bias_integers_bit_exact(dt):
    # integer data and an integer bias: every step is exact, and so is ReLU
    p = P(f"epi-int-{dt}", dt, 264, 136, 200, alpha=2.0, beta=1.0, bias=True, act=RELU)
    rng = np.random.default_rng(88)
    bias = rng.integers(-200, 201, p.N).astype(np.float32)
    bias = bias if dt == "f32" else workloads.to_16bit(bias, dt)
    res, _ = check(p, kernel="sgemm_mfma_dma" if dt == "f32" else "hgemm_mfma_dma",
                   host=_int_host(p, rng), bias_host=bias)
    assert res.max_err == 0.0 and res.max_ulp == 0


# ------------------------------------------------------------------ split-K path (few tiles, long K)

F32_SPLITK_SHAPES = [(256, 256, 256), (32, 4096, 4096), (24, 8, 4096), (40, 1000, 1736),
                     (260, 132, 512), (24, 520, 300), (1000, 1028, 1004)]


@pytest.mark.parametrize("shape", F32_SPLITK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_f32_splitk_path(shape, orders):
    # under 128 tiles of 128 x 128 and K >= 256: the workgroup splits K eight
    # ways (slices ragged against K where 8*32 does not divide it)
    M, N, K = shape
    oa, ob = orders
    big = M * N * K > 100_000_000
    check(P("splitk-f32", "f32", M, N, K, alpha=0.75, beta=-0.5, order_a=oa, order_b=ob),
          kernel="sgemm_splitk", seed=M + 5 * N + K, sample="auto" if big else None)


def test_f32_splitk_batch_col_major_c_and_integers():
    check(P("splitk-f32-batch", "f32", 24, 520, 2048, beta=1.0, batch=3), kernel="sgemm_splitk",
          seed=61)
    check(P("splitk-f32-colC", "f32", 520, 24, 2048, order_c=COL, beta=0.5), kernel="sgemm_splitk",
          seed=62)
    # integer inputs: the fixed-order reduction of the slices is exact
    p = P("splitk-f32-int", "f32", 24, 264, 4096, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="sgemm_splitk", host=_int_host(p, np.random.default_rng(63)))
    assert res.max_err == 0.0


SPLITK_SHAPES = [(32, 4096, 4096), (24, 8, 4096), (40, 1000, 1736), (256, 256, 8192), (24, 520, 512)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SPLITK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_splitk_path(dt, shape, orders):
    # under 64 tiles of 256 x 256 and K >= 512: the workgroup splits K eight
    # ways (slices ragged against K where 8*64 does not divide it)
    M, N, K = shape
    oa, ob = orders
    big = M * N * K > 100_000_000
    check(P(f"splitk-{dt}", dt, M, N, K, alpha=0.75, beta=-0.5, order_a=oa, order_b=ob),
          kernel="hgemm_splitk", seed=M + 3 * N + K, sample="auto" if big else None)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_splitk_fp32_output_batch_and_col_major_c(dt):
    check(P(f"splitk-f32out-{dt}", dt, 24, 520, 2048, c_dtype="f32", beta=1.0, batch=3),
          kernel="hgemm_splitk", seed=41)
    check(P(f"splitk-colC-{dt}", dt, 520, 24, 2048, order_c=COL, beta=0.5), kernel="hgemm_splitk",
          seed=42)
    # integer inputs: every partial sum exact in fp32, so the fixed-order
    # reduction of the eight slices must reproduce the oracle bit for bit
    p = P(f"splitk-int-{dt}", dt, 24, 264, 4096, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="hgemm_splitk", host=_int_host(p, np.random.default_rng(43)))
    assert res.max_err == 0.0 and res.max_ulp == 0


# ------------------------------------------------------------------ 8-bit float inputs

F8_PAIRS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]
TN = dict(order_a=ROW, order_b=COL)  # both operands contiguous along K


def F8(name, fa, fb, out, M, N, K, **kw):
    return Problem(name, fa, out, M, N, K, b_dtype=fb, **kw)


def f8_kernel(oa, ob, K):
    # operands with default (tight) leading dimensions and 16-byte aligned
    # buffers: the direct-load kernel needs K-contiguous A and B and K a
    # multiple of 16
    return "f8gemm_mfma_dma" if (oa, ob) == (ROW, COL) and K % 16 == 0 else "f8gemm_mfma"


@pytest.mark.parametrize("pair", F8_PAIRS, ids="-".join)
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_f8_direct_load_formats_and_outputs(pair, out):
    fa, fb = pair
    check(F8(f"f8dma-{fa}-{fb}-{out}", fa, fb, out, 300, 264, 208, alpha=0.75, beta=-0.5, **TN),
          kernel="f8gemm_mfma_dma", seed=60)


F8_DMA_SHAPES = [(1, 1, 16), (16, 16, 16), (256, 256, 128), (264, 520, 144), (513, 257, 400),
                 (1000, 1032, 1008), (24, 4096, 512), (2048, 264, 2064)]


@pytest.mark.parametrize("shape", F8_DMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f8_direct_load_ragged(shape):
    # extents that are not multiples of the 256 x 256 x 128 tile: the direct
    # loads' range check and the last-stage k mask produce the edge zeros
    M, N, K = shape
    check(F8("f8dma-ragged", "e4m3", "e5m2", "bf16", M, N, K, beta=1.0, **TN),
          kernel="f8gemm_mfma_dma", seed=M + N + K)


F8_GENERAL_SHAPES = [(1, 1, 1), (7, 9, 13), (129, 127, 200), (264, 512, 144), (300, 290, 333),
                     (513, 130, 77)]


@pytest.mark.parametrize("pair", [("e4m3", "e4m3"), ("e5m2", "e4m3")], ids="-".join)
@pytest.mark.parametrize("shape", F8_GENERAL_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_f8_every_layout(pair, shape, orders):
    M, N, K = shape
    oa, ob = orders
    fa, fb = pair
    check(F8(f"f8-layout-{fa}-{fb}", fa, fb, "bf16", M, N, K, alpha=1.25, beta=0.5, order_a=oa,
             order_b=ob), kernel=f8_kernel(oa, ob, K), seed=M * 3 + N + K)


@pytest.mark.parametrize("orders", [(a, b, c) for a in (ROW, COL) for b in (ROW, COL)
                                    for c in (ROW, COL)], ids=lambda o: "%d%d%d" % o)
def test_f8_padded_ld_and_misaligned_bases(orders):
    oa, ob, oc = orders
    M, N, K = 261, 199, 150
    lda = (K if oa == ROW else M) + 13
    ldb = (N if ob == ROW else K) + 8
    ldc = (N if oc == ROW else M) + 5
    p = F8("f8-padded", "e4m3", "e5m2", "f32", M, N, K, alpha=1.25, beta=0.5, order_a=oa,
           order_b=ob, order_c=oc, lda=lda, ldb=ldb, ldc=ldc)
    check(p, kernel="f8gemm_mfma", seed=63)
    check(p.with_(name="f8-misaligned"), kernel="f8gemm_mfma", seed=64, base_offset=(1, 3, 1))


def test_f8_general_kernel_forced_on_aligned_problem(switches):
    switches(binding.TEST_FORCE_GENERAL)
    check(F8("f8-forced", "e5m2", "e4m3", "f16", 1000, 1032, 1008, beta=1.0, **TN),
          kernel="f8gemm_mfma", seed=65)


@pytest.mark.parametrize("kernel", ["f8gemm_mfma_dma", "f8gemm_mfma"])
def test_f8_batches_and_col_major_c(switches, kernel):
    if kernel == "f8gemm_mfma":
        switches(binding.TEST_FORCE_GENERAL)
    M, N, K = 130, 264, 96
    check(F8("f8-batch", "e4m3", "e5m2", "f32", M, N, K, batch=3, beta=1.0,
             stride_c=M * N + 17, **TN), kernel=kernel, seed=66)
    check(F8("f8-batch-shared-b", "e4m3", "e4m3", "bf16", M, N, K, batch=3, stride_b=0, **TN),
          kernel=kernel, seed=67)
    check(F8("f8-colC", "e5m2", "e4m3", "bf16", 520, 24, 512, order_c=COL, beta=0.5, **TN),
          kernel=kernel, seed=68)


def _int_host_f8(p, rng):
    # integers in [-8, 8] are exact in both 8-bit formats
    def mk(n, dt):
        v = rng.integers(-8, 9, n).astype(np.float32)
        return workloads.to_8bit(v, dt)
    c = rng.integers(-4, 5, p.buffer_elems("c")).astype(np.float32)
    c = c if p.c_dtype == "f32" else workloads.to_16bit(c, p.c_dtype)
    return mk(p.buffer_elems("a"), p.in_dtype), mk(p.buffer_elems("b"), p.b_dtype), c


@pytest.mark.parametrize("pair", F8_PAIRS, ids="-".join)
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("orders", [(ROW, COL), (ROW, ROW)], ids=["TN", "NN"])
def test_f8_integer_inputs_bit_exact(pair, out, orders):
    # products of small integers and their partial sums are exact in fp32,
    # so both kernels must reproduce the oracle's correctly rounded result
    fa, fb = pair
    oa, ob = orders
    p = F8(f"f8-int-{fa}-{fb}-{out}", fa, fb, out, 264, 520, 512, alpha=2.0, beta=1.0,
           order_a=oa, order_b=ob)
    res, _ = check(p, kernel=f8_kernel(oa, ob, p.K), host=_int_host_f8(p, np.random.default_rng(69)))
    assert res.max_err == 0.0 and res.max_ulp == 0


def test_f8_beta_zero_ignores_nan_in_c_and_scale_only_paths():
    check(F8("f8-beta0nan", "e4m3", "e4m3", "bf16", 140, 150, 64, **TN),
          kernel="f8gemm_mfma_dma", seed=70, c_init=0x7FC0)
    check(F8("f8-alpha0", "e4m3", "e5m2", "f32", 77, 65, 32, alpha=0.0, beta=-2.0, **TN),
          kernel="scale", seed=71)
    check(F8("f8-k0", "e5m2", "e5m2", "f16", 77, 65, 0, alpha=1.5, beta=0.5),
          kernel="scale", seed=72)


def test_f8_repeat_runs_bit_identical():
    check(F8("f8-determinism", "e4m3", "e4m3", "bf16", 520, 700, 304, beta=0.5, **TN),
          kernel="f8gemm_mfma_dma", seed=73, repeat=3)


@pytest.mark.parametrize("kernel", ["f8gemm_mfma_dma", "f8gemm_mfma"])
def test_f8_nan_and_infinity_propagate(switches, kernel):
    # A NaN in A makes its row of C NaN; an E5M2 infinity at A(i, k) makes
    # C(i, j) an infinity of the sign of B(k, j), or NaN where B(k, j) == 0.
    if kernel == "f8gemm_mfma":
        switches(binding.TEST_FORCE_GENERAL)
    M, N, K = 64, 72, 96
    p = F8("f8-special", "e5m2", "e5m2", "f32", M, N, K, **TN)
    a, b, c = workloads.generate(p, seed=74)
    a = a.copy()
    a[3 * K + 5] = 0x7F              # NaN at A(3, 5)
    a[10 * K + 7] = 0x7C             # +inf at A(10, 7)
    b = b.copy()
    b[np.arange(0, N, 9) * K + 7] = 0  # zeros in row 7 of B every ninth column
    from parity import GUARD, run as raw_run
    res, out = raw_run(p, host=(a, b, c))
    assert res.kernel == kernel
    got = out[GUARD:GUARD + M * N].view(np.float32).reshape(M, N)
    assert np.all(np.isnan(got[3]))
    bk = oracle.decode("e5m2", b.reshape(N, K)[:, 7])
    want10 = np.where(bk > 0, np.inf, np.where(bk < 0, -np.inf, np.nan))
    assert np.array_equal(np.isnan(got[10]), np.isnan(want10))
    fin = ~np.isnan(want10)
    assert np.array_equal(got[10][fin], want10[fin])
    rest = np.ones(M, bool)
    rest[[3, 10]] = False
    assert np.all(np.isfinite(got[rest]))


def test_f8_full_size_fp32_output():
    p = workloads.config("fp8_4096")
    check(p.with_(name=p.name + "-f32out", c_dtype="f32", b_dtype="e5m2"), sample="auto",
          kernel="f8gemm_mfma_dma")


def test_f8_truncation_worst_case_within_bound():
    # The construction that makes the instruction's truncation largest: in
    # every group of 8 consecutive k one product is 1 and the other seven
    # are 0.875 * 2^-13, just under the 2^-13 cut-off, all of one sign, so
    # each is dropped whole and the errors add up: 6.1 * 2^-13 = 7.5e-4 of
    # den per element.  The result must stay within the 1e-3 * den bound.
    M, N, K = 64, 72, 256
    p = F8("f8-truncation", "e4m3", "e5m2", "f32", M, N, K, **TN)
    rng = np.random.default_rng(75)
    a = np.full((M, K), 0.875 * 2.0 ** -6)             # 7/8 * 2^-6: an E4M3 subnormal
    a[:, ::8] = 1.0
    sign = rng.choice([-1.0, 1.0], (M, K // 8))         # one sign per group
    sign[0] = 1.0
    a *= np.repeat(sign, 8, axis=1)
    b = np.full((N, K), 2.0 ** -7)                       # B stored column-major: N rows of K
    b[:, ::8] = 1.0
    host = (workloads.to_8bit(a.astype(np.float32).ravel(), "e4m3"),
            workloads.to_8bit(b.astype(np.float32).ravel(), "e5m2"), np.zeros(M * N, np.float32))
    res, _ = check(p, kernel="f8gemm_mfma_dma", host=host)
    log(f"f8 truncation worst case: max normalised error {res.max_err:.3e}")


# ------------------------------------------------------------------ stream-K schedule (workspace entry points)

# Shapes on the general kernel (leading dimensions not multiples of 8
# elements) whose tiles do not fill whole waves of 256 workgroups: few tiles
# with a long K, every tile cut across many workgroups.
SK_SHAPES = [(300, 290, 8193), (513, 770, 3001), (1000, 1030, 1701)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_streamk_general_kernel(dt, shape, orders):
    M, N, K = shape
    oa, ob = orders
    check(P(f"streamk-{dt}", dt, M, N, K, alpha=0.75, beta=0.5, order_a=oa, order_b=ob),
          kernel="hgemm_mfma_streamk", seed=M + K, use_workspace=True, repeat=2)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_streamk_fp32_output_batch_and_col_major_c(dt):
    check(P(f"streamk-f32out-{dt}", dt, 300, 290, 4099, c_dtype="f32", beta=1.0, batch=3),
          kernel="hgemm_mfma_streamk", seed=80, use_workspace=True)
    check(P(f"streamk-colC-{dt}", dt, 290, 300, 8197, order_c=COL, ldc=293, beta=0.5),
          kernel="hgemm_mfma_streamk", seed=81, use_workspace=True)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_streamk_integers_bit_exact(dt):
    # every partial sum of small integers is exact in fp32, so the fixed-order
    # fix-up must reproduce the oracle bit for bit
    p = P(f"streamk-int-{dt}", dt, 513, 770, 3001, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="hgemm_mfma_streamk", host=_int_host(p, np.random.default_rng(82)),
                   use_workspace=True)
    assert res.max_err == 0.0 and res.max_ulp == 0


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_streamk_whole_waves_and_cut_tail(dt):
    # 65 batches of 2 x 2 tiles: 256 tiles computed whole, 4 cut over the
    # grid; beta = 0.5, so the fix-up also reads C.  K = 3001 makes the
    # aligned copies (233 MB) larger than the workspace, so the general
    # kernel runs on the caller's operands.
    check(P(f"streamk-dp-{dt}", dt, 300, 290, 3001, beta=0.5, batch=65),
          kernel="hgemm_mfma_streamk", seed=84, use_workspace=True, repeat=2)


# The direct-load kernel's stream-K schedule: aligned operands (extents and
# leading dimensions multiples of 8 elements) and at least 64 tiles (fewer
# go to the split-K kernel).  Its cost model only picks it for large
# problems with a short cut wave (the bf16_tail workload below), so these
# small cases switch the model off (the GEMM_TEST_FORCE_STREAMK switch).
DMA_SK_SHAPES = [(2048, 2304, 1024), (2304, 2048, 1536)]


@pytest.fixture
def force_streamk(switches):
    switches(binding.TEST_FORCE_STREAMK)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", DMA_SK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_dma_streamk(dt, shape, orders, force_streamk):
    M, N, K = shape
    oa, ob = orders
    check(P(f"dma-streamk-{dt}", dt, M, N, K, alpha=0.75, beta=0.5, order_a=oa, order_b=ob),
          kernel="hgemm_mfma_dma_streamk", seed=M + N + K, use_workspace=True, repeat=2)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_dma_streamk_whole_waves_fp32_output_and_col_major_c(dt, force_streamk):
    # 65 batches of 2 x 2 tiles: 256 whole, 4 cut over the grid
    check(P(f"dma-streamk-dp-{dt}", dt, 512, 512, 2048, beta=0.5, batch=65),
          kernel="hgemm_mfma_dma_streamk", seed=90, use_workspace=True, repeat=2)
    check(P(f"dma-streamk-f32out-{dt}", dt, 512, 768, 2048, c_dtype="f32", beta=1.0, batch=12),
          kernel="hgemm_mfma_dma_streamk", seed=91, use_workspace=True)
    check(P(f"dma-streamk-colC-{dt}", dt, 2304, 2048, 1024, order_c=COL, beta=0.5),
          kernel="hgemm_mfma_dma_streamk", seed=92, use_workspace=True)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_dma_streamk_integers_bit_exact(dt, force_streamk):
    p = P(f"dma-streamk-int-{dt}", dt, 2048, 2304, 1024, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="hgemm_mfma_dma_streamk", host=_int_host(p, np.random.default_rng(93)),
                   use_workspace=True)
    assert res.max_err == 0.0 and res.max_ulp == 0


def test_dma_streamk_tail_config_sampled():
    # aligned 4096 x 4352 x 4096: 272 tiles on 256 compute units
    check(workloads.config("bf16_tail"), kernel="hgemm_mfma_dma_streamk", sample="auto",
          use_workspace=True, repeat=2)


# The general fp32 kernel's stream-K schedule (128 x 128 tiles, four
# workgroups per compute unit).
F32_SK_SHAPES = [(300, 290, 8193), (1000, 1030, 2001)]


@pytest.mark.parametrize("shape", F32_SK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_f32_streamk(shape, orders):
    M, N, K = shape
    oa, ob = orders
    check(P("f32-streamk", "f32", M, N, K, alpha=0.75, beta=0.5, order_a=oa, order_b=ob),
          kernel="sgemm_mfma_streamk", seed=M + K + 7, use_workspace=True, repeat=2)


def test_f32_streamk_whole_waves_batches_and_col_major_c():
    # 114 batches of 3 x 3 tiles: 1024 whole, 2 cut over the grid
    check(P("f32-streamk-dp", "f32", 300, 290, 1001, beta=0.5, batch=114),
          kernel="sgemm_mfma_streamk", seed=94, use_workspace=True, repeat=2)
    check(P("f32-streamk-colC", "f32", 1030, 1000, 2001, order_c=COL, ldc=1033, beta=0.5),
          kernel="sgemm_mfma_streamk", seed=95, use_workspace=True)


def test_f32_streamk_integers_bit_exact():
    p = P("f32-streamk-int", "f32", 1000, 1030, 2001, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="sgemm_mfma_streamk", host=_int_host(p, np.random.default_rng(96)),
                   use_workspace=True)
    assert res.max_err == 0.0


def test_f32_packed_edge_config_sampled():
    # the unaligned 4095 x 4097 x 1001 fp32 problem with a workspace: copied
    # to aligned operands, then the direct-load kernel on 4095 x 4096 (1024
    # tiles, whole waves) and the one remaining column on the split-K kernel
    check(workloads.config("f32_edge"), kernel="sgemm_mfma_dma_packed", sample="auto",
          use_workspace=True, repeat=2)


def test_streamk_workspace_too_small_is_the_plain_call():
    p = P("streamk-small-ws", "bf16", 513, 770, 3001, beta=0.5)
    host = workloads.generate(p, seed=83)
    _, plain = check(p, kernel="hgemm_mfma", host=host)
    _, small = check(p, kernel="hgemm_mfma", host=host, use_workspace=True,
                     workspace_bytes=1 << 20)
    assert np.array_equal(plain, small)


def test_packed_edge_config_sampled():
    # the unaligned 4095 x 4097 x 1001 problem with a workspace: copied to
    # aligned, zero-padded operands, then the direct-load kernel
    check(workloads.config("bf16_edge"), kernel="hgemm_mfma_dma_packed", sample="auto",
          use_workspace=True, repeat=2)


# ------------------------------------------------------------------ packed operands (workspace entry points)

# Problems with unaligned operands and enough tiles for the direct-load
# kernels: the workspace entry points copy A and B into zero-padded aligned
# buffers first.  Extents and leading dimensions are odd, so every operand
# row starts at a different alignment, and K is padded (1001 -> 1008).
PACK_SHAPES = [(2047, 2049, 1001), (2305, 1999, 515)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", PACK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_packed_16bit(dt, shape, orders):
    M, N, K = shape
    oa, ob = orders
    check(P(f"packed-{dt}", dt, M, N, K, alpha=0.75, beta=0.5, order_a=oa, order_b=ob),
          kernel="hgemm_mfma_dma_packed", seed=M + N + K + 3, use_workspace=True, repeat=2)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("orders", [(ROW, ROW), (COL, COL)], ids=lambda o: "%d%d" % o)
def test_packed_16bit_padded_ld_and_misaligned_bases(dt, orders):
    # aligned extents but padded odd leading dimensions, then misaligned base
    # pointers with leading dimensions that are multiples of 8
    oa, ob = orders
    M, N, K = 2048, 2304, 1024
    lda = (K if oa == ROW else M) + 3
    ldb = (N if ob == ROW else K) + 5
    check(P(f"packed-ld-{dt}", dt, M, N, K, beta=0.5, order_a=oa, order_b=ob, lda=lda, ldb=ldb,
            ldc=N + 7), kernel="hgemm_mfma_dma_packed", seed=101, use_workspace=True)
    check(P(f"packed-base-{dt}", dt, M, N, K, alpha=-1.5, order_a=oa, order_b=ob),
          kernel="hgemm_mfma_dma_packed", seed=102, use_workspace=True, base_offset=(1, 3, 1))


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_packed_16bit_batches_fp32_output_and_col_major_c(dt):
    # 65 batches of 2 x 2 tiles: copied, then the direct-load stream-K
    # schedule (256 tiles whole, 4 cut); a batch sharing one B (stride 0);
    # fp32 output; a column-major C (computed as C^T = B^T A^T)
    check(P(f"packed-batch-{dt}", dt, 300, 290, 1001, beta=0.5, batch=65),
          kernel="hgemm_mfma_dma_streamk_packed", seed=103, use_workspace=True, repeat=2)
    check(P(f"packed-shared-b-{dt}", dt, 1025, 777, 333, batch=9, stride_b=0),
          kernel="hgemm_mfma_dma_packed", seed=104, use_workspace=True)
    check(P(f"packed-f32out-{dt}", dt, 2047, 2049, 1001, c_dtype="f32", beta=1.0),
          kernel="hgemm_mfma_dma_packed", seed=105, use_workspace=True)
    check(P(f"packed-colC-{dt}", dt, 2049, 2047, 1001, order_c=COL, ldc=2051, beta=0.5),
          kernel="hgemm_mfma_dma_packed", seed=106, use_workspace=True)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_packed_16bit_integers_bit_exact(dt):
    p = P(f"packed-int-{dt}", dt, 2047, 2049, 1001, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="hgemm_mfma_dma_packed", host=_int_host(p, np.random.default_rng(107)),
                   use_workspace=True)
    assert res.max_err == 0.0 and res.max_ulp == 0


def test_packed_16bit_forced_streamk(force_streamk):
    # every tile of a 72-tile problem cut across the grid, on the copies
    p = P("packed-sk-bf16", "bf16", 2047, 2049, 1001, alpha=0.75, beta=0.5, order_b=COL)
    check(p, kernel="hgemm_mfma_dma_streamk_packed", seed=108, use_workspace=True, repeat=2)
    res, _ = check(p, kernel="hgemm_mfma_dma_streamk_packed",
                   host=_int_host(p, np.random.default_rng(109)), use_workspace=True)
    assert res.max_ulp == 0


# (shape, kernel): 182 tiles of 17 k steps are cut over the grid by the
# direct-load stream-K schedule; 187 tiles of 63 steps would need more
# partial tiles than the workspace holds beside the copies, so they run on
# the plain direct-load kernel.
F32_PACK_SHAPES = [((1537, 1665, 257), "sgemm_mfma_dma_streamk_packed"),
                   ((2049, 1283, 1001), "sgemm_mfma_dma_packed")]


@pytest.mark.parametrize("shape,kernel", F32_PACK_SHAPES, ids=lambda s: "x".join(map(str, s))
                         if isinstance(s, tuple) else s.rsplit("_", 1)[-1])
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_packed_f32(shape, kernel, orders):
    M, N, K = shape
    oa, ob = orders
    check(P("packed-f32", "f32", M, N, K, alpha=0.75, beta=0.5, order_a=oa, order_b=ob),
          kernel=kernel, seed=M + N + K + 5, use_workspace=True, repeat=2)


def test_packed_f32_bases_batch_col_major_c_and_integers():
    check(P("packed-f32-base", "f32", 1664, 1664, 256, beta=0.5),
          kernel="sgemm_mfma_dma_streamk_packed", seed=110, use_workspace=True,
          base_offset=(1, 2, 0))
    check(P("packed-f32-batch", "f32", 515, 517, 203, batch=8, beta=1.0),
          kernel="sgemm_mfma_dma_streamk_packed", seed=111, use_workspace=True)
    check(P("packed-f32-colC", "f32", 1665, 1537, 257, order_c=COL, ldc=1669, beta=0.5),
          kernel="sgemm_mfma_dma_streamk_packed", seed=112, use_workspace=True)
    p = P("packed-f32-int", "f32", 1537, 1665, 257, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="sgemm_mfma_dma_streamk_packed",
                   host=_int_host(p, np.random.default_rng(113)), use_workspace=True)
    assert res.max_err == 0.0


# The fp32 direct-load kernel's stream-K schedule on aligned operands: 272
# tiles, all cut over the grid, and 1056 tiles (1024 whole, 32 cut).
F32_DMA_SK_SHAPES = [(2048, 2176, 1000), (4096, 4224, 256)]


@pytest.mark.parametrize("shape", F32_DMA_SK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=lambda o: "%d%d" % o)
def test_f32_dma_streamk(shape, orders):
    M, N, K = shape
    oa, ob = orders
    check(P("f32-dma-streamk", "f32", M, N, K, alpha=0.75, beta=0.5, order_a=oa, order_b=ob),
          kernel="sgemm_mfma_dma_streamk", seed=M + K + 11, use_workspace=True, repeat=2)


def test_f32_dma_streamk_batches_col_major_c_and_integers():
    # 114 batches of 3 x 3 tiles (1026 tiles: 1024 whole, 2 cut); a
    # column-major C with a padded leading dimension; integer-valued inputs,
    # exact in fp32
    check(P("f32-dma-sk-dp", "f32", 384, 384, 1000, beta=0.5, batch=114),
          kernel="sgemm_mfma_dma_streamk", seed=114, use_workspace=True, repeat=2)
    check(P("f32-dma-sk-colC", "f32", 2048, 2176, 1000, order_c=COL, ldc=2051, beta=-1.0),
          kernel="sgemm_mfma_dma_streamk", seed=115, use_workspace=True)
    p = P("f32-dma-sk-int", "f32", 2048, 2176, 1000, alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="sgemm_mfma_dma_streamk", host=_int_host(p, np.random.default_rng(117)),
                   use_workspace=True)
    assert res.max_err == 0.0


# ------------------------------------------------------------------ block-scaled (MX) inputs

from parity import mx_int_patterns, run_mx  # noqa: E402

MX_PAIRS = [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e2m3", "e2m3"), ("e3m2", "e2m3"),
            ("e2m1", "e2m1")]


def check_mx(p, kernel="mxgemm_mfma_dma", **kw):
    res, out = run_mx(p, **kw)
    assert res.ok, res.why
    assert res.kernel == kernel, f"{p.name} ran on {res.kernel!r}"
    return res, out


@pytest.mark.parametrize("fa,fb", MX_PAIRS, ids=lambda f: f)
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 260, 320), (64, 96, 64), (513, 257, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mx_formats_and_shapes(fa, fb, out, shape):
    # K = 320 leaves a last stage of 64 k (its scale padding bytes are NaN
    # patterns the kernel must not use); ragged M and N cut the edge tiles
    M, N, K = shape
    check_mx(workloads.MxProblem(f"mx-{fa}-{fb}", fa, fb, out, M, N, K, alpha=0.5, beta=1.0),
             seed=M + K, repeat=2)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e5m2"), ("e3m2", "e3m2"), ("e2m1", "e2m1")],
                         ids=lambda f: f)
def test_mx_layouts_batches_and_col_major_c(fa, fb):
    # padded leading dimensions of the operands and of the scales; fp16
    # output where the elements stay small (8-bit elements with scales up to
    # 2^4 reach past fp16's range)
    out = "bf16" if workloads.MX_WIDTH[fa] == 8 else "f16"
    check_mx(workloads.MxProblem("mx-ld", fa, fb, out, 260, 300, 256, lda=384, ldb=320, ldsa=16,
                                 ldsb=12, beta=-0.5), seed=3)
    # column-major C (computed as C^T = B^T A^T, operands and scales swapped)
    check_mx(workloads.MxProblem("mx-colC", fa, fb, "bf16", 300, 200, 192, order_c=COL, ldc=303,
                                 beta=2.0), seed=4)
    # a batch with one shared B (and shared B scales), per-entry A scales
    check_mx(workloads.MxProblem("mx-batch", fa, fb, "f32", 130, 140, 128, batch=3, stride_b=0,
                                 stride_sb=0, beta=1.0), seed=5)


@pytest.mark.parametrize("fa,fb", MX_PAIRS, ids=lambda f: f)
def test_mx_integers_bit_exact(fa, fb):
    # small integers with scales 2^-1 .. 2^1: every product and partial sum
    # is exact, and so is alpha = 2 (beta = 0: a random C0 would add one
    # fp32 rounding), so the fp32 result must equal the oracle bit for bit
    M, N, K, batch = 200, 230, 384, 2
    rng = np.random.default_rng(17)
    pats = (mx_int_patterns(rng, fa, batch, M, K), mx_int_patterns(rng, fb, batch, N, K))
    p = workloads.MxProblem("mx-int", fa, fb, "f32", M, N, K, alpha=2.0, beta=0.0, batch=batch,
                            scale_lo=126, scale_hi=128)
    res, _ = check_mx(p, seed=18, patterns=pats)
    assert res.max_err == 0.0


def test_mx_alpha_zero_and_k_zero_scale_c():
    p = workloads.MxProblem("mx-alpha0", "e2m1", "e2m1", "bf16", 100, 70, 128, alpha=0.0,
                            beta=0.5)
    res, _ = run_mx(p, seed=6)
    assert res.ok and res.kernel == "scale", res.why


@pytest.mark.parametrize("name", ["mxfp4_4096", "mxfp6_4096", "mxfp8_4096"])
def test_mx_full_size_sampled(name):
    check_mx(workloads.config(name), sample="auto")


# ------------------------------------------------------------------ 8-bit and MX stream-K (workspace)

# The narrow-float direct-load kernel's stream-K schedule (256 x 256 tiles,
# 128-k steps).  Small problems only take it when forced; the shapes cover
# a K that ends in a partial stage (1040 = 8 * 128 + 16, 1088 = 8.5 * 128),
# ragged M and N, all cut tiles (fewer tiles than compute units) and whole
# waves plus a cut remainder (batches).
F8_SK_SHAPES = [(2048, 2304, 1024), (2000, 2100, 1040), (1300, 1100, 1088)]


@pytest.mark.parametrize("pair", [("e4m3", "e4m3"), ("e5m2", "e4m3")], ids="-".join)
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("shape", F8_SK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f8_streamk(pair, out, shape, force_streamk):
    fa, fb = pair
    M, N, K = shape
    check(F8(f"f8-streamk-{fa}-{fb}-{out}", fa, fb, out, M, N, K, alpha=0.75, beta=0.5, **TN),
          kernel="f8gemm_mfma_dma_streamk", seed=M + N + K, use_workspace=True, repeat=2)


def test_f8_streamk_whole_waves_fp16_output_and_col_major_c(force_streamk):
    # 65 batches of 2 x 2 tiles: 256 whole, 4 cut over the grid
    check(F8("f8-streamk-dp", "e4m3", "e5m2", "f16", 512, 512, 2048, beta=0.5, batch=65, **TN),
          kernel="f8gemm_mfma_dma_streamk", seed=94, use_workspace=True, repeat=2)
    check(F8("f8-streamk-colC", "e5m2", "e4m3", "bf16", 2304, 2048, 1024, order_c=COL,
             beta=0.5, **TN), kernel="f8gemm_mfma_dma_streamk", seed=95, use_workspace=True)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_f8_streamk_integers_bit_exact(out, force_streamk):
    p = F8(f"f8-streamk-int-{out}", "e4m3", "e5m2", out, 2048, 2304, 1024, alpha=2.0, beta=1.0,
           **TN)
    res, _ = check(p, kernel="f8gemm_mfma_dma_streamk",
                   host=_int_host_f8(p, np.random.default_rng(96)), use_workspace=True, repeat=2)
    assert res.max_err == 0.0 and res.max_ulp == 0


def test_f8_streamk_tail_config_sampled():
    # 4096 x 4352 x 4096 in E4M3: 272 tiles on 256 compute units, the cost
    # model's own choice (no switch), compared on sampled elements
    check(workloads.config("fp8_tail"), kernel="f8gemm_mfma_dma_streamk", sample="auto",
          use_workspace=True, repeat=2)


MX_SK_PAIRS = [("e4m3", "e5m2"), ("e2m3", "e3m2"), ("e2m1", "e2m1")]


@pytest.mark.parametrize("fa,fb", MX_SK_PAIRS, ids=lambda f: f)
@pytest.mark.parametrize("shape", [(600, 700, 1088), (1300, 1100, 2048)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mx_streamk(fa, fb, shape, force_streamk):
    # K = 1088 leaves a last stage of 64 k: the piece that ends there must
    # not use the scale padding bytes (NaN patterns) past the last block
    M, N, K = shape
    check_mx(workloads.MxProblem(f"mx-streamk-{fa}-{fb}", fa, fb, "bf16", M, N, K, alpha=0.5,
                                 beta=1.0), kernel="mxgemm_mfma_dma_streamk", seed=M + K,
             repeat=2, use_workspace=True)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e2m1", "e2m1")], ids=lambda f: f)
def test_mx_streamk_integers_bit_exact_batches_and_col_major_c(fa, fb, force_streamk):
    M, N, K, batch = 520, 600, 1024, 3
    rng = np.random.default_rng(98)
    pats = (mx_int_patterns(rng, fa, batch, M, K), mx_int_patterns(rng, fb, batch, N, K))
    p = workloads.MxProblem("mx-streamk-int", fa, fb, "f32", M, N, K, alpha=2.0, beta=0.0,
                            batch=batch, scale_lo=126, scale_hi=128)
    res, _ = check_mx(p, kernel="mxgemm_mfma_dma_streamk", seed=99, patterns=pats,
                      use_workspace=True, repeat=2)
    assert res.max_err == 0.0
    check_mx(workloads.MxProblem("mx-streamk-colC", fa, fb, "bf16", 700, 520, 512, order_c=COL,
                                 ldc=703, beta=2.0), kernel="mxgemm_mfma_dma_streamk", seed=100,
             use_workspace=True)


def test_mx_streamk_tail_config_sampled():
    # MXFP4 at 4096 x 4352 x 4096 (272 tiles): the cost model's own choice,
    # sampled; without the workspace the same workload runs one workgroup
    # per tile
    check_mx(workloads.config("mxfp4_tail"), kernel="mxgemm_mfma_dma_streamk", sample="auto",
             use_workspace=True)
    check_mx(workloads.config("mxfp4_tail"), sample="auto")


def _random_sk_cases():
    # seeded random shapes for the narrow-float stream-K schedule: ragged M
    # and N, K from one 16-byte chunk up (MX: from one 64-k pair of blocks),
    # every output type, batches, both orders of C for MX
    rng = np.random.default_rng(2024)
    f8, mx = [], []
    for n in range(6):
        M, N = (int(v) for v in rng.integers(200, 2600, 2))
        K = int(rng.integers(1, 190)) * 16
        fa, fb = (str(v) for v in rng.choice(["e4m3", "e5m2"], 2))
        f8.append(F8(f"f8-sk-rand{n}", fa, fb, str(rng.choice(["f32", "bf16", "f16"])), M, N, K,
                     alpha=float(rng.choice([1.0, 0.5])), beta=float(rng.choice([0.0, 1.0])),
                     batch=int(rng.integers(1, 3)), **TN))
    for n in range(6):
        fa, fb = [("e4m3", "e5m2"), ("e2m3", "e3m2"), ("e2m1", "e2m1")][n % 3]
        M, N = (int(v) for v in rng.integers(200, 2600, 2))
        mx.append(workloads.MxProblem(f"mx-sk-rand{n}", fa, fb, str(rng.choice(["f32", "bf16"])), M, N,
                                      int(rng.integers(1, 48)) * 64, alpha=0.5,
                                      beta=float(rng.choice([0.0, 1.0])), batch=int(rng.integers(1, 3)),
                                      order_c=int(rng.choice([ROW, COL]))))
    return f8, mx


SK_RAND_F8, SK_RAND_MX = _random_sk_cases()


@pytest.mark.parametrize("p", SK_RAND_F8, ids=lambda p: p.name)
def test_f8_streamk_random_shapes(p, force_streamk):
    check(p, kernel="f8gemm_mfma_dma_streamk", seed=7, sample="auto", use_workspace=True, repeat=2)


@pytest.mark.parametrize("p", SK_RAND_MX, ids=lambda p: p.name)
def test_mx_streamk_random_shapes(p, force_streamk):
    check_mx(p, kernel="mxgemm_mfma_dma_streamk", seed=8, sample="auto", use_workspace=True, repeat=2)


# ------------------------------------------------------------------ quantised (8-bit) output

QUANT_SHAPES = [(8, 8, 8), (256, 256, 64), (264, 520, 72), (1000, 1032, 1000), (24, 4096, 512)]


@pytest.mark.parametrize("fmt,scale", [("e4m3", 0.5), ("e5m2", 64.0)])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", QUANT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=["nn", "nt", "tn", "tt"])
def test_quant_output(fmt, scale, dt, shape, orders):
    M, N, K = shape
    oa, ob = orders
    res, _ = check(P(f"quant-{dt}-{fmt}", dt, M, N, K, c_dtype=fmt, alpha=0.75, beta=0.0,
                     order_a=oa, order_b=ob, entry="quant", c_scale=scale),
                   kernel="hgemm_mfma_dma", seed=M + N + K)
    assert res.max_ulp <= 1


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quant_output_epilogue_layouts_batches(fmt):
    for act, name in [(GELU, "gelu"), (RELU, "relu")]:
        check(P(f"quant-{name}", "bf16", 520, 264, 200, c_dtype=fmt, beta=0.0, bias=True, act=act,
                entry="quant", c_scale=2.0), kernel="hgemm_mfma_dma", seed=61 + act)
    check(P("quant-colC", "f16", 264, 520, 200, c_dtype=fmt, beta=0.0, order_c=COL, bias=True,
            act=GELU, entry="quant", c_scale=0.25), kernel="hgemm_mfma_dma", seed=63)
    check(P("quant-batch", "bf16", 264, 136, 200, c_dtype=fmt, beta=0.0, batch=3, bias=True,
            stride_bias=0, entry="quant", c_scale=1.0), kernel="hgemm_mfma_dma", seed=64)
    # a scale that sends most values past the largest finite one (saturation)
    # and one that sends most below the smallest normal (subnormals and zeros)
    check(P("quant-saturate", "bf16", 264, 264, 256, c_dtype=fmt, beta=0.0, entry="quant",
            c_scale=1e5), kernel="hgemm_mfma_dma", seed=65)
    check(P("quant-tiny", "bf16", 264, 264, 256, c_dtype=fmt, beta=0.0, entry="quant",
            c_scale=2.0 ** -18), kernel="hgemm_mfma_dma", seed=66)


def test_quant_output_integers_exact():
    # small integers: the fp32 result is exact, so its rounding is the oracle's
    for fmt in ["e4m3", "e5m2"]:
        p = P(f"quant-int-{fmt}", "bf16", 520, 264, 264, c_dtype=fmt, alpha=1.0, beta=0.0,
              entry="quant", c_scale=0.5)
        a, b, _ = _int_host(p, np.random.default_rng(67), -4, 4)
        res, _ = check(p, kernel="hgemm_mfma_dma", repeat=2,
                       host=(a, b, np.zeros(p.buffer_elems("c"), np.uint8)))
        assert res.max_ulp == 0


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quant_rounding_is_exact_at_every_midpoint(fmt):
    # alpha = 0: C = Q(c_scale * bias).  The bias holds every finite value of
    # the format, every midpoint between neighbours (ties: to even), a hair
    # either side of each midpoint, values past the largest finite one,
    # infinities and NaN; all are bf16 values, the scale is 1, so the fp32
    # input of the conversion is exact and the result must equal the
    # oracle's rounding bit for bit.
    vals = oracle.decode(fmt, np.arange(128, dtype=np.uint8))
    v = vals[np.isfinite(vals)]
    mids = (v[:-1] + v[1:]) / 2
    gap = v[1:] - v[:-1]
    cand = np.concatenate([v, mids, mids - gap / 64, mids + gap / 64,
                           [v[-1] * 2, v[-1] * 4, 2.0 ** 100, np.inf, np.nan]])
    cand = np.concatenate([cand, -cand])
    # keep the values bf16 holds exactly
    bf = workloads.to_16bit(cand.astype(np.float32), "bf16")
    exact = oracle.decode("bf16", bf)
    keep = np.isnan(cand) | (exact == cand)
    bias = bf[keep]
    n = bias.size
    p = P(f"quant-midpoints-{fmt}", "bf16", 8, n, 16, c_dtype=fmt, alpha=0.0, beta=0.0, bias=True,
          entry="quant", c_scale=1.0)
    res, out = check(p, kernel="scale", bias_host=bias)
    assert res.max_ulp == 0 and res.strict_fail == 0
    assert n > 400 and np.isnan(oracle.decode("bf16", bias)).sum() == 2


# ------------------------------------------------------------------ fp32 as three bf16 products

X3_SHAPES = [(8, 8, 8), (256, 256, 256), (264, 520, 1001), (1000, 1032, 1000), (4095, 97, 333),
             (16, 4096, 4096), (3, 5, 7)]


@pytest.mark.parametrize("shape", X3_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],
                         ids=["nn", "nt", "tn", "tt"])
def test_bf16x3(shape, orders):
    # fp32 within the fp32 criterion; the copies are always K-contiguous and
    # aligned, whatever the caller's layout (K not a multiple of 8 padded)
    M, N, K = shape
    oa, ob = orders
    res, _ = check(P("x3", "f32", M, N, K, alpha=0.75, beta=0.5, order_a=oa, order_b=ob,
                     entry="bf16x3"), seed=M + N + K)
    assert res.kernel in ("hgemm_mfma_dma", "hgemm_splitk", "gemm_skinny"), res.kernel


def test_bf16x3_col_major_c_batches_and_beta_zero():
    check(P("x3-colC", "f32", 520, 264, 300, order_c=COL, beta=-1.0, entry="bf16x3"), seed=51)
    check(P("x3-batch", "f32", 264, 136, 520, batch=3, beta=0.5, entry="bf16x3"), seed=52)
    check(P("x3-shared-b", "f32", 264, 136, 520, batch=3, stride_b=0, entry="bf16x3"), seed=53)
    check(P("x3-shared-a", "f32", 264, 136, 520, batch=3, stride_a=0, entry="bf16x3"), seed=54)
    # beta = 0: C is not read (NaN there does not propagate)
    check(P("x3-nan-c", "f32", 300, 200, 100, entry="bf16x3"), seed=55, c_init=np.nan)


def test_bf16x3_misaligned_bases():
    # fp32 operands 4 or 12 bytes off a 16-byte boundary: the split reads them
    # element by element; its copies are aligned all the same
    for oa, ob in [(ROW, ROW), (COL, COL)]:
        res, _ = check(P("x3-misaligned", "f32", 264, 520, 512, beta=0.5, order_a=oa, order_b=ob,
                         entry="bf16x3"), seed=60, base_offset=(1, 3, 1))
        assert res.kernel == "hgemm_splitk"  # six tiles of K' = 1536


def test_bf16x3_nothing_to_multiply():
    res, _ = check(P("x3-alpha0", "f32", 130, 70, 40, alpha=0.0, beta=0.5, entry="bf16x3"),
                   seed=56)
    assert res.kernel == "scale"
    res, _ = check(P("x3-k0", "f32", 130, 70, 0, beta=-1.5, entry="bf16x3"), seed=57)
    assert res.kernel == "scale"


def test_bf16x3_integers_bit_exact():
    # small integers split with lo = 0: every product and sum is exact
    p = P("x3-int", "f32", 520, 1032, 2000, alpha=2.0, beta=1.0, batch=2, entry="bf16x3")
    res, _ = check(p, host=_int_host(p, np.random.default_rng(58)), repeat=2)
    assert res.max_err == 0.0


def test_bf16x3_wide_exponent_range():
    # operands spread over 2^-40 .. 2^40: the split is relative, so the
    # normalised error stays at the fp32 level
    p = P("x3-range", "f32", 264, 264, 520, entry="bf16x3")
    rng = np.random.default_rng(59)
    def mk(n):
        return (rng.uniform(-1, 1, n) * np.exp2(rng.integers(-40, 41, n))).astype(np.float32)
    host = (mk(p.buffer_elems("a")), mk(p.buffer_elems("b")), mk(p.buffer_elems("c")))
    res, _ = check(p, host=host)
    assert res.max_err < 2.0 ** -14, res.max_err


def test_bf16x3_workload_full_size():
    res, _ = check(workloads.config("f32_4096_bf16x3"), sample="auto")
    assert res.kernel == "hgemm_mfma_dma"


# ------------------------------------------------------------------ skinny split-K across workgroups (workspace)

# (5, 8192, 4008): slices of four 128-row rounds, the last slice ending in a
# partial round whose last instruction step is itself partial
SKINNY_SK_SHAPES = [(16, 4096, 4096), (1, 1024, 3000), (7, 1000, 2048), (12, 520, 1024), (5, 8192, 4008)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SKINNY_SK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_skinny_splitk(dt, shape):
    # 128-column blocks of a row-major B split over K across workgroups, the
    # slices added in fixed order by a second kernel: run twice, bit for bit
    M, N, K = shape
    check(P(f"skinny-sk-{dt}", dt, M, N, K, alpha=0.5, beta=1.5), kernel="gemm_skinny_splitk",
          seed=M + N + K, use_workspace=True, repeat=2)


def test_skinny_splitk_fp32_output_batches_and_integers():
    check(P("skinny-sk-f32out", "bf16", 16, 2048, 4096, c_dtype="f32", beta=-1.0),
          kernel="gemm_skinny_splitk", seed=31, use_workspace=True)
    check(P("skinny-sk-batch", "f16", 9, 1536, 2048, batch=3, beta=0.5),
          kernel="gemm_skinny_splitk", seed=32, use_workspace=True)
    check(P("skinny-sk-shared-b", "bf16", 16, 1024, 2048, batch=2, stride_b=0),
          kernel="gemm_skinny_splitk", seed=33, use_workspace=True)
    p = P("skinny-sk-int", "bf16", 16, 4096, 4096, c_dtype="f32", alpha=2.0, beta=1.0)
    res, _ = check(p, kernel="gemm_skinny_splitk", host=_int_host(p, np.random.default_rng(34)),
                   use_workspace=True)
    assert res.max_err == 0.0


def test_skinny_splitk_workload_full_size():
    check(workloads.config("bf16_skinny"), kernel="gemm_skinny_splitk", use_workspace=True,
          repeat=2)
