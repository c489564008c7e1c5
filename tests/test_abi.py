"""The C ABI on the CPU: every declared symbol is exported, and argument
validation returns its status codes before any HIP call (so none of these
tests needs a GPU: no call here reaches a kernel launch)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgemm.h")


@pytest.fixture(scope="module")
def lib():
    from dense_gemm_optimisation_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from dense_gemm_optimisation_amd import build
        build.build()
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["gemm_abi_version", "gemm_bf16", "gemm_bf16_bias_act",
                                    "gemm_bf16_noalloc", "gemm_bf16_quant", "gemm_bf16_ws",
                                    "gemm_f16",
                                    "gemm_f16_bias_act",
                                    "gemm_f16_quant",
                                    "gemm_f16_ws", "gemm_f32", "gemm_f32_bf16x3",
                                    "gemm_f32_bf16x3_workspace_size", "gemm_f32_bias_act",
                                    "gemm_f32_valu", "gemm_f32_ws",
                                    "gemm_f8",
                                    "gemm_f8_kernel_name", "gemm_f8_kernel_name_ws",
                                    "gemm_f8_ws", "gemm_kernel_name",
                                    "gemm_kernel_name_bf16x3", "gemm_kernel_name_quant",
                                    "gemm_kernel_name_ws", "gemm_mx", "gemm_mx_kernel_name",
                                    "gemm_mx_kernel_name_ws", "gemm_mx_ws",
                                    "gemm_status_string",
                                    "gemm_test_switches", "gemm_workspace_size"]


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib.library(), name) is not None


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "libgemm.h"\nint f(void){return gemm_abi_version();}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-c",
                    str(src), "-o", str(tmp_path / "use.o")], check=True)


def test_status_strings(lib):
    assert lib.status_string(0) == "GEMM_OK"
    for code in (-1, -2, -3, -4):
        assert lib.status_string(code).startswith("GEMM_ERR_")
    assert lib.status_string(7) == "unknown gemm_status_t"
    assert lib.abi_version() == 1


P = 0x10000  # a fake, never-dereferenced device address


def call(lib, fn="f32", M=8, N=8, K=8, alpha=1.0, A=P, lda=8, oa=0, B=P * 3, ldb=8, ob=0,
         beta=0.0, C=P * 5, ldc=8, oc=0, c_dtype=0, batch=1, sa=0, sb=0, sc=0, fa=0, fb=0,
         type_c=1):
    if fn == "e4m3":  # gemm_f8, formats fa / fb, C of type type_c (bf16 by default)
        return lib.gemm_f8(M, N, K, alpha, A, lda, oa, fa, B, ldb, ob, fb, beta, C, ldc, oc,
                           type_c, batch, sa, sb, sc, 0, raise_on_error=False)
    if fn == "f32":
        return lib.gemm_f32(M, N, K, alpha, A, lda, oa, B, ldb, ob, beta, C, ldc, oc, batch, sa,
                            sb, sc, 0, raise_on_error=False)
    f = lib.gemm_bf16 if fn == "bf16" else lib.gemm_f16
    return f(M, N, K, alpha, A, lda, oa, B, ldb, ob, beta, C, ldc, oc, c_dtype, batch, sa, sb,
             sc, 0, raise_on_error=False)


INVALID = {
    "negative M": dict(M=-1),
    "negative N": dict(N=-1),
    "negative K": dict(K=-2),
    "negative batch": dict(batch=-1),
    "negative stride": dict(sa=-1),
    "order A out of range": dict(oa=2),
    "order B out of range": dict(ob=-1),
    "order C out of range": dict(oc=5),
    "lda < K (row-major A)": dict(lda=7),
    "lda < M (col-major A)": dict(oa=1, M=9, lda=8),
    "ldb < N (row-major B)": dict(ldb=7),
    "ldb < K (col-major B)": dict(ob=1, ldb=7),
    "ldc < N": dict(ldc=7),
    "ldc < M (col-major C)": dict(oc=1, M=12, lda=8, ldc=8),
    "ld zero": dict(M=1, K=0, lda=0),
    "null A": dict(A=0),
    "null B": dict(B=0),
    "null C": dict(C=0),
    "C overlaps A": dict(C=P + 4 * 10),
    "C overlaps B": dict(C=P * 3 + 4 * 63),
    "C slices overlap": dict(batch=2, sc=63),
    "C slices coincide": dict(batch=3, sc=0),
}


@pytest.mark.parametrize("fn", ["f32", "bf16", "f16", "e4m3"])
@pytest.mark.parametrize("case", sorted(INVALID))
def test_invalid_arguments(lib, fn, case):
    kw = dict(INVALID[case])
    esz = {"f32": 4, "bf16": 2, "f16": 2, "e4m3": 1}[fn]  # A and B span 64 elements
    if case == "C overlaps A":
        kw["C"] = P + esz * 10
    if case == "C overlaps B":
        kw["C"] = P * 3 + esz * 63
    assert call(lib, fn, **kw) == lib.ERR_INVALID_ARG, case


@pytest.mark.parametrize("fn", ["f32", "bf16", "f16", "e4m3"])
def test_pointers_off_their_element_size(lib, fn):
    # C is fp32 for f32 and bf16 for e4m3 (type_c default); A and B have
    # the input element size (no constraint for 8-bit inputs)
    esz = {"f32": 4, "bf16": 2, "f16": 2, "e4m3": 1}[fn]
    esz_c = 4 if fn == "f32" else 2
    for off in range(1, esz_c):
        assert call(lib, fn, C=P * 5 + off) == lib.ERR_INVALID_ARG, off
    for off in range(1, esz):
        assert call(lib, fn, A=P + off) == lib.ERR_INVALID_ARG, off
        assert call(lib, fn, B=P * 3 + off) == lib.ERR_INVALID_ARG, off


def mx_call(lib, M=300, N=260, K=256, alpha=1.0, A=P, lda=256, fa=4, SA=P * 2, ldsa=8, B=P * 3,
            ldb=256, fb=4, SB=P * 4, ldsb=8, beta=0.0, C=P * 5, ldc=260, oc=0, tc=1, batch=1,
            sa=0, sb=0, ssa=0, ssb=0, sc=0, name=False):
    """gemm_mx (or, with name=True, gemm_mx_kernel_name) with fake addresses:
    by default an MXFP4 300 x 260 x 256 problem, bf16 C."""
    args = (M, N, K, alpha, A, lda, fa, SA, ldsa, B, ldb, fb, SB, ldsb, beta, C, ldc, oc, tc, batch,
            sa, sb, ssa, ssb, sc)
    if name:
        return lib.mx_kernel_name(*args)
    return lib.gemm_mx(*args, 0, raise_on_error=False)


MX_INVALID = {
    "K not a multiple of 64": dict(K=224),
    "negative M": dict(M=-1),
    "negative scale stride": dict(ssa=-4),
    "format out of range": dict(fa=5),
    "format negative": dict(fb=-1),
    "typeC out of range": dict(tc=3),
    "order C out of range": dict(oc=2),
    "lda not a multiple of 64": dict(lda=288, K=256),
    "ldb below K": dict(ldb=192),
    "A not 16-byte aligned": dict(A=P + 8),
    "B not 16-byte aligned": dict(B=P * 3 + 4),
    "ldsa not a multiple of 4": dict(ldsa=10),
    "ldsb below 4*ceil(K/128)": dict(ldsb=4, K=256),
    "scale not 4-byte aligned": dict(SA=P * 2 + 2),
    "scale stride not a multiple of 4": dict(batch=2, ssa=6, sa=300 * 256, sb=0, sc=300 * 260),
    "A stride not a multiple of 64": dict(batch=2, sa=32, sc=300 * 260),
    "null scale": dict(SB=0),
    "null A": dict(A=0),
    "C not element-aligned": dict(C=P * 5 + 1),
    "ldc below N": dict(ldc=259),
    "C slices overlap": dict(batch=2, sc=100),
    "C overlaps a scale array": dict(C=P * 2 + 64),
    "C overlaps A": dict(C=P + 64),
}


@pytest.mark.parametrize("case", sorted(MX_INVALID))
def test_mx_invalid_arguments(lib, case):
    assert mx_call(lib, **MX_INVALID[case]) == lib.ERR_INVALID_ARG, case
    assert mx_call(lib, name=True, **MX_INVALID[case]) is None, case


def test_mx_kernel_choice_and_unsupported_pairs(lib):
    assert mx_call(lib, name=True) == "mxgemm_mfma_dma"
    for fa, fb in ((0, 0), (0, 1), (1, 0), (1, 1), (2, 2), (2, 3), (3, 2), (3, 3), (4, 4)):
        assert mx_call(lib, name=True, fa=fa, fb=fb) == "mxgemm_mfma_dma", (fa, fb)
    # formats of different widths share no stage layout
    for fa, fb in ((0, 4), (4, 2), (2, 1)):
        assert mx_call(lib, fa=fa, fb=fb) == lib.ERR_UNSUPPORTED, (fa, fb)
    # column-major C, padded leading dimensions, K = 64 mod 128, batches
    assert mx_call(lib, name=True, oc=1, ldc=300) == "mxgemm_mfma_dma"
    assert mx_call(lib, name=True, K=320, lda=384, ldb=320, ldsa=12, ldsb=12) == "mxgemm_mfma_dma"
    assert mx_call(lib, name=True, batch=3, sa=300 * 256, sb=0, ssa=300 * 8, ssb=0,
                   sc=300 * 260) == "mxgemm_mfma_dma"
    # alpha == 0 or K == 0: only beta * C, the operands and scales are not checked
    assert mx_call(lib, name=True, alpha=0.0, A=0, SA=0) == "scale"
    assert mx_call(lib, name=True, K=0, lda=64, ldsa=0, ldsb=0) == "scale"
    assert mx_call(lib, name=True, M=0) == ""
    # slices too large for 32-bit offsets
    far = 1 << 40
    assert mx_call(lib, M=70000, N=4, K=32768, lda=32768, ldb=32768, ldsa=1024, ldsb=1024, ldc=4,
                   SA=far, B=2 * far, SB=3 * far, C=4 * far) == lib.ERR_UNSUPPORTED


def test_f8_bad_formats_and_output_type(lib):
    for kw in (dict(fa=2), dict(fa=-1), dict(fb=2), dict(type_c=3), dict(type_c=-1)):
        assert call(lib, "e4m3", **kw) == lib.ERR_INVALID_ARG, kw
    for fa in (0, 1):
        for fb in (0, 1):
            for tc in (0, 1, 2):
                assert call(lib, "e4m3", M=0, fa=fa, fb=fb, type_c=tc) == lib.OK


@pytest.mark.parametrize("fn", ["bf16", "f16"])
def test_bad_c_dtype(lib, fn):
    assert call(lib, fn, c_dtype=2) == lib.ERR_INVALID_ARG
    assert call(lib, fn, c_dtype=-1) == lib.ERR_INVALID_ARG


@pytest.mark.parametrize("fn", ["f32", "bf16", "f16", "e4m3"])
@pytest.mark.parametrize("kw", [dict(M=0), dict(N=0), dict(batch=0),
                                dict(M=0, A=0, B=0, C=0), dict(batch=0, A=0, B=0, C=0)])
def test_empty_problems_return_ok_without_work(lib, fn, kw):
    assert call(lib, fn, **kw) == lib.OK


def test_adjacent_buffers_are_not_overlap(lib):
    # C starting exactly where A ends is fine; validation must not flag it.
    # (M == 0 keeps the call from launching anything.)
    assert call(lib, "f32", M=0, C=P + 4 * 64) == lib.OK


def epi_call(lib, fn="f32", bias=P * 7, stride_bias=0, act=0, **kw):
    args = dict(M=8, N=8, K=8, alpha=1.0, A=P, lda=8, oa=0, B=P * 3, ldb=8, ob=0, beta=0.0,
                C=P * 5, ldc=8, oc=0, c_dtype=0, batch=1, sa=0, sb=0, sc=0)
    args.update(kw)
    a = args
    if fn == "f32":
        return lib.gemm_f32_bias_act(a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["oa"],
                                     a["B"], a["ldb"], a["ob"], a["beta"], a["C"], a["ldc"],
                                     a["oc"], a["batch"], a["sa"], a["sb"], a["sc"], bias,
                                     stride_bias, act, 0, raise_on_error=False)
    f = lib.gemm_bf16_bias_act if fn == "bf16" else lib.gemm_f16_bias_act
    return f(a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["oa"], a["B"], a["ldb"],
             a["ob"], a["beta"], a["C"], a["ldc"], a["oc"], a["c_dtype"], a["batch"], a["sa"],
             a["sb"], a["sc"], bias, stride_bias, act, 0, raise_on_error=False)


@pytest.mark.parametrize("fn", ["f32", "bf16", "f16"])
def test_fused_epilogue_invalid_arguments(lib, fn):
    esz = 4 if fn == "f32" else 2
    assert epi_call(lib, fn, act=3) == lib.ERR_INVALID_ARG
    assert epi_call(lib, fn, act=-1) == lib.ERR_INVALID_ARG
    assert epi_call(lib, fn, stride_bias=-1) == lib.ERR_INVALID_ARG
    # the bias may not overlap C (C spans 64 elements from P*5)
    assert epi_call(lib, fn, bias=P * 5 + esz * 60) == lib.ERR_INVALID_ARG
    # ... nor, through its batch stride, reach into C
    assert epi_call(lib, fn, bias=P * 5 - esz * 100, stride_bias=70, batch=3, sc=64) == \
        lib.ERR_INVALID_ARG
    # the usual checks still apply
    assert epi_call(lib, fn, M=-1) == lib.ERR_INVALID_ARG
    assert epi_call(lib, fn, lda=7) == lib.ERR_INVALID_ARG
    if fn != "f32":
        assert epi_call(lib, fn, c_dtype=2) == lib.ERR_INVALID_ARG


@pytest.mark.parametrize("fn", ["f32", "bf16", "f16"])
def test_fused_epilogue_empty_problems_and_null_bias(lib, fn):
    assert epi_call(lib, fn, M=0, act=2) == lib.OK
    assert epi_call(lib, fn, batch=0, bias=0, act=1) == lib.OK
    # a bias right after C is fine (C is 64 elements); M == 0 launches nothing
    esz = 4 if fn == "f32" else 2
    assert epi_call(lib, fn, M=0, bias=P * 5 + esz * 64) == lib.OK


def test_raises_on_error(lib):
    with pytest.raises(lib.GemmError) as e:
        lib.gemm_f32(-1, 1, 1, 1.0, P, 1, 0, P, 1, 0, 0.0, P, 1, 0)
    assert e.value.status == lib.ERR_INVALID_ARG


# ------------------------------------------------------------------ kernel choice (host only)

GB = 1 << 32  # operands 4 GiB apart: fake, never-dereferenced, 16-byte aligned addresses


def kname(lib, dt, M, N, K, alpha=1.0, oa=0, ob=0, oc=0, lda=None, ldb=None, ldc=None,
          A=GB, B=2 * GB, C=3 * GB, beta=0.0, c_dtype=0, batch=1, sa=0, sb=0, sc=0, bdt=None,
          out="bf16"):
    lda = lda or (K if oa == 0 else M)
    ldb = ldb or (N if ob == 0 else K)
    ldc = ldc or (N if oc == 0 else M)
    return lib.kernel_name(dt, M, N, K, alpha, A, lda, oa, B, ldb, ob, beta, C, ldc, oc, c_dtype,
                           batch, sa, sb, sc, b_dtype=bdt, out_dtype=out)


@pytest.fixture
def clean_env(switches):
    """No kernel-choice override is set (the switches fixture clears them
    before and after the test)."""
    return switches


KERNEL_CASES = [
    # (dtype, M, N, K, extra arguments, kernel)
    ("f32", 4096, 4096, 4096, {}, "sgemm_mfma_dma"),
    ("f32", 4096, 4096, 4096, dict(A=GB + 4), "sgemm_mfma"),        # base not 16-byte aligned
    ("f32", 4096, 4096, 4096, dict(lda=4097), "sgemm_mfma"),        # rows not 16-byte aligned
    ("f32", 4096, 4096, 4098, {}, "sgemm_mfma"),                    # K not a multiple of 4
    ("f32", 256, 256, 256, {}, "sgemm_splitk"),                     # 4 tiles of 128 x 128
    ("f32", 1536, 1536, 1536, {}, "sgemm_splitk"),                  # 144 tiles
    ("f32", 2048, 2048, 2048, {}, "sgemm_mfma_dma"),                # 256 tiles
    ("f32", 256, 256, 128, {}, "sgemm_mfma_dma"),                   # K too short to split
    ("f32", 16, 4096, 4096, {}, "sgemm_splitk"),                    # N-contiguous B: split-K
    ("f32", 16, 4096, 4096, dict(ob=1), "gemm_skinny"),
    ("f32", 16, 16384, 4096, dict(ob=1), "sgemm_splitk"),
    ("f32", 16, 4096, 4096, dict(oa=1, ob=1), "sgemm_splitk"),      # skinny needs K-contiguous A
    ("f32", 17, 4096, 4096, {}, "sgemm_splitk"),
    ("bf16", 4096, 4096, 4096, {}, "hgemm_mfma_dma"),
    ("f16", 4096, 4096, 4096, dict(ob=1), "hgemm_mfma_dma"),
    ("bf16", 4095, 4097, 1001, {}, "hgemm_mfma"),
    ("bf16", 4096, 4096, 4096, dict(B=2 * GB + 2), "hgemm_mfma"),
    ("bf16", 16, 4096, 4096, {}, "gemm_skinny"),
    ("bf16", 1, 4096, 4096, dict(ob=1), "gemm_skinny"),
    ("bf16", 32, 4096, 4096, {}, "hgemm_splitk"),
    ("bf16", 256, 256, 8192, {}, "hgemm_splitk"),
    ("bf16", 256, 256, 256, {}, "hgemm_mfma_dma"),                  # K too short to split
    ("bf16", 4096, 12288, 4096, {}, "hgemm_mfma_dma"),
    ("bf16", 4096, 4096, 4096, dict(alpha=0.0, beta=2.0), "scale"),
    ("f32", 4096, 4096, 0, dict(beta=2.0, lda=1), "scale"),
    ("bf16", 0, 4096, 4096, {}, ""),
    ("f32", 4096, 4096, 4096, dict(lda=100), None),                 # invalid: lda < K
    # column-major C: computed as C^T = B^T A^T, so the roles of M and N swap
    ("bf16", 4096, 16, 4096, dict(oc=1, ob=1), "gemm_skinny"),
    ("bf16", 4096, 16, 4096, dict(oc=1), "hgemm_splitk"),
    # 8-bit floats: the direct-load kernel for K-contiguous, aligned A and B
    ("e4m3", 4096, 4096, 4096, dict(ob=1), "f8gemm_mfma_dma"),
    ("e5m2", 4096, 4096, 4096, dict(ob=1, bdt="e4m3", out="f32"), "f8gemm_mfma_dma"),
    ("e4m3", 4096, 4096, 4096, dict(ob=1, oc=1, out="f16"), "f8gemm_mfma_dma"),
    ("e4m3", 16, 4096, 4096, dict(ob=1), "f8gemm_mfma_dma"),       # no skinny kernel for 8-bit
    ("e4m3", 4095, 4097, 4096, dict(ob=1), "f8gemm_mfma_dma"),     # ragged M, N are fine
    ("e4m3", 4096, 4096, 4096, {}, "f8gemm_mfma"),                 # N-contiguous B
    ("e4m3", 4096, 4096, 4096, dict(oa=1, ob=1), "f8gemm_mfma"),   # M-contiguous A
    ("e4m3", 4096, 4096, 4104, dict(ob=1), "f8gemm_mfma"),         # K not a multiple of 16
    ("e4m3", 4096, 4096, 4096, dict(ob=1, A=GB + 8), "f8gemm_mfma"),
    ("e4m3", 4096, 4096, 4096, dict(ob=1, ldb=4100), "f8gemm_mfma"),
    ("e4m3", 4096, 4096, 4096, dict(ob=1, batch=2, sa=4096 * 4096 + 8, sb=0,
                                    sc=4096 * 4096), "f8gemm_mfma"),
    ("e4m3", 4096, 4096, 4096, dict(ob=1, alpha=0.0, beta=1.0), "scale"),
    ("e4m3", 4096, 4096, 4096, dict(ob=1, lda=100), None),
]


@pytest.mark.parametrize("case", KERNEL_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[5]}")
def test_kernel_choice(lib, clean_env, case):
    dt, M, N, K, kw, want = case
    assert kname(lib, dt, M, N, K, **kw) == want


def test_kernel_choice_testing_switches(lib, clean_env):
    clean_env(lib.TEST_NO_SPLITK)
    assert kname(lib, "f32", 256, 256, 256) == "sgemm_mfma_dma"
    assert kname(lib, "bf16", 16, 4096, 4096) == "hgemm_mfma_dma"
    clean_env(lib.TEST_FORCE_GENERAL)
    assert kname(lib, "f32", 4096, 4096, 4096) == "sgemm_mfma"
    assert kname(lib, "bf16", 16, 4096, 4096) == "hgemm_mfma"
    assert kname(lib, "e4m3", 4096, 4096, 4096, ob=1) == "f8gemm_mfma"
    clean_env(lib.TEST_NO_SPLITK)
    assert kname(lib, "e4m3", 4096, 4096, 4096, ob=1) == "f8gemm_mfma_dma"
    clean_env(lib.TEST_F32_VALU)
    assert kname(lib, "f32", 16, 4096, 4096, ob=1) == "sgemm_valu"
    assert kname(lib, "bf16", 4096, 4096, 4096) == "hgemm_mfma_dma"
    # the setter returns the previous set; flags outside the four are dropped
    assert lib.test_switches(0xff) == lib.TEST_F32_VALU
    assert lib.test_switches(0) == 15
    # an environment variable no longer changes anything
    import os
    os.environ["LIBGEMM_FORCE_GENERAL"] = "1"
    try:
        assert kname(lib, "f32", 4096, 4096, 4096) == "sgemm_mfma_dma"
    finally:
        del os.environ["LIBGEMM_FORCE_GENERAL"]


def test_kernel_choice_for_every_workload(lib, clean_env):
    # the kernel each benchmark workload runs on, with its own layouts and
    # (16-byte aligned) buffers
    import workloads
    want = {"f32_256": "sgemm_splitk", "f32_4096": "sgemm_mfma_dma",
            "bf16_4096": "hgemm_mfma_dma", "f16_4096": "hgemm_mfma_dma",
            "bf16_qkv": "hgemm_mfma_dma", "bf16_ffn_up": "hgemm_mfma_dma",
            "bf16_ffn_down": "hgemm_mfma_dma", "f32_edge": "sgemm_mfma",
            "bf16_edge": "hgemm_mfma", "bf16_tail": "hgemm_mfma_dma", "bf16_skinny": "gemm_skinny",
            "bf16_attn_qk": "hgemm_mfma_dma", "bf16_attn_pv": "hgemm_mfma_dma",
            "bf16_ffn_up_gelu": "hgemm_mfma_dma", "fp8_4096": "f8gemm_mfma_dma",
            "fp8_tail": "f8gemm_mfma_dma",
            "bf16_ffn_up_gelu_e4m3": "hgemm_mfma_dma",
            # called through gemm_f32_valu and gemm_f32_bf16x3; gemm_kernel_name
            # describes gemm_f32
            "f32_4096_valu": "sgemm_mfma_dma", "f32_4096_bf16x3": "sgemm_mfma_dma"}
    mx = {n for n, p in workloads.CONFIGS.items() if isinstance(p, workloads.MxProblem)}
    assert mx == {"mxfp4_4096", "mxfp6_4096", "mxfp8_4096", "mxfp4_tail"}
    assert sorted(want) == sorted(set(workloads.CONFIGS) - mx)
    for name in mx:
        p = workloads.config(name)
        got = lib.mx_kernel_name(p.M, p.N, p.K, p.alpha, GB, p.lda, lib.MX_FORMAT[p.fa], 4 * GB,
                                 p.ldsa, 2 * GB, p.ldb, lib.MX_FORMAT[p.fb], 5 * GB, p.ldsb, p.beta,
                                 3 * GB, p.ldc, p.order_c, lib.OUTPUT_BF16, p.batch, p.stride_a,
                                 p.stride_b, p.stride_sa, p.stride_sb, p.stride_c)
        assert got == "mxgemm_mfma_dma", name
    for name, k in want.items():
        p = workloads.config(name)
        c_dt = 1 if (p.c_dtype == "f32" and p.in_dtype != "f32") else 0
        got = lib.kernel_name(p.in_dtype, p.M, p.N, p.K, p.alpha, GB, p.lda, p.order_a, 2 * GB,
                              p.ldb, p.order_b, p.beta, 3 * GB, p.ldc, p.order_c, c_dt, p.batch,
                              p.stride_a, p.stride_b, p.stride_c, b_dtype=p.b_dtype,
                              out_dtype=p.c_dtype)
        assert got == k, name


# ------------------------------------------------------------------ workspace entry points (host only)

WS = 5 * GB  # fake, 256-byte aligned workspace address


def test_workspace_size(lib):
    # two 256 x 256 fp32 partial tiles per workgroup, 256 workgroups
    assert lib.workspace_size() == 2 * 256 * 256 * 256 * 4


def kname_ws(lib, dt, M, N, K, ws=WS, nbytes=None, **kw):
    oa, ob, oc = kw.pop("oa", 0), kw.pop("ob", 0), kw.pop("oc", 0)
    lda = kw.pop("lda", K if oa == 0 else M)
    ldb = kw.pop("ldb", N if ob == 0 else K)
    ldc = kw.pop("ldc", N if oc == 0 else M)
    nbytes = lib.workspace_size() if nbytes is None else nbytes
    batch = kw.pop("batch", 1)
    strides = (M * K, K * N, M * N) if batch > 1 else (0, 0, 0)
    return lib.kernel_name(dt, M, N, K, kw.pop("alpha", 1.0), GB, lda, oa, 2 * GB, ldb, ob, 0.0,
                           3 * GB, ldc, oc, 0, batch, *strides, workspace=ws,
                           workspace_bytes=nbytes)


def test_streamk_kernel_choice(lib, clean_env):
    # unaligned with at least 64 tiles: operands copied into the workspace,
    # then the direct-load kernel (272 tiles of 16 k-steps: the cut tail
    # saves less than its exchange costs) or its stream-K schedule (64 steps)
    assert kname_ws(lib, "bf16", 4095, 4097, 1001) == "hgemm_mfma_dma_packed"
    assert kname_ws(lib, "bf16", 4095, 4351, 4095) == "hgemm_mfma_dma_streamk_packed"
    assert kname_ws(lib, "f16", 4095, 4095, 1001, oa=1, ob=1) == "hgemm_mfma_dma_packed"
    # fewer than 64 tiles: the general kernel's stream-K schedule
    assert kname_ws(lib, "f16", 300, 290, 8193) == "hgemm_mfma_streamk"
    # workspace too small, or absent: the plain general kernel
    assert kname_ws(lib, "bf16", 4095, 4097, 1001, nbytes=1 << 20) == "hgemm_mfma"
    assert kname_ws(lib, "bf16", 4095, 4097, 1001, ws=0, nbytes=0) == "hgemm_mfma"
    # copies larger than the workspace (16384 x 4104 bf16 is 134 MB): the
    # general kernel (4096 tiles are whole waves, nothing to cut)
    assert kname_ws(lib, "bf16", 16383, 16383, 4097) == "hgemm_mfma"
    # too little work for stream-K on few tiles
    assert kname_ws(lib, "bf16", 300, 290, 131) == "hgemm_mfma"
    # 500 tiles: the last wave (244 tiles) is nearly full, the exchange would cost more
    assert kname_ws(lib, "bf16", 5119, 6399, 1001) == "hgemm_mfma_dma_packed"
    # 65 batches of 4 tiles: copied, 256 tiles whole and 4 cut over the grid
    assert kname_ws(lib, "bf16", 300, 290, 1001, batch=65) == "hgemm_mfma_dma_streamk_packed"
    # aligned: the direct-load kernel's schedule where the saved steps exceed
    # its exchange (the shapes and outcomes measured on MI355X: 272 tiles of
    # 32 and 64 steps gain, 16 steps and 136 tiles lose, 288 tiles of 32 tie)
    assert kname_ws(lib, "bf16", 4096, 4352, 4096) == "hgemm_mfma_dma_streamk"
    assert kname_ws(lib, "bf16", 4096, 4352, 2048) == "hgemm_mfma_dma_streamk"
    assert kname_ws(lib, "bf16", 4096, 4352, 1024) == "hgemm_mfma_dma"
    assert kname_ws(lib, "bf16", 2048, 4352, 2048) == "hgemm_mfma_dma"
    assert kname_ws(lib, "bf16", 4096, 4608, 2048) == "hgemm_mfma_dma"
    assert kname_ws(lib, "f16", 2048, 2304, 1024, oa=1, ob=1) == "hgemm_mfma_dma"
    # fewer than 64 tiles: the split-K kernel, workspace or not
    assert kname_ws(lib, "bf16", 512, 768, 8192) == "hgemm_splitk"
    assert kname_ws(lib, "bf16", 4096, 4352, 256) == "hgemm_mfma_dma"       # 4 steps per tile
    assert kname_ws(lib, "bf16", 4096, 4096, 4096) == "hgemm_mfma_dma"      # whole waves
    # GEMM_TEST_FORCE_STREAMK skips the cost model, not the structural checks
    clean_env(lib.TEST_FORCE_STREAMK)
    assert kname_ws(lib, "f16", 2048, 2304, 1024, oa=1, ob=1) == "hgemm_mfma_dma_streamk"
    assert kname_ws(lib, "bf16", 4096, 4352, 256) == "hgemm_mfma_dma_streamk"
    assert kname_ws(lib, "bf16", 300, 290, 131) == "hgemm_mfma_streamk"
    assert kname_ws(lib, "bf16", 4096, 4096, 4096) == "hgemm_mfma_dma"      # nothing to cut
    assert kname_ws(lib, "bf16", 512, 768, 8192) == "hgemm_splitk"
    # N = 4097: the one-column last tile column runs on its own (split-K on
    # the copies), and the rest is whole waves; a wider last column (54) is
    # kept in the grid, whose last wave is then cut
    assert kname_ws(lib, "bf16", 4095, 4097, 1001) == "hgemm_mfma_dma_packed"
    assert kname_ws(lib, "bf16", 4095, 4150, 1001) == "hgemm_mfma_dma_streamk_packed"
    clean_env(0)
    # fp32: unaligned with at least 160 tiles of 128 x 128 is copied for the
    # direct-load kernel, on its stream-K schedule where the cut tail pays
    # (1056 tiles of 63 k steps: 1024 whole and 32 cut); fewer tiles use the
    # general kernel's schedule (128 x 128 tiles, 1024 workgroups).  N = 4097
    # leaves one column in its last tile column: that column runs on its own
    # and the remaining 1024 tiles are whole waves
    assert kname_ws(lib, "f32", 4095, 4097, 1001) == "sgemm_mfma_dma_packed"
    assert kname_ws(lib, "f32", 4095, 4140, 1001) == "sgemm_mfma_dma_streamk_packed"  # last column: 44
    assert kname_ws(lib, "f32", 4095, 4097, 129) == "sgemm_mfma_dma_packed"
    # 187 tiles of 63 steps: the partial tiles and copies exceed the workspace
    assert kname_ws(lib, "f32", 2049, 1283, 1001) == "sgemm_mfma_dma_packed"
    assert kname_ws(lib, "f32", 1500, 1300, 2001) == "sgemm_mfma_streamk"   # 132 tiles
    assert kname_ws(lib, "f32", 1500, 1300, 129) == "sgemm_mfma"            # 9 steps per tile
    # aligned: the direct-load kernel, on its stream-K schedule when tiles are cut
    assert kname_ws(lib, "f32", 4096, 4096, 4096) == "sgemm_mfma_dma"       # whole waves
    assert kname_ws(lib, "f32", 4096, 4224, 256) == "sgemm_mfma_dma_streamk"
    assert kname_ws(lib, "f32", 2048, 2176, 1000, oa=1, ob=1) == "sgemm_mfma_dma_streamk"
    assert kname_ws(lib, "f32", 4096, 4224, 64) == "sgemm_mfma_dma"         # 4 steps per tile
    assert kname_ws(lib, "f32", 4095, 4097, 1001, nbytes=1 << 20) == "sgemm_mfma"
    # at most 16 rows of C with a row-major (N-contiguous) 16-bit B: split-K
    # across workgroups with a fixed-order reduction; a K-contiguous B keeps
    # the skinny kernel (whole lines already), and so do short K or narrow N
    assert kname_ws(lib, "bf16", 16, 4096, 4096) == "gemm_skinny_splitk"
    assert kname_ws(lib, "f16", 1, 4096, 4096) == "gemm_skinny_splitk"
    assert kname_ws(lib, "bf16", 7, 1000, 2048, batch=3) == "gemm_skinny_splitk"
    assert kname_ws(lib, "bf16", 16, 4096, 4096, ob=1) == "gemm_skinny"
    assert kname_ws(lib, "bf16", 16, 4096, 512) == "gemm_skinny"
    assert kname_ws(lib, "bf16", 16, 200, 4096) == "gemm_skinny"
    assert kname_ws(lib, "bf16", 16, 4096, 4096, ws=0, nbytes=0) == "gemm_skinny"
    assert kname_ws(lib, "f32", 16, 4096, 4096) == "sgemm_splitk"
    # K = 0 scales C
    assert kname_ws(lib, "bf16", 4095, 4097, 0, lda=1) == "scale"
    clean_env(lib.TEST_FORCE_GENERAL)
    assert kname_ws(lib, "bf16", 4095, 4097, 1001) == "hgemm_mfma"


def test_workspace_invalid_arguments(lib):
    n = lib.workspace_size()
    assert kname_ws(lib, "bf16", 4095, 4097, 1001, ws=0, nbytes=n) is None       # NULL
    assert kname_ws(lib, "bf16", 4095, 4097, 1001, ws=WS + 16) is None           # misaligned
    assert kname_ws(lib, "bf16", 4095, 4097, 1001, ws=3 * GB - 256) is None      # overlaps C
    assert kname_ws(lib, "bf16", 4095, 4097, 1001, ws=GB + 1024) is None         # overlaps A
    args = (8, 8, 8, 1.0, P, 8, 0, P * 3, 8, 0, 0.0, P * 5, 8, 0, 0, 1, 0, 0, 0)
    for fn in (lib.gemm_bf16_ws, lib.gemm_f16_ws):
        assert fn(*args, 0, n, 0, raise_on_error=False) == lib.ERR_INVALID_ARG
        assert fn(*args, P * 5 - 256, n, 0, raise_on_error=False) == lib.ERR_INVALID_ARG  # over C
        assert fn(-1, *args[1:], WS, n, 0, raise_on_error=False) == lib.ERR_INVALID_ARG
        assert fn(0, *args[1:], WS, n, 0, raise_on_error=False) == lib.OK
        assert fn(*args[:14], 2, *args[15:], WS, n, 0, raise_on_error=False) == lib.ERR_INVALID_ARG
    # gemm_f32_ws: the same checks (it has no c_dtype argument)
    f32args = args[:14] + args[15:]
    f = lib.gemm_f32_ws
    assert f(*f32args, 0, n, 0, raise_on_error=False) == lib.ERR_INVALID_ARG              # NULL
    assert f(*f32args, WS + 16, n, 0, raise_on_error=False) == lib.ERR_INVALID_ARG        # misaligned
    assert f(*f32args, P * 5 - 256, n, 0, raise_on_error=False) == lib.ERR_INVALID_ARG    # over C
    assert f(*f32args, P * 3, n, 0, raise_on_error=False) == lib.ERR_INVALID_ARG          # over B
    assert f(-1, *f32args[1:], WS, n, 0, raise_on_error=False) == lib.ERR_INVALID_ARG
    assert f(0, *f32args[1:], WS, n, 0, raise_on_error=False) == lib.OK
    assert kname_ws(lib, "f32", 4095, 4097, 1001, ws=WS + 16) is None
    assert kname_ws(lib, "f32", 4095, 4097, 1001, ws=3 * GB - 256) is None


# ------------------------------------------------------------------ allocation-free entry point (host only)

def test_noalloc_refuses_calls_beyond_its_scratch(lib):
    # unaligned 300 x 290 x 8193: 4 tiles of 129 k-steps cut over 144
    # workgroups of the general kernel's stream-K schedule, whose partial
    # tiles (72 MiB) exceed the 64 MiB scratch: refused before any HIP call
    # (the pointers here are never dereferenced)
    args = (300, 290, 8193, 1.0, GB, 8193, 0, 2 * GB, 290, 0, 0.0, 3 * GB, 290, 0, 0, 1, 0, 0, 0)
    assert kname_ws(lib, "bf16", 300, 290, 8193) == "hgemm_mfma_streamk"
    assert lib.gemm_bf16_noalloc(*args, raise_on_error=False) == lib.ERR_SCRATCH
    assert lib.NOALLOC_SCRATCH_BYTES == 64 << 20
    # invalid arguments and empty problems are answered as by gemm_bf16
    assert lib.gemm_bf16_noalloc(-1, *args[1:], raise_on_error=False) == lib.ERR_INVALID_ARG
    assert lib.gemm_bf16_noalloc(*args[:14], 2, *args[15:], raise_on_error=False) == \
        lib.ERR_INVALID_ARG
    assert lib.gemm_bf16_noalloc(0, *args[1:], raise_on_error=False) == lib.OK


# ------------------------------------------------------------------ fp32 as three bf16 products

def kname_x3(lib, M, N, K, ws=WS, nbytes=None, **kw):
    oa, ob, oc = kw.pop("oa", 0), kw.pop("ob", 0), kw.pop("oc", 0)
    lda = kw.pop("lda", K if oa == 0 else M)
    ldb = kw.pop("ldb", N if ob == 0 else K)
    ldc = kw.pop("ldc", N if oc == 0 else M)
    batch = kw.pop("batch", 1)
    sa, sb = kw.pop("sa", M * K if batch > 1 else 0), kw.pop("sb", K * N if batch > 1 else 0)
    nbytes = lib.bf16x3_workspace_size(M, N, K, batch) if nbytes is None else nbytes
    return lib.kernel_name_bf16x3(M, N, K, kw.pop("alpha", 1.0), GB, lda, oa, 2 * GB, ldb, ob, 0.0,
                                  3 * GB, ldc, oc, batch, sa, sb, M * N if batch > 1 else 0,
                                  workspace=ws, workspace_bytes=nbytes)


def test_bf16x3_workspace_size(lib):
    # two bf16 copies of 3 Kp (K rounded up to a multiple of 8) per row of A
    # and per column of B, each rounded up to 256 bytes
    assert lib.bf16x3_workspace_size(4096, 4096, 4096, 1) == 2 * 4096 * 3 * 4096 * 2
    assert lib.bf16x3_workspace_size(100, 30, 1001, 1) == \
        -(-100 * 3 * 1008 * 2 // 256) * 256 + -(-30 * 3 * 1008 * 2 // 256) * 256
    assert lib.bf16x3_workspace_size(8, 8, 8, 3) == 2 * 1280     # 3 x 8 x 24 x 2 = 1152, to 256
    assert lib.bf16x3_workspace_size(0, 8, 8, 1) == 512   # B's copy: 8 x 24 x 2 bytes, to 256
    assert lib.bf16x3_workspace_size(-1, 8, 8, 1) == 0
    assert lib.bf16x3_workspace_size(1 << 40, 1 << 40, 1 << 40, 1) == 0   # overflows


def test_bf16x3_kernel_choice(lib, clean_env):
    # the bf16 kernel on the split copies (K-contiguous, 16-byte aligned,
    # K' = 3 * Kp): the same choice as a bf16 problem of that K'
    assert kname_x3(lib, 4096, 4096, 4096) == "hgemm_mfma_dma"
    assert kname_x3(lib, 4095, 4097, 1001, oa=1, ob=1) == "hgemm_mfma_dma"   # any layout copies aligned
    assert kname_x3(lib, 16, 4096, 4096) == "gemm_skinny"
    assert kname_x3(lib, 4096, 16, 4096, oc=1) == "gemm_skinny"             # C^T has 16 rows
    assert kname_x3(lib, 256, 256, 256) == "hgemm_splitk"                  # K' = 768
    assert kname_x3(lib, 256, 256, 128) == "hgemm_mfma_dma"                # K' = 384: too short to split
    assert kname_x3(lib, 520, 264, 200, batch=3, sb=0) == "hgemm_splitk"   # 18 tiles, K' = 600
    # nothing to multiply: gemm_f32's quick paths, workspace not needed
    assert kname_x3(lib, 4096, 4096, 4096, alpha=0.0, ws=0, nbytes=0) == "scale"
    assert kname_x3(lib, 4096, 4096, 0, lda=1, ws=0, nbytes=0) == "scale"
    assert kname_x3(lib, 0, 4096, 4096, ws=0, nbytes=0) == ""
    clean_env(lib.TEST_NO_SPLITK)
    assert kname_x3(lib, 256, 256, 256) == "hgemm_mfma_dma"


def test_bf16x3_invalid_workspace(lib):
    n = lib.bf16x3_workspace_size(520, 264, 200, 1)
    assert kname_x3(lib, 520, 264, 200) is not None
    assert kname_x3(lib, 520, 264, 200, nbytes=n - 1) is None               # too small
    assert kname_x3(lib, 520, 264, 200, ws=0) is None                       # NULL
    assert kname_x3(lib, 520, 264, 200, ws=WS + 16) is None                 # not 256-byte aligned
    assert kname_x3(lib, 520, 264, 200, ws=GB + 256) is None                # overlaps A
    assert kname_x3(lib, 520, 264, 200, ws=3 * GB - 256) is None            # overlaps C
    assert kname_x3(lib, 520, 264, 200, lda=100) is None                    # lda < K
    # a broadcast operand is copied once: A's one copy (520 x 600 x 2 bytes,
    # to 256) and B's four
    need = 624128 + 4 * 520 * 600 * 2
    assert kname_x3(lib, 520, 520, 200, batch=4, sa=0, nbytes=need) is not None
    assert kname_x3(lib, 520, 520, 200, batch=4, sa=0, nbytes=need - 1) is None
    assert kname_x3(lib, 520, 520, 200, batch=4, nbytes=need) is None


# ------------------------------------------------------------------ quantised (8-bit) output

def kname_q(lib, dt, M, N, K, fmt="e4m3", **kw):
    oa, ob, oc = kw.pop("oa", 0), kw.pop("ob", 0), kw.pop("oc", 0)
    lda = kw.pop("lda", K if oa == 0 else M)
    ldb = kw.pop("ldb", N if ob == 0 else K)
    ldc = kw.pop("ldc", N if oc == 0 else M)
    return lib.kernel_name_quant(dt, M, N, K, kw.pop("alpha", 1.0), kw.pop("A", GB), lda, oa,
                                 kw.pop("B", 2 * GB), ldb, ob, kw.pop("C", 3 * GB), ldc, oc, fmt,
                                 kw.pop("batch", 1), kw.pop("sa", 0), kw.pop("sb", 0),
                                 kw.pop("sc", 0))


def test_quant_kernel_choice(lib, clean_env):
    # always the 16-bit direct-load kernel (no split-K or skinny variant of
    # the 8-bit store), in any order; the scale kernel when nothing is multiplied
    assert kname_q(lib, "bf16", 4096, 4096, 4096) == "hgemm_mfma_dma"
    assert kname_q(lib, "f16", 4096, 4096, 4096, "e5m2", oa=1, ob=1, oc=1) == "hgemm_mfma_dma"
    assert kname_q(lib, "bf16", 16, 4096, 4096) == "hgemm_mfma_dma"
    assert kname_q(lib, "bf16", 256, 256, 8192) == "hgemm_mfma_dma"
    # C needs no alignment (bytes; ldc = 4095)
    assert kname_q(lib, "bf16", 4096, 4095, 4096, ob=1, C=3 * GB + 1) == "hgemm_mfma_dma"
    assert kname_q(lib, "bf16", 4096, 4096, 4096, alpha=0.0) == "scale"
    assert kname_q(lib, "bf16", 4096, 4096, 0, lda=1) == "scale"
    assert kname_q(lib, "bf16", 0, 4096, 4096) == ""


def test_quant_unsupported_and_invalid(lib):
    # operands the direct-load kernel cannot read: GEMM_ERR_UNSUPPORTED, before
    # any HIP call (so these calls are safe without a GPU)
    def call(**kw):
        oa, ob = kw.pop("oa", 0), kw.pop("ob", 0)
        M, N, K = kw.pop("M", 4096), kw.pop("N", 4096), kw.pop("K", 4096)
        return lib.gemm_quant(kw.pop("dt", "bf16"), M, N, K, 1.0, kw.pop("A", GB),
                              kw.pop("lda", K if oa == 0 else M), oa, 2 * GB,
                              kw.pop("ldb", N if ob == 0 else K), ob, 3 * GB, N, 0,
                              kw.pop("fmt", "e4m3"), 1.0, raise_on_error=False)
    assert call(A=GB + 2) == -2                      # A not 16-byte aligned
    assert call(lda=4100) == -2                      # rows not 16-byte aligned
    assert call(K=4095, lda=4095) == -2              # K-contiguous extent not a multiple of 8
    assert call(dt="f16", oa=1, M=4095, lda=4095) == -2
    assert kname_q(lib, "bf16", 4096, 4096, 4096, A=GB + 2) is None
    assert call(lda=100) == -1                       # lda < K
    assert lib.library().gemm_bf16_quant(64, 64, 64, 1.0, GB, 64, 0, 2 * GB, 64, 0, 3 * GB, 64, 0,
                                         7, 1.0, 1, 0, 0, 0, None, 0, 0, None) == -1  # bad format
    assert call(dt="f16", fmt="e5m2", oa=1, ob=1, M=4095, N=4095, lda=4095) == -2


# ------------------------------------------------------------------ 8-bit and MX workspace entry points


def f8_ws(lib, M, N, K, ws=WS, nbytes=None, name=True, **kw):
    """gemm_f8_ws (name=False) or gemm_f8_kernel_name_ws with fake addresses:
    E4M3 x E5M2, row-major A, column-major B (both K-contiguous), bf16 C."""
    oa, ob = kw.pop("oa", 0), kw.pop("ob", 1)
    lda = kw.pop("lda", K if oa == 0 else M)
    ldb = kw.pop("ldb", N if ob == 0 else K)
    batch = kw.pop("batch", 1)
    strides = (M * K, K * N, M * N) if batch > 1 else (0, 0, 0)
    C = kw.pop("C", 3 * GB)
    nbytes = lib.workspace_size() if nbytes is None else nbytes
    args = (M, N, K, kw.pop("alpha", 1.0), GB, lda, oa, lib.F8_E4M3, 2 * GB, ldb, ob,
            lib.F8_E5M2, 0.0, C, N, 0, lib.OUTPUT_BF16, batch, *strides)
    assert not kw, kw
    if name:
        return lib.f8_kernel_name(*args, workspace=ws, workspace_bytes=nbytes)
    return lib.gemm_f8_ws(*args, ws, nbytes, raise_on_error=False)


def test_f8_streamk_kernel_choice(lib, clean_env):
    # 272 tiles of 32 k steps (128 k each): the cut tail pays for its exchange
    assert f8_ws(lib, 4096, 4352, 4096) == "f8gemm_mfma_dma_streamk"
    assert f8_ws(lib, 4096, 4352, 4096, batch=2) == "f8gemm_mfma_dma"   # 544 tiles: nearly full
    assert f8_ws(lib, 4096, 4096, 4096) == "f8gemm_mfma_dma"            # whole waves
    assert f8_ws(lib, 4096, 4352, 512) == "f8gemm_mfma_dma"             # 4 steps per tile
    assert f8_ws(lib, 2048, 2304, 1024) == "f8gemm_mfma_dma"            # 72 tiles of 8 steps
    # no workspace, or one that is too small: the plain kernel
    assert f8_ws(lib, 4096, 4352, 4096, ws=0, nbytes=0) == "f8gemm_mfma_dma"
    assert f8_ws(lib, 4096, 4352, 4096, nbytes=1 << 20) == "f8gemm_mfma_dma"
    assert lib.f8_kernel_name(4096, 4352, 4096, 1.0, GB, 4096, 0, 0, 2 * GB, 4096, 1, 1, 0.0,
                              3 * GB, 4352, 0, 1) == "f8gemm_mfma_dma"
    # operands the direct-load kernel cannot read keep the general kernel
    assert f8_ws(lib, 4096, 4352, 4096, ob=0) == "f8gemm_mfma"
    assert f8_ws(lib, 4096, 4352, 4104, lda=4104, ldb=4104) == "f8gemm_mfma"
    clean_env(lib.TEST_FORCE_STREAMK)
    assert f8_ws(lib, 2048, 2304, 1024) == "f8gemm_mfma_dma_streamk"
    assert f8_ws(lib, 4096, 4352, 512) == "f8gemm_mfma_dma_streamk"
    assert f8_ws(lib, 4096, 4096, 4096) == "f8gemm_mfma_dma"            # nothing to cut
    assert f8_ws(lib, 4096, 4352, 4096, ob=0) == "f8gemm_mfma"
    clean_env(lib.TEST_FORCE_GENERAL)
    assert f8_ws(lib, 4096, 4352, 4096) == "f8gemm_mfma"


def test_f8_ws_invalid_workspace(lib):
    assert f8_ws(lib, 4096, 4352, 4096, ws=WS + 8) is None              # not 256-byte aligned
    assert f8_ws(lib, 4096, 4352, 4096, ws=0) is None                   # NULL with bytes
    assert f8_ws(lib, 4096, 4352, 4096, ws=2 * GB) is None              # overlaps B
    assert f8_ws(lib, 4096, 4352, 4096, C=WS + 4096) is None            # C inside it
    for kw in (dict(ws=WS + 8), dict(ws=0), dict(ws=GB + 256)):
        assert f8_ws(lib, 4096, 4352, 4096, name=False, **kw) == lib.ERR_INVALID_ARG, kw
    # a format or output type out of range
    assert lib.gemm_f8_ws(8, 8, 8, 1.0, GB, 8, 0, 2, 2 * GB, 8, 1, 0, 0.0, 3 * GB, 8, 0, 1, 1, 0,
                          0, 0, WS, lib.workspace_size(), raise_on_error=False) == lib.ERR_INVALID_ARG
    assert f8_ws(lib, 0, 4352, 4096, name=False) == lib.OK              # empty: nothing launched


def mx_ws(lib, ws=WS, nbytes=None, **kw):
    """gemm_mx_kernel_name_ws (name=True, default) or gemm_mx_ws for an MXFP4
    problem, 4096 x 4352 x 4096 unless given, bf16 C, with fake addresses 4
    GiB apart: A at GB, its scales at 2 GB, B at 3 GB, B's scales at 4 GB, C
    at 6 GB (the workspace WS sits at 5 GB)."""
    M, N, K = kw.pop("M", 4096), kw.pop("N", 4352), kw.pop("K", 4096)
    name = kw.pop("name", True)
    sb = 4 * (-(-K // 128))
    args = (M, N, K, 1.0, GB, K, 4, 2 * GB, sb, 3 * GB, K, 4, 4 * GB, sb, 0.0, 6 * GB, N, 0, 1, 1,
            0, 0, 0, 0, 0)
    assert not kw, kw
    nbytes = lib.workspace_size() if nbytes is None else nbytes
    if name:
        return lib.mx_kernel_name(*args, workspace=ws, workspace_bytes=nbytes)
    return lib.gemm_mx_ws(*args, ws, nbytes, raise_on_error=False)


def test_mx_streamk_kernel_choice(lib, clean_env):
    assert mx_ws(lib) == "mxgemm_mfma_dma_streamk"                      # 272 tiles, 32 steps
    assert mx_ws(lib, N=4096) == "mxgemm_mfma_dma"                      # whole waves
    assert mx_ws(lib, K=512) == "mxgemm_mfma_dma"                       # 4 steps per tile
    assert mx_ws(lib, ws=0, nbytes=0) == "mxgemm_mfma_dma"
    assert mx_ws(lib, nbytes=1 << 20) == "mxgemm_mfma_dma"
    clean_env(lib.TEST_FORCE_STREAMK)
    assert mx_ws(lib, M=300, N=260, K=256) == "mxgemm_mfma_dma_streamk"
    assert mx_ws(lib, K=512) == "mxgemm_mfma_dma_streamk"
    assert mx_ws(lib, N=4096) == "mxgemm_mfma_dma"                      # nothing to cut
    clean_env(lib.TEST_FORCE_GENERAL)
    assert mx_ws(lib) == "mxgemm_mfma_dma"                              # one workgroup per tile


def test_mx_ws_invalid_workspace(lib):
    # misaligned, NULL with bytes, and overlapping A, A's scales, B, B's
    # scales or C
    for ws in (WS + 4, 0, GB + 256, 2 * GB, 3 * GB + 4096, 4 * GB, 6 * GB + 512):
        assert mx_ws(lib, ws=ws) is None, ws
        assert mx_ws(lib, ws=ws, name=False) == lib.ERR_INVALID_ARG, ws
    # without a workspace NULL is fine
    assert mx_ws(lib, ws=0, nbytes=0) == "mxgemm_mfma_dma"
