"""Pins for the CPU oracle, against things other than the oracle itself.

Each test checks the oracle against a fact fixed by mathematics or by an
independent library routine: exact rational arithmetic on tiny problems,
closed forms (identity, permutation, all-ones, rank-1), numpy's own float16
and float32 conversions, exhaustive decoding of every 16-bit pattern, layout
and batch invariants, and a hand-worked example of the definition.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import COL, ROW

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -53  # unit roundoff of double


# --------------------------------------------------------------- independent helpers

def np_decode(dtype, bits):
    """Decode stored patterns with numpy only (independent of the oracle)."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return np.asarray(bits, np.float32).astype(np.float64) if bits.dtype != np.uint32 \
            else bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rne_fraction(x: Fraction, p: int, emin: int, emax: int) -> float:
    """Exact round-to-nearest-even of a rational to a p-bit binary format."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - p + 1)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    if r > (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax:
        return sign * math.inf
    return sign * float(r)


FORMATS = {"bf16": (8, -126, 127), "f16": (11, -14, 15), "f32": (24, -126, 127)}


def rand_bits(rng, dtype, n, scale=1.0):
    if dtype in ("e4m3", "e5m2"):
        # any finite pattern: E4M3 S.1111.111 is NaN, E5M2 exponent 31 is Inf/NaN
        b = rng.integers(0, 256, n).astype(np.uint8)
        bad = (b & 0x7F) == 0x7F if dtype == "e4m3" else ((b >> 2) & 0x1F) == 0x1F
        return np.where(bad, b & 0xF3, b).astype(np.uint8)
    x = rng.standard_normal(n) * scale
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    f = x.astype(np.float32).view(np.uint32)
    return (f >> 16).astype(np.uint16)  # truncation is fine: any pattern is a valid input


def stored(dtype, values):
    """Exactly representable small values -> stored patterns."""
    v = np.asarray(values, np.float64)
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def put(mat, order, ld=None):
    """Store a 2-D float array in row- or column-major order with leading dim ld."""
    r, c = mat.shape
    if order == ROW:
        ld = ld or c
        out = np.zeros(max(0, (r - 1) * ld + c) if r and c else 0, mat.dtype)
        for i in range(r):
            out[i * ld:i * ld + c] = mat[i]
    else:
        ld = ld or r
        out = np.zeros(max(0, (c - 1) * ld + r) if r and c else 0, mat.dtype)
        for j in range(c):
            out[j * ld:j * ld + r] = mat[:, j]
    return out, ld


# --------------------------------------------------------------- decoding / rounding

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_every_16bit_pattern(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(dtype, bits)
    want = np_decode(dtype, bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def _round_cases(rng):
    x = np.concatenate([
        rng.standard_normal(20000),
        rng.standard_normal(5000) * 1e-6,
        rng.standard_normal(5000) * 1e4,
        np.ldexp(rng.uniform(1, 2, 2000), rng.integers(-160, 140, 2000)),
    ])
    return x


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(1)
    x = _round_cases(rng)
    # exact ties between neighbouring f16 values, and ties nudged by 2^-40
    base = rng.standard_normal(4000).astype(np.float16).astype(np.float64)
    ulp = np.spacing(base.astype(np.float16)).astype(np.float64)
    ties = base + ulp / 2
    x = np.concatenate([x, ties, ties + np.abs(ties) * 2.0 ** -40, ties - np.abs(ties) * 2.0 ** -40,
                        [65504.0, 65519.99, 65520.0, 1e6, -7e4, 2.0 ** -24, 2.0 ** -25,
                         3 * 2.0 ** -26, 0.0, -0.0]])
    got = oracle.round_bits("f16", x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(2)
    x = _round_cases(rng)
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(oracle.round_bits("f32", x), want)


def test_round_bf16_matches_exact_rational():
    rng = np.random.default_rng(3)
    x = np.concatenate([_round_cases(rng)[:6000],
                        # ties of bf16 (1 + 2^-8) and ties nudged below float's resolution,
                        # which a double -> float -> bf16 path would round the wrong way
                        [1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8,
                         -(1 + 2.0 ** -8 + 2.0 ** -40), 3.3895313892515355e38, 3.4e38,
                         2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135]])
    got = oracle.decode("bf16", oracle.round_bits("bf16", x))
    p, emin, emax = FORMATS["bf16"]
    want = np.array([rne_fraction(Fraction(v), p, emin, emax) for v in x])
    assert np.array_equal(got, want)
    # the nudged tie rounds up, the exact tie rounds to even (down)
    assert got[6000] == 1.0 and got[6001] == 1 + 2.0 ** -7


def test_round_bf16_agrees_with_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x32 = rng.standard_normal(50000).astype(np.float32) * 3
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bits("bf16", x32.astype(np.float64))
    assert np.array_equal(got, want)


# --------------------------------------------------------------- brute force, exact rationals

def exact_problem(rng, dtype, c_dtype, M, N, K, oA, oB, oC, alpha, beta, batch, bcast):
    A_mats = [rand_bits(rng, dtype, M * K).reshape(M, K) for _ in range(batch)]
    B_mats = [rand_bits(rng, dtype, K * N).reshape(K, N) for _ in range(batch)]
    C_mats = [rand_bits(rng, c_dtype, M * N).reshape(M, N) for _ in range(batch)]
    if bcast == "a":
        A_mats = [A_mats[0]] * batch
    if bcast == "b":
        B_mats = [B_mats[0]] * batch

    def pack(mats, order, ld_pad, bc):
        bufs, ld = [], None
        for m in mats[:1] if bc else mats:
            buf, ld = put(m, order, (m.shape[1] if order == ROW else m.shape[0]) + ld_pad)
            bufs.append(buf)
        stride = 0 if bc else bufs[0].size + 3
        total = np.zeros(stride * (len(bufs) - 1) + bufs[0].size, bufs[0].dtype)
        for b, buf in enumerate(bufs):
            total[b * stride:b * stride + buf.size] = buf
        return total, ld, stride

    A, lda, sA = pack(A_mats, oA, 2, bcast == "a")
    B, ldb, sB = pack(B_mats, oB, 1, bcast == "b")
    C, ldc, sC = pack(C_mats, oC, 0, False)
    ref, den = oracle.gemm(dtype, c_dtype, M, N, K, alpha, A, lda, oA, B, ldb, oB, beta, C, ldc,
                           oC, batch=batch, stride_a=sA, stride_b=sB, stride_c=sC)
    fa, fb, fc = (lambda m: np_decode(dtype, m)), (lambda m: np_decode(dtype, m)), \
        (lambda m: np_decode(c_dtype, m))
    exact = np.empty((batch, M, N), object)
    scale = np.empty((batch, M, N), object)
    for b in range(batch):
        a, bb, c = fa(A_mats[b]), fb(B_mats[b]), fc(C_mats[b])
        for i in range(M):
            for j in range(N):
                terms = [Fraction(a[i, k]) * Fraction(bb[k, j]) for k in range(K)]
                s = Fraction(alpha) * sum(terms, Fraction(0))
                t = abs(Fraction(alpha)) * sum((abs(x) for x in terms), Fraction(0))
                if beta != 0:
                    s += Fraction(beta) * Fraction(c[i, j])
                    t += abs(Fraction(beta)) * abs(Fraction(c[i, j]))
                exact[b, i, j], scale[b, i, j] = s, t
    return ref, den, exact, scale


CASES = []
_r = np.random.default_rng(7)
for n in range(60):
    dt = ["f32", "bf16", "f16"][n % 3]
    CASES.append(dict(
        seed=100 + n, dtype=dt, c_dtype=dt if n % 4 else "f32",
        M=int(_r.integers(1, 7)), N=int(_r.integers(1, 7)), K=int(_r.integers(1, 9)),
        oA=int(_r.integers(0, 2)), oB=int(_r.integers(0, 2)), oC=int(_r.integers(0, 2)),
        alpha=float([1.0, 0.5, -1.75, 3.0][n % 4]), beta=float([0.0, 1.0, -0.25, 2.0][(n // 4) % 4]),
        batch=int(_r.integers(1, 4)), bcast=["", "a", "b", ""][n % 4]))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['dtype']}-{c['M']}x{c['N']}x{c['K']}-"
                         f"o{c['oA']}{c['oB']}{c['oC']}-b{c['batch']}{c['bcast']}-s{c['seed']}")
def test_oracle_vs_exact_rationals(case):
    rng = np.random.default_rng(case["seed"])
    K = case["K"]
    ref, den, exact, scale = exact_problem(
        rng, case["dtype"], case["c_dtype"], case["M"], case["N"], K, case["oA"], case["oB"],
        case["oC"], case["alpha"], case["beta"], case["batch"], case["bcast"])
    bound = (K + 3) * U
    for idx in np.ndindex(ref.shape):
        ex, sc = exact[idx], scale[idx]
        assert abs(Fraction(ref[idx]) - ex) <= Fraction(bound) * sc, idx
        assert abs(Fraction(den[idx]) - sc) <= Fraction(bound) * sc, idx
    # 16-bit results: rounding the double result gives the exact result's rounding
    for dt in ("bf16", "f16"):
        p, emin, emax = FORMATS[dt]
        q = oracle.decode(dt, oracle.round_bits(dt, ref))
        for idx in np.ndindex(ref.shape):
            want = rne_fraction(exact[idx], p, emin, emax)
            if q[idx] != want:
                # only allowed when the exact value sits within the error bound of a tie
                lo, hi = sorted([q[idx], want])
                mid = (Fraction(lo) + Fraction(hi)) / 2
                assert abs(mid - exact[idx]) <= Fraction(bound) * scale[idx], idx


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_2x2.json")))
    A = np.array(g["A"], np.float32).ravel()
    B = np.array(g["B"], np.float32).ravel()
    C0 = np.array(g["C0"], np.float32).ravel()
    ref, den = oracle.gemm("f32", "f32", 2, 2, 2, g["alpha"], A, 2, ROW, B, 2, ROW, g["beta"], C0,
                           2, ROW)
    assert np.array_equal(ref[0], np.array(g["C"], np.float64))
    assert np.array_equal(den[0], np.array(g["abs_scale"], np.float64))


# --------------------------------------------------------------- closed forms

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_identity(dtype):
    rng = np.random.default_rng(11)
    M = N = 13
    A = stored(dtype, np.eye(M))
    B = rand_bits(rng, dtype, M * N)
    C0 = rand_bits(rng, dtype, M * N)
    ref, _ = oracle.gemm(dtype, dtype, M, N, M, 1.0, A, M, ROW, B, N, ROW, 0.0, C0, N, ROW)
    assert np.array_equal(ref[0].ravel(), np_decode(dtype, B))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_permutation(dtype):
    rng = np.random.default_rng(12)
    M, N = 17, 9
    perm = rng.permutation(M)
    P = np.zeros((M, M))
    P[np.arange(M), perm] = 1.0
    B = rand_bits(rng, dtype, M * N)
    ref, _ = oracle.gemm(dtype, dtype, M, N, M, 1.0, stored(dtype, P.ravel()), M, ROW, B, N, ROW,
                         0.0, None, N, ROW)
    assert np.array_equal(ref[0], np_decode(dtype, B).reshape(M, N)[perm])


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_all_ones_closed_form(dtype):
    # every C_ij = K*alpha + beta*C0_ij, exactly (all values small integers / halves)
    rng = np.random.default_rng(13)
    M, N, K = 7, 11, 300
    alpha, beta = 1.5, -2.0
    c0 = rng.integers(-8, 9, M * N).astype(np.float64)
    ref, den = oracle.gemm(dtype, dtype, M, N, K, alpha, stored(dtype, np.ones(M * K)), K, ROW,
                           stored(dtype, np.ones(K * N)), N, ROW, beta, stored(dtype, c0), N, ROW)
    assert np.array_equal(ref[0].ravel(), K * alpha + beta * c0)
    assert np.array_equal(den[0].ravel(), K * abs(alpha) + abs(beta) * np.abs(c0))


def test_rank_one_closed_form():
    rng = np.random.default_rng(14)
    M, N, K = 9, 10, 57
    a = rng.integers(-5, 6, M).astype(np.float64)
    b = rng.integers(-5, 6, N).astype(np.float64)
    A = np.repeat(a[:, None], K, axis=1)
    B = np.repeat(b[None, :], K, axis=0)
    ref, _ = oracle.gemm("f32", "f32", M, N, K, 1.0, stored("f32", A.ravel()), K, ROW,
                         stored("f32", B.ravel()), N, ROW, 0.0, None, N, ROW)
    assert np.array_equal(ref[0], K * np.outer(a, b))


def test_integer_product_matches_int64_matmul():
    # integer entries keep every double operation exact, so the oracle must equal the
    # exact integer product (numpy int64 matmul) for any shape and layout
    rng = np.random.default_rng(15)
    M, N, K = 23, 31, 45
    A = rng.integers(-8, 9, (M, K))
    B = rng.integers(-8, 9, (K, N))
    want = (A @ B).astype(np.float64)
    for oA in (ROW, COL):
        for oB in (ROW, COL):
            Ab, lda = put(A.astype(np.float32), oA, (K if oA == ROW else M) + 5)
            Bb, ldb = put(B.astype(np.float32), oB)
            ref, _ = oracle.gemm("f32", "f32", M, N, K, 1.0, Ab, lda, oA, Bb, ldb, oB, 0.0, None,
                                 N, ROW)
            assert np.array_equal(ref[0], want), (oA, oB)


def test_close_to_numpy_float64_matmul():
    rng = np.random.default_rng(16)
    M, N, K = 33, 47, 61
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    ref, den = oracle.gemm("f32", "f32", M, N, K, 1.0, A.ravel(), K, ROW, B.ravel(), N, ROW, 0.0,
                           None, N, ROW)
    want = A.astype(np.float64) @ B.astype(np.float64)
    assert np.all(np.abs(ref[0] - want) <= 2 * K * U * den[0])
    assert np.allclose(den[0], np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)),
                       rtol=4 * K * U, atol=0)


# --------------------------------------------------------------- layout, batch, quick returns

def test_layouts_give_identical_doubles():
    rng = np.random.default_rng(17)
    M, N, K = 12, 19, 33
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    base = None
    for oA in (ROW, COL):
        for oB in (ROW, COL):
            for oC in (ROW, COL):
                Ab, lda = put(A, oA, None)
                Bb, ldb = put(B, oB, None)
                Cb, ldc = put(C, oC, None)
                ref, den = oracle.gemm("f32", "f32", M, N, K, 0.75, Ab, lda, oA, Bb, ldb, oB,
                                       -1.25, Cb, ldc, oC)
                if base is None:
                    base = (ref, den)
                assert np.array_equal(ref, base[0]) and np.array_equal(den, base[1])


def test_batch_slices_equal_single_calls():
    rng = np.random.default_rng(18)
    M, N, K, batch = 6, 5, 7, 4
    A = rng.uniform(-1, 1, batch * M * K).astype(np.float32)
    B = rng.uniform(-1, 1, K * N).astype(np.float32)  # broadcast: stride 0
    C = rng.uniform(-1, 1, batch * M * N).astype(np.float32)
    ref, den = oracle.gemm("f32", "f32", M, N, K, 1.0, A, K, ROW, B, N, ROW, 0.5, C, N, ROW,
                           batch=batch, stride_a=M * K, stride_b=0, stride_c=M * N)
    for b in range(batch):
        r1, d1 = oracle.gemm("f32", "f32", M, N, K, 1.0, A[b * M * K:(b + 1) * M * K], K, ROW, B,
                             N, ROW, 0.5, C[b * M * N:(b + 1) * M * N], N, ROW)
        assert np.array_equal(ref[b], r1[0]) and np.array_equal(den[b], d1[0])


def test_gemm_at_matches_full():
    rng = np.random.default_rng(19)
    M, N, K, batch = 9, 8, 10, 3
    A = rand_bits(rng, "bf16", batch * M * K)
    B = rand_bits(rng, "bf16", batch * K * N)
    C = rand_bits(rng, "bf16", batch * M * N)
    kw = dict(stride_a=M * K, stride_b=K * N, stride_c=M * N)
    ref, den = oracle.gemm("bf16", "bf16", M, N, K, 2.0, A, M, COL, B, N, ROW, 1.0, C, N, ROW,
                           batch=batch, **kw)
    idx = np.stack([rng.integers(0, batch, 50), rng.integers(0, M, 50), rng.integers(0, N, 50)], 1)
    r, d = oracle.gemm_at("bf16", "bf16", M, N, K, 2.0, A, M, COL, B, N, ROW, 1.0, C, N, ROW,
                          idx, **kw)
    assert np.array_equal(r, ref[idx[:, 0], idx[:, 1], idx[:, 2]])
    assert np.array_equal(d, den[idx[:, 0], idx[:, 1], idx[:, 2]])


PATHS = [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"), ("f16", "f16", "f32"),
         ("e4m3", "e5m2", "bf16"), ("e5m2", "e4m3", "f16")]


@pytest.mark.parametrize("ta,tb,tc", PATHS, ids=lambda x: str(x))
@pytest.mark.parametrize("orders", [(ROW, ROW, ROW), (COL, ROW, COL), (ROW, COL, ROW),
                                    (COL, COL, COL)], ids=lambda o: "%d%d%d" % o)
def test_full_matrix_path_equals_element_path(ta, tb, tc, orders):
    # orc_gemm (row blocks, i-k-j order over a decoded B) against orc_gemm_at
    # (one textbook dot product per element) on every element, bit for bit:
    # M not a multiple of the row block, padded leading dimensions, strided
    # batches, then a batch sharing one B, a bias and an activation
    rng = np.random.default_rng(23)
    oA, oB, oC = orders
    M, N, K, batch = 37, 29, 41, 3
    lda = (K if oA == ROW else M) + 3
    ldb = (N if oB == ROW else K) + 2
    ldc = (N if oC == ROW else M) + 1
    sA = lda * (M if oA == ROW else K) + 5
    sB = ldb * (K if oB == ROW else N) + 7
    sC = ldc * (M if oC == ROW else N) + 2
    A = rand_bits(rng, ta, batch * sA)
    B = rand_bits(rng, tb, batch * sB)
    C = rand_bits(rng, tc, batch * sC)
    bias = rand_bits(rng, ta, batch * N) if ta in ("f32", "bf16", "f16") else None
    idx = np.stack(np.meshgrid(np.arange(batch), np.arange(M), np.arange(N), indexing="ij"),
                   -1).reshape(-1, 3)
    for stride_b, act, alpha, beta, with_bias in ((sB, oracle.ACT_NONE, 0.75, 1.5, False),
                                                   (0, oracle.ACT_GELU, -2.0, 0.0, True),
                                                   (sB, oracle.ACT_RELU, 1.0, -0.5, True)):
        kw = dict(stride_a=sA, stride_b=stride_b, stride_c=sC, b_dtype=tb,
                  bias=bias if with_bias else None, stride_bias=N, act=act)
        ref, den = oracle.gemm(ta, tc, M, N, K, alpha, A, lda, oA, B, ldb, oB, beta, C, ldc, oC,
                               batch=batch, **kw)
        r, d = oracle.gemm_at(ta, tc, M, N, K, alpha, A, lda, oA, B, ldb, oB, beta, C, ldc, oC,
                              idx, **kw)
        assert np.array_equal(r.view(np.int64), ref.reshape(-1).view(np.int64))
        assert np.array_equal(d.view(np.int64), den.reshape(-1).view(np.int64))


def test_beta_zero_does_not_read_c():
    rng = np.random.default_rng(20)
    M, N, K = 4, 5, 6
    A = rng.uniform(-1, 1, M * K).astype(np.float32)
    B = rng.uniform(-1, 1, K * N).astype(np.float32)
    C = np.full(M * N, np.nan, np.float32)
    ref, den = oracle.gemm("f32", "f32", M, N, K, 1.0, A, K, ROW, B, N, ROW, 0.0, C, N, ROW)
    assert np.all(np.isfinite(ref)) and np.all(np.isfinite(den))


def test_alpha_zero_and_k_zero_scale_c_only():
    M, N, K = 4, 5, 6
    A = np.full(M * K, np.nan, np.float32)
    B = np.full(K * N, np.nan, np.float32)
    C = np.arange(M * N, dtype=np.float32) - 7
    ref, _ = oracle.gemm("f32", "f32", M, N, K, 0.0, A, K, ROW, B, N, ROW, -0.5, C, N, ROW)
    assert np.array_equal(ref[0].ravel(), -0.5 * C.astype(np.float64))
    ref, _ = oracle.gemm("f32", "f32", M, N, 0, 3.0, None, 1, ROW, None, N, ROW, 2.0, C, N, ROW)
    assert np.array_equal(ref[0].ravel(), 2.0 * C.astype(np.float64))


def test_page_throughput_figures_follow_2mnk():
    # the TFLOPS figures the pages print are 2*M*N*K / t; the benchmark uses the same count
    g = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    for e in g["entries"]:
        flop = 2 * e["M"] * e["N"] * e["K"]
        if "gflop" in e:
            assert abs(flop / 1e9 - e["gflop"]) <= e["gflop_rel_tol"] * e["gflop"], e["cite"]
        if "tflops" in e:
            assert abs(flop / e["time_s"] / 1e12 - e["tflops"]) <= e["tflops_rel_tol"] * e["tflops"], \
                e["cite"]


# --------------------------------------------------------------- fused epilogue

def one_by_one(x, act, bias=None, dtype="f32"):
    """A 1 x 1 x 1 product x * 1, so the value entering the epilogue is x exactly."""
    b = None if bias is None else stored(dtype, [bias])
    ref, den = oracle.gemm(dtype, dtype, 1, 1, 1, 1.0, stored(dtype, [x]), 1, ROW,
                           stored(dtype, [1.0]), 1, ROW, 0.0, None, 1, ROW, bias=b, act=act)
    return ref[0, 0, 0], den[0, 0, 0]


def test_gelu_matches_the_normal_table():
    table = json.load(open(os.path.join(GOLDEN, "normal_cdf.json")))
    for x, phi in table["phi"]:
        for xs, ph in ((x, phi), (-x, 1.0 - phi)):
            got, _ = one_by_one(xs, oracle.ACT_GELU)
            assert abs(got - xs * ph) <= 1e-14 * max(1.0, abs(xs)), (xs, got, xs * ph)
    assert one_by_one(0.0, oracle.ACT_GELU)[0] == 0.0
    # Phi(8) = 1 - 6.2e-16: GELU is the identity above and zero below, to double precision
    assert abs(one_by_one(8.0, oracle.ACT_GELU)[0] - 8.0) < 1e-13
    assert abs(one_by_one(-8.0, oracle.ACT_GELU)[0]) < 1e-13


def test_relu_of_x_then_bias_order():
    # the activation comes after the bias: relu(-1 + 2) = 1, not relu(-1) + 2 = 2
    assert one_by_one(-1.0, oracle.ACT_RELU, bias=2.0)[0] == 1.0
    assert one_by_one(-3.0, oracle.ACT_RELU, bias=2.0)[0] == 0.0
    assert one_by_one(3.0, oracle.ACT_RELU)[0] == 3.0
    assert one_by_one(-3.0, oracle.ACT_NONE, bias=2.0) == (-1.0, 5.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_bias_and_activations_on_integers_match_int64(dtype):
    # integer data keep every double operation exact: the oracle must equal
    # max(2*(A@B) + bias_j, 0) computed in int64, for bias broadcast along rows
    rng = np.random.default_rng(21)
    M, N, K = 13, 17, 29
    A = rng.integers(-6, 7, (M, K))
    B = rng.integers(-6, 7, (K, N))
    bias = rng.integers(-50, 51, N)
    pre = 2 * (A @ B) + bias[None, :]
    for act, want in ((oracle.ACT_NONE, pre), (oracle.ACT_RELU, np.maximum(pre, 0))):
        ref, den = oracle.gemm(dtype, dtype, M, N, K, 2.0, stored(dtype, A.ravel()), K, ROW,
                               stored(dtype, B.ravel()), N, ROW, 0.0, None, N, ROW,
                               bias=stored(dtype, bias), act=act)
        assert np.array_equal(ref[0], want.astype(np.float64)), act
        assert np.array_equal(den[0], (2 * (np.abs(A) @ np.abs(B)) + np.abs(bias)[None, :])
                              .astype(np.float64))


def test_bias_is_per_column_and_per_batch_entry():
    # A = 0: C = beta*C0 + bias_j; M != N so a bias indexed by the row would differ
    M, N, K, batch = 3, 5, 4, 2
    c0 = np.arange(batch * M * N, dtype=np.float64)
    bias = np.arange(batch * N, dtype=np.float64) * 10
    for stride in (N, 0):
        ref, den = oracle.gemm("f32", "f32", M, N, K, 1.0, stored("f32", np.zeros(M * K)), K, ROW,
                               stored("f32", np.zeros(K * N)), N, ROW, 0.5,
                               stored("f32", c0), N, ROW, batch=batch, stride_c=M * N,
                               bias=stored("f32", bias), stride_bias=stride)
        for b in range(batch):
            want = 0.5 * c0[b * M * N:(b + 1) * M * N].reshape(M, N) + \
                bias[b * stride:b * stride + N][None, :]
            assert np.array_equal(ref[b], want), (stride, b)


# --------------------------------------------------------------- 8-bit inputs

def torch_decode_8bit(dtype, bits):
    """Decode 8-bit patterns with torch's float8 types (independent of the oracle)."""
    import torch
    tdt = torch.float8_e4m3fn if dtype == "e4m3" else torch.float8_e5m2
    return torch.from_numpy(np.asarray(bits, np.uint8)).view(tdt).to(torch.float64).numpy()


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_decode_every_8bit_pattern(dtype):
    bits = np.arange(256, dtype=np.uint8)
    got = oracle.decode(dtype, bits)
    want = torch_decode_8bit(dtype, bits)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    # the format limits the pages' formats imply
    if dtype == "e4m3":
        assert np.nanmax(got) == 448.0 and np.isnan(got).sum() == 2 and not np.isinf(got).any()
    else:
        assert np.nanmax(got[~np.isinf(got)]) == 57344.0 and np.isinf(got).sum() == 2


# --------------------------------------------------------------- 8-bit outputs

F8_MAX = {"e4m3": (448.0, 0x7E, 0x7F), "e5m2": (57344.0, 0x7B, 0x7E)}  # max, its pattern, NaN


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_round_8bit_every_finite_pattern_round_trips(dtype):
    bits = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(dtype, bits)
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.round_bits(dtype, vals[fin]), bits[fin])


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_round_8bit_midpoints_go_to_even(dtype):
    bits = np.arange(0, 128, dtype=np.uint8)
    vals = oracle.decode(dtype, bits)
    fin = np.isfinite(vals)
    v, b = vals[fin], bits[fin]           # increasing, 0 .. max
    mid = (v[:-1] + v[1:]) / 2
    got = oracle.round_bits(dtype, mid)
    even = np.where(b[:-1] % 2 == 0, b[:-1], b[1:])
    assert np.array_equal(got, even)
    # a hair either side of a midpoint goes to the nearer neighbour
    eps = (v[1:] - v[:-1]) * 1e-6
    assert np.array_equal(oracle.round_bits(dtype, mid - eps), b[:-1])
    assert np.array_equal(oracle.round_bits(dtype, mid + eps), b[1:])
    # and the negative side mirrors it with the sign bit
    assert np.array_equal(oracle.round_bits(dtype, -mid), even | 0x80)


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_round_8bit_saturates(dtype):
    mx, pat, nan = F8_MAX[dtype]
    x = np.array([mx, mx * 1.0001, mx * 1.07, 1e30, np.inf, -mx * 3, -np.inf, np.nan, 0.0, -0.0])
    want = np.array([pat, pat, pat, pat, pat, pat | 0x80, pat | 0x80, nan, 0x00, 0x80], np.uint8)
    assert np.array_equal(oracle.round_bits(dtype, x), want)
    # below half the smallest subnormal: zero; at half: a tie, to even (zero)
    tiny = oracle.decode(dtype, np.array([1], np.uint8))[0]
    assert list(oracle.round_bits(dtype, np.array([tiny * 0.49, tiny * 0.5, tiny * 0.51, -tiny * 0.49]))) \
        == [0, 0, 1, 0x80]


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_round_8bit_agrees_with_torch_in_range(dtype):
    torch = pytest.importorskip("torch")
    mx = F8_MAX[dtype][0]
    rng = np.random.default_rng(9)
    x = (rng.uniform(-1, 1, 200000) * np.exp2(rng.integers(-22, 17, 200000))).astype(np.float32)
    x = x[np.abs(x) <= mx]                       # torch does not saturate: compare in range only
    tdt = torch.float8_e4m3fn if dtype == "e4m3" else torch.float8_e5m2
    want = torch.from_numpy(x).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(oracle.round_bits(dtype, x.astype(np.float64)), want)


def stored8(dtype, values):
    import torch
    tdt = torch.float8_e4m3fn if dtype == "e4m3" else torch.float8_e5m2
    t = torch.from_numpy(np.asarray(values, np.float32)).to(tdt)
    return t.view(torch.uint8).numpy()


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2"),
                                   ("e5m2", "e4m3")])
def test_8bit_integer_product_matches_int64(fa, fb):
    # integers of magnitude <= 7 are exact in both formats and every double
    # operation on them is exact: the oracle must equal the int64 product
    rng = np.random.default_rng(31)
    M, N, K = 19, 23, 41
    A = rng.integers(-7, 8, (M, K))
    B = rng.integers(-7, 8, (K, N))
    for oA, oB in ((ROW, COL), (ROW, ROW), (COL, ROW)):
        Ab, lda = put(stored8(fa, A), oA)
        Bb, ldb = put(stored8(fb, B), oB)
        ref, den = oracle.gemm(fa, "f32", M, N, K, 1.0, Ab, lda, oA, Bb, ldb, oB, 0.0, None, N,
                               ROW, b_dtype=fb)
        assert np.array_equal(ref[0], (A @ B).astype(np.float64)), (oA, oB)
        assert np.array_equal(den[0], (np.abs(A) @ np.abs(B)).astype(np.float64))


def test_8bit_formats_are_read_per_operand():
    # 0x3c is 1.5 in E4M3 and 1.0 in E5M2; a 1 x 1 x 1 product tells them apart
    a = np.array([0x3c], np.uint8)
    for fa, fb, want in (("e4m3", "e4m3", 2.25), ("e4m3", "e5m2", 1.5), ("e5m2", "e4m3", 1.5),
                         ("e5m2", "e5m2", 1.0)):
        ref, _ = oracle.gemm(fa, "f32", 1, 1, 1, 1.0, a, 1, ROW, a, 1, ROW, 0.0, None, 1, ROW,
                             b_dtype=fb)
        assert ref[0, 0, 0] == want, (fa, fb)


# --------------------------------------------------------------- block-scaled (MX) inputs

MX_WIDTH = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}


def mx_pack(fmt, patterns):
    """Pack element patterns (one per entry, low bits) into a little-endian
    bit stream of MX_WIDTH[fmt] bits per element."""
    w = MX_WIDTH[fmt]
    p = np.asarray(patterns, np.uint64).ravel()
    out = np.zeros((p.size * w + 7) // 8, np.uint8)
    for i, v in enumerate(p.tolist()):
        bit = i * w
        word = int(v) << (bit % 8)
        for b in range(bit // 8, (bit + w + 7) // 8):
            out[b] |= (word >> (8 * (b - bit // 8))) & 0xFF
    return out


def test_decode_every_e8m0_pattern_matches_torch():
    import torch
    bits = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e8m0", bits)
    want = torch.from_numpy(bits).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(got[255]) and np.isnan(want[255])
    assert np.array_equal(got[:255], want[:255])
    # bias 127: pattern 127 is 1; every step doubles
    assert got[127] == 1.0 and np.all(got[1:255] == 2 * got[:254])


def test_decode_e2m1_is_the_eight_listed_magnitudes():
    got = oracle.decode("e2m1", np.arange(16, dtype=np.uint8))
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert got[:8].tolist() == mags
    assert got[8:].tolist() == [-m for m in mags]
    assert math.copysign(1.0, got[8]) == -1.0  # pattern 0x8 is -0


@pytest.mark.parametrize("fmt,largest,min_normal,min_sub,within", [
    ("e2m3", 7.5, 1.0, 0.125, "e4m3"),
    ("e3m2", 28.0, 0.25, 0.0625, "e5m2"),
    ("e2m1", 6.0, 1.0, 0.5, "e2m3"),
])
def test_small_formats_extremes_order_and_containment(fmt, largest, min_normal, min_sub, within):
    n = 1 << MX_WIDTH[fmt]
    got = oracle.decode(fmt, np.arange(n, dtype=np.uint8))
    half = n // 2
    pos, neg = got[:half], got[half:]
    assert not np.isnan(got).any() and not np.isinf(got).any()
    assert np.array_equal(neg, -pos)
    assert np.all(np.diff(pos) > 0)  # patterns in increasing order of value
    assert pos.max() == largest and pos[1] == min_sub
    mbits = {"e2m3": 3, "e3m2": 2, "e2m1": 1}[fmt]
    assert pos[1 << mbits] == min_normal
    # every value is exactly a value of the wider format of the same family
    wider = oracle.decode(within, np.arange(256 if within in ("e4m3", "e5m2") else 64,
                                            dtype=np.uint8))
    assert set(pos.tolist()) <= set(wider[~np.isnan(wider)].tolist())


def test_mx_stream_bit_order():
    # E2M1: two per byte, the lower index in the low half: 0x21 holds
    # element 0 = 0x1 (0.5) and element 1 = 0x2 (1.0)
    s4 = np.array([0x21, 0xF7], np.uint8)
    assert [oracle.mx_element("e2m1", s4, i) for i in range(4)] == [0.5, 1.0, 6.0, -6.0]
    # E2M3: patterns 1, 2, 3, 4 as one 24-bit little-endian word
    # 1 | 2<<6 | 3<<12 | 4<<18 = 0x103081 -> bytes 81 30 10
    s6 = np.array([0x81, 0x30, 0x10], np.uint8)
    want = oracle.decode("e2m3", np.array([1, 2, 3, 4], np.uint8)).tolist()
    assert [oracle.mx_element("e2m3", s6, i) for i in range(4)] == want
    assert want == [0.125, 0.25, 0.375, 0.5]
    # the packer used by the tests agrees with the hand-written bytes
    assert mx_pack("e2m3", [1, 2, 3, 4]).tolist() == [0x81, 0x30, 0x10]
    assert mx_pack("e2m1", [1, 2, 7, 15]).tolist() == [0x21, 0xF7]
    # E4M3 elements are whole bytes
    assert oracle.mx_element("e4m3", np.array([0x00, 0x38], np.uint8), 1) == 1.0


def mx_int_operand(rng, fmt, rows, K):
    """rows x K integer-valued elements of fmt (magnitudes exact in every
    format), packed row by row, with their values."""
    pats = {"e2m1": {0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 6: 7},
            "e2m3": {0: 0, 1: 8, 2: 16, 3: 20, 4: 24, 6: 28, 7: 30},
            "e3m2": {0: 0, 1: 12, 2: 16, 3: 18, 4: 20, 6: 22, 7: 23},
            "e4m3": {0: 0, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 6: 0x4C, 7: 0x4E},
            "e5m2": {0: 0, 1: 0x3C, 2: 0x40, 3: 0x42, 4: 0x44, 6: 0x46, 7: 0x47}}[fmt]
    sign = {"e2m1": 8, "e2m3": 32, "e3m2": 32, "e4m3": 128, "e5m2": 128}[fmt]
    mags = np.array(sorted(pats))
    vals = rng.choice(mags, (rows, K)) * rng.choice([-1, 1], (rows, K))
    bits = np.array([[pats[abs(int(v))] | (sign if v < 0 else 0) for v in r] for r in vals])
    # check the table against the oracle's decoder once
    assert np.array_equal(oracle.decode(fmt, bits.astype(np.uint8).ravel()),
                          np.abs(vals).ravel() * np.sign(vals).ravel() + 0.0)
    return mx_pack(fmt, bits), vals


@pytest.mark.parametrize("fa,fb", [("e2m1", "e2m1"), ("e2m3", "e3m2"), ("e4m3", "e2m1"),
                                   ("e5m2", "e5m2"), ("e3m2", "e2m3")])
def test_mx_integer_products_with_scales_match_exact_arithmetic(fa, fb):
    rng = np.random.default_rng(41)
    M, N, K, batch = 5, 7, 96, 2
    A, va, SA, B, vb, SB = [], [], [], [], [], []
    for _ in range(batch):
        a, x = mx_int_operand(rng, fa, M, K)
        b, y = mx_int_operand(rng, fb, N, K)
        A.append(a); va.append(x); B.append(b); vb.append(y)
        SA.append(rng.integers(122, 133, (M, K // 32)).astype(np.uint8))
        SB.append(rng.integers(122, 133, (N, K // 32)).astype(np.uint8))
    bytes_a, bytes_b = A[0].size, B[0].size
    Af, Bf = np.concatenate(A), np.concatenate(B)
    SAf, SBf = np.concatenate([s.ravel() for s in SA]), np.concatenate([s.ravel() for s in SB])
    C0 = rng.integers(-5, 6, (batch, M, N)).astype(np.float32)
    ref, den = oracle.mx_gemm(fa, fb, "f32", M, N, K, 2.0, Af, K, SAf, K // 32, Bf, K, SBf,
                              K // 32, -1.0, C0.ravel(), N, ROW, batch=batch,
                              stride_a=bytes_a * 8 // MX_WIDTH[fa], stride_b=bytes_b * 8 // MX_WIDTH[fb],
                              stride_sa=M * K // 32, stride_sb=N * K // 32, stride_c=M * N)
    for b in range(batch):
        for i in range(M):
            for j in range(N):
                s = sum(Fraction(int(va[b][i, k]) * int(vb[b][j, k])) *
                        Fraction(2) ** (int(SA[b][i, k // 32]) + int(SB[b][j, k // 32]) - 254)
                        for k in range(K))
                assert ref[b, i, j] == float(2 * s - Fraction(float(C0[b, i, j])))
                t = sum(Fraction(abs(int(va[b][i, k]) * int(vb[b][j, k]))) *
                        Fraction(2) ** (int(SA[b][i, k // 32]) + int(SB[b][j, k // 32]) - 254)
                        for k in range(K))
                assert den[b, i, j] == float(2 * t + abs(Fraction(float(C0[b, i, j]))))


@pytest.mark.parametrize("f", ["e4m3", "e5m2"])
def test_mx_with_unit_scales_is_the_8bit_gemm(f):
    # every scale 127 (a factor of 1): the block-scaled product of 8-bit
    # elements is the plain 8-bit GEMM of A row-major and B column-major
    rng = np.random.default_rng(43)
    M, N, K = 9, 11, 128
    A = rng.integers(0, 256, (M, K)).astype(np.uint8)
    B = rng.integers(0, 256, (N, K)).astype(np.uint8)
    A[(A & 0x7F) >= (0x7F if f == "e4m3" else 0x7C)] = 0x11  # no NaN or Inf
    B[(B & 0x7F) >= (0x7F if f == "e4m3" else 0x7C)] = 0x22
    C0 = rng.standard_normal((M, N)).astype(np.float32)
    one = lambda r: np.full((r, K // 32), 127, np.uint8)
    ref, den = oracle.mx_gemm(f, f, "f32", M, N, K, 0.5, A, K, one(M), K // 32, B, K, one(N),
                              K // 32, 2.0, C0, N, ROW)
    ref8, den8 = oracle.gemm(f, "f32", M, N, K, 0.5, A, K, ROW, B, K, COL, 2.0, C0, N, ROW)
    assert np.array_equal(ref, ref8) and np.array_equal(den, den8)


def test_mx_scale_applies_to_its_32_element_block_only():
    # K = 96: three blocks; raising one block's scale by d multiplies that
    # block's share of the dot product by 2^d and leaves the others alone
    rng = np.random.default_rng(47)
    M, N, K = 3, 4, 96
    a, va = mx_int_operand(rng, "e2m1", M, K)
    b, vb = mx_int_operand(rng, "e2m1", N, K)
    SB = np.full((N, 3), 127, np.uint8)
    part = [(va[:, 32 * q:32 * q + 32] @ vb[:, 32 * q:32 * q + 32].T).astype(np.float64)
            for q in range(3)]
    for q in range(3):
        for d in (-3, 2):
            SA = np.full((M, 3), 127, np.uint8)
            SA[:, q] = 127 + d
            ref, _ = oracle.mx_gemm("e2m1", "e2m1", "f32", M, N, K, 1.0, a, K, SA, 3, b, K, SB, 3,
                                    0.0, None, N, ROW)
            want = sum(part) + (2.0 ** d - 1) * part[q]
            assert np.array_equal(ref[0], want), (q, d)
    # a scale on one row of A (or column of B) touches only that row (column)
    SA = np.full((M, 3), 127, np.uint8)
    SA[1, :] = 128
    SB2 = SB.copy()
    SB2[2, :] = 126
    ref, _ = oracle.mx_gemm("e2m1", "e2m1", "f32", M, N, K, 1.0, a, K, SA, 3, b, K, SB2, 3, 0.0,
                            None, N, ROW)
    want = sum(part) * np.outer([1, 2, 1], [1, 1, 0.5, 1])
    assert np.array_equal(ref[0], want)


def test_mx_nan_scale_poisons_only_its_rows_and_columns():
    rng = np.random.default_rng(53)
    M, N, K = 4, 5, 64
    a, _ = mx_int_operand(rng, "e2m3", M, K)
    b, _ = mx_int_operand(rng, "e2m3", N, K)
    SA = np.full((M, 2), 127, np.uint8)
    SB = np.full((N, 2), 127, np.uint8)
    SA[2, 1] = 255
    SB[3, 0] = 255
    ref, _ = oracle.mx_gemm("e2m3", "e2m3", "f32", M, N, K, 1.0, a, K, SA, 2, b, K, SB, 2, 0.0,
                            None, N, ROW)
    nan = np.isnan(ref[0])
    assert nan[2, :].all() and nan[:, 3].all() and nan.sum() == N + M - 1


def test_mx_gemm_at_and_leading_dimensions_match_full():
    rng = np.random.default_rng(59)
    M, N, K, lda, ldb = 6, 5, 128, 192, 160
    pa = rng.integers(0, 16, (M, lda))
    pb = rng.integers(0, 16, (N, ldb))
    A, B = mx_pack("e2m1", pa), mx_pack("e2m1", pb)
    SA = rng.integers(120, 135, (M, 7)).astype(np.uint8)
    SB = rng.integers(120, 135, (N, 6)).astype(np.uint8)
    C0 = rng.standard_normal((N, M)).astype(np.float32)  # column-major C, ldc = M
    ref, den = oracle.mx_gemm("e2m1", "e2m1", "f32", M, N, K, 1.0, A, lda, SA.ravel(), 7, B, ldb,
                              SB.ravel(), 6, 0.5, C0.ravel(), M, COL)
    # the same problem with the padding cut away and C transposed to row-major
    A2, B2 = mx_pack("e2m1", pa[:, :K]), mx_pack("e2m1", pb[:, :K])
    ref2, den2 = oracle.mx_gemm("e2m1", "e2m1", "f32", M, N, K, 1.0, A2, K,
                                np.ascontiguousarray(SA[:, :4]).ravel(), 4, B2, K,
                                np.ascontiguousarray(SB[:, :4]).ravel(), 4, 0.5,
                                np.ascontiguousarray(C0.T).ravel(), N, ROW)
    assert np.array_equal(ref, ref2) and np.array_equal(den, den2)
    idx = np.array([[0, i, j] for i in range(M) for j in range(N)])
    r, d = oracle.mx_gemm_at("e2m1", "e2m1", "f32", M, N, K, 1.0, A, lda, SA.ravel(), 7, B, ldb,
                             SB.ravel(), 6, 0.5, C0.ravel(), M, COL, idx)
    assert np.array_equal(r, ref[0].ravel()) and np.array_equal(d, den[0].ravel())
