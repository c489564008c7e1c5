"""The accuracy claim of gemm_f32_bf16x3, checked on the CPU.

The fp32 product a*b is taken as hi_a*hi_b + hi_a*lo_b + lo_a*hi_b, where
hi = v rounded to bf16 (nearest, ties to even; truncated when that would
overflow) and lo = (v - hi) rounded to bf16.  The header states that the
terms left out are at most 2^-15 |a*b|; with every product exact in fp32,
that bound plus fp32 accumulation is the whole error of an element, well
inside the 1e-4 relative criterion the fp32 parity tests apply.  Here the
bound is checked in exact (float64) arithmetic on random pairs over the whole
fp32 exponent range and on the values where rounding to bf16 is least kind:
ties, values just below a power of two, the largest finite fp32.
"""
import numpy as np


def bf16_hi(v: np.ndarray) -> np.ndarray:
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    over = ((r & 0x7FFF) == 0x7F80) & ((u & 0x7FFFFFFF) != 0x7F800000)
    r = np.where(over, (u >> 16) & 0xFFFF, r)
    return (r.astype(np.uint32) << 16).view(np.float32)


def split(v):
    v = np.asarray(v, np.float32)
    hi = bf16_hi(v)
    lo = bf16_hi((v - hi).astype(np.float32))  # v - hi is exact in fp32
    return hi, lo


def left_out(a, b):
    ha, la = split(a)
    hb, lb = split(b)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    kept = (ha.astype(np.float64) * hb + ha.astype(np.float64) * lb + la.astype(np.float64) * hb)
    return np.abs(a64 * b64 - kept), np.abs(a64 * b64)


def test_split_pieces_are_exact_sums():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(100000) * np.exp2(rng.integers(-60, 60, 100000))).astype(np.float32)
    hi, lo = split(v)
    # hi carries 8 significant bits; v - hi is exactly representable; lo is
    # v - hi rounded to 8 bits, so the residual is at most 2^-17 |v|
    assert np.all(np.abs(v.astype(np.float64) - hi) <= np.exp2(-8) * np.abs(v))
    assert np.all(np.abs(v.astype(np.float64) - hi - lo) <= np.exp2(-17) * np.abs(v) * 1.0000001)


def test_left_out_terms_random():
    rng = np.random.default_rng(1)
    n = 1_000_000
    a = (rng.uniform(-1, 1, n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    b = (rng.uniform(-1, 1, n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    err, mag = left_out(a, b)
    assert np.all(err <= np.exp2(-15) * mag)
    # and the bound is not loose by orders of magnitude
    assert np.max(err / np.where(mag > 0, mag, 1)) > np.exp2(-18)


def test_left_out_terms_adversarial():
    # ties to even, just below powers of two, the largest finite value (whose
    # rounding to bf16 would overflow: hi is truncated instead), bf16-exact
    # values (lo = 0) and the smallest normal
    base = np.array([1.0, 1.5, 1.99999988, 2.0 - 2.0 ** -8, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9,
                     1.0 + 2.0 ** -8 + 2.0 ** -16, 3.4028235e38, 3.3961776e38, 1.1754944e-38,
                     0.1, 1.0 / 3.0, 2.0 ** 100 * 1.00390625, 65504.0, 1e-30],
                    np.float64)
    vals = np.concatenate([base, -base]).astype(np.float32)
    assert np.all(np.isfinite(vals))
    a, b = np.meshgrid(vals, vals)
    a, b = a.ravel(), b.ravel()
    ok = np.isfinite(a.astype(np.float64) * b) & (np.abs(a.astype(np.float64) * b) < 3.4e38)
    err, mag = left_out(a[ok], b[ok])
    assert np.all(err <= np.exp2(-15) * mag)
    hi, lo = split(np.float32(3.4028235e38))
    assert np.isfinite(hi) and hi <= 3.4028235e38 and np.isfinite(lo)


def test_integers_split_exactly():
    # small integers are bf16 values: lo = 0 and hi*hi is the exact product,
    # which the GPU tests use to require bit-exact results
    v = np.arange(-256, 257, dtype=np.float32)
    hi, lo = split(v)
    assert np.array_equal(hi, v) and np.all(lo == 0)
