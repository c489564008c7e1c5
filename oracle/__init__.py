"""CPU oracle for dense GEMM, C = act(alpha*A*B + beta*C + bias).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the GPU library and
its Python binding never do, and nothing here imports them.

The arithmetic lives in ``gemm_oracle.c`` (plain C, double accumulation, see
its header for the passages it follows).  This module only marshals numpy
buffers into it.

Element types: ``"f32"`` buffers are float32 (or their uint32 bit patterns),
``"bf16"`` and ``"f16"`` buffers are uint16 bit patterns, ``"e4m3"`` and
``"e5m2"`` (8-bit floats) uint8 bit patterns.  Block-scaled (MX) operands
are packed uint8 streams of ``"e4m3"``, ``"e5m2"``, ``"e2m3"``, ``"e3m2"`` or
``"e2m1"`` elements with uint8 E8M0 scales, one per 32 elements along K
(``mx_gemm``); ``decode`` also takes those formats and ``"e8m0"`` one value
per byte.  Matrices are flat
buffers addressed with a leading dimension, an order (``ROW`` or ``COL``) and
a per-batch stride in elements, exactly as the GEMM library takes them.
"""
import ctypes
import os

import numpy as np

from . import build as _build

ROW, COL = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2
_TYPES = {"f32": 0, "bf16": 1, "f16": 2, "e4m3": 3, "e5m2": 4, "e2m3": 5, "e3m2": 6,
          "e2m1": 7, "e8m0": 8}
MX_FORMATS = ("e4m3", "e5m2", "e2m3", "e3m2", "e2m1")

_lib = None


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB lets the mutation test load a deliberately broken build.
        path = os.environ.get("ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        prob = [i32, i32, i64, i64, i64, dbl, vp, i64, i32, vp, i64, i32, dbl, vp, i64,
                i32, i64, i64, i64, vp, i64, i32, i32]
        lib.orc_gemm.argtypes = prob + [i64, vp, vp]
        lib.orc_gemm.restype = None
        lib.orc_gemm_at.argtypes = prob + [i64, vp, vp, vp]
        lib.orc_gemm_at.restype = None
        lib.orc_decode.argtypes = [i32, vp, vp, i64]
        lib.orc_decode.restype = None
        lib.orc_round.argtypes = [i32, vp, vp, i64]
        lib.orc_round.restype = None
        mx = [i32, i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, vp, i64, vp, i64, dbl, vp,
              i64, i32, i64, i64, i64, i64, i64]
        lib.orc_mx_gemm.argtypes = mx + [i64, vp, vp]
        lib.orc_mx_gemm.restype = None
        lib.orc_mx_gemm_at.argtypes = mx + [i64, vp, vp, vp]
        lib.orc_mx_gemm_at.restype = None
        lib.orc_mx_element.argtypes = [i32, vp, i64]
        lib.orc_mx_element.restype = dbl
        lib.orc_max_threads.restype = i32
        lib.orc_set_threads.argtypes = [i32]
        lib.orc_set_threads.restype = None
        _lib = lib
    return _lib


def _storage(dtype):
    if dtype == "f32":
        return np.float32
    return np.uint16 if dtype in ("bf16", "f16") else np.uint8


def _buf(x, dtype):
    """Contiguous host buffer of the stored element type (keeps a reference)."""
    if x is None:
        return None, None
    a = np.ascontiguousarray(x)
    if dtype == "f32" and a.dtype == np.uint32:
        a = a.view(np.float32)
    want = _storage(dtype)
    if a.dtype != want:
        raise TypeError(f"oracle: {dtype} buffer must be {np.dtype(want).name}, got {a.dtype}")
    return a, a.ctypes.data


def max_threads() -> int:
    return int(_load().orc_max_threads())


def set_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use from now on."""
    _load().orc_set_threads(int(n))


def decode(dtype, bits) -> np.ndarray:
    """Exact values of stored elements, as float64."""
    a, p = _buf(bits, dtype)
    out = np.empty(a.size, np.float64)
    _load().orc_decode(_TYPES[dtype], p, out.ctypes.data, a.size)
    return out.reshape(a.shape)


def round_bits(dtype, x) -> np.ndarray:
    """Round float64 values to ``dtype`` (nearest-even, directly from double).

    Returns the stored patterns: uint32 for f32, uint16 for bf16/f16, uint8
    for e4m3/e5m2 (saturating: beyond the largest finite value, infinities
    included, gives that value; NaN the canonical NaN).
    """
    src = np.ascontiguousarray(x, dtype=np.float64)
    store = {"f32": np.uint32, "e4m3": np.uint8, "e5m2": np.uint8}.get(dtype, np.uint16)
    out = np.empty(src.size, store)
    _load().orc_round(_TYPES[dtype], src.ctypes.data, out.ctypes.data, src.size)
    return out.reshape(src.shape)


def _args(in_dtype, c_dtype, M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C0,
          ldc, order_c, stride_a, stride_b, stride_c, bias, stride_bias, act, b_dtype):
    b_dtype = b_dtype or in_dtype
    keep = []
    ptrs = []
    for x, dt in ((A, in_dtype), (B, b_dtype), (C0, c_dtype), (bias, in_dtype)):
        a, p = _buf(x, dt)
        keep.append(a)
        ptrs.append(p)
    args = [_TYPES[in_dtype], _TYPES[c_dtype], M, N, K, float(alpha), ptrs[0], lda, order_a,
            ptrs[1], ldb, order_b, float(beta), ptrs[2], ldc, order_c, stride_a, stride_b,
            stride_c, ptrs[3], stride_bias, int(act), _TYPES[b_dtype]]
    return args, keep


def gemm(in_dtype, c_dtype, M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C0,
         ldc, order_c, batch=1, stride_a=0, stride_b=0, stride_c=0, bias=None, stride_bias=0,
         act=ACT_NONE, b_dtype=None):
    """Every element: returns (ref, den) as float64 arrays [batch][M][N].

    ref = act(alpha*sum_k A_ik B_kj + beta*C0_ij + bias_j) and
    den = |alpha|*sum_k |A_ik B_kj| + |beta|*|C0_ij| + |bias_j|, accumulated in
    double.  ``bias`` (optional) holds N input-type elements per batch entry,
    ``stride_bias`` apart; ``act`` is ACT_NONE, ACT_RELU or ACT_GELU.
    ``b_dtype`` is B's element type when it differs from A's (8-bit inputs).
    """
    args, keep = _args(in_dtype, c_dtype, M, N, K, alpha, A, lda, order_a, B, ldb, order_b,
                       beta, C0, ldc, order_c, stride_a, stride_b, stride_c, bias, stride_bias,
                       act, b_dtype)
    ref = np.empty((batch, M, N), np.float64)
    den = np.empty((batch, M, N), np.float64)
    _load().orc_gemm(*args, batch, ref.ctypes.data, den.ctypes.data)
    del keep
    return ref, den


def gemm_at(in_dtype, c_dtype, M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C0,
            ldc, order_c, idx, stride_a=0, stride_b=0, stride_c=0, bias=None, stride_bias=0,
            act=ACT_NONE, b_dtype=None):
    """Only the elements listed in ``idx`` (an (n, 3) array of (b, i, j))."""
    idx = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 3)
    args, keep = _args(in_dtype, c_dtype, M, N, K, alpha, A, lda, order_a, B, ldb, order_b,
                       beta, C0, ldc, order_c, stride_a, stride_b, stride_c, bias, stride_bias,
                       act, b_dtype)
    n = idx.shape[0]
    ref = np.empty(n, np.float64)
    den = np.empty(n, np.float64)
    _load().orc_gemm_at(*args, n, idx.ctypes.data, ref.ctypes.data, den.ctypes.data)
    del keep
    return ref, den


def _mx_args(fa, fb, c_dtype, M, N, K, alpha, A, lda, SA, ldsa, B, ldb, SB, ldsb, beta, C0, ldc,
             order_c, stride_a, stride_b, stride_sa, stride_sb, stride_c):
    keep, ptrs = [], []
    for x in (A, SA, B, SB):
        a = np.ascontiguousarray(x)
        if a.dtype != np.uint8:
            raise TypeError(f"oracle: MX operands and scales are uint8, got {a.dtype}")
        keep.append(a)
        ptrs.append(a.ctypes.data)
    c, pc = _buf(C0, c_dtype)
    keep.append(c)
    args = [_TYPES[fa], _TYPES[fb], _TYPES[c_dtype], M, N, K, float(alpha), ptrs[0], lda,
            ptrs[1], ldsa, ptrs[2], ldb, ptrs[3], ldsb, float(beta), pc, ldc, order_c,
            stride_a, stride_b, stride_sa, stride_sb, stride_c]
    return args, keep


def mx_gemm(fa, fb, c_dtype, M, N, K, alpha, A, lda, SA, ldsa, B, ldb, SB, ldsb, beta, C0, ldc,
            order_c, batch=1, stride_a=0, stride_b=0, stride_sa=0, stride_sb=0, stride_c=0):
    """Block-scaled GEMM, every element: (ref, den) as float64 [batch][M][N].

    A(i, k) is element b*stride_a + i*lda + k of the packed stream A (format
    fa), scaled by 2^(SA[b*stride_sa + i*ldsa + k//32] - 127); B(k, j) is
    element b*stride_b + j*ldb + k of B (format fb: K contiguous along each
    column), scaled by SB[b*stride_sb + j*ldsb + k//32].  ref = alpha *
    sum_k A(i,k) B(k,j) + beta * C0_ij; den the matching sum of magnitudes.
    """
    args, keep = _mx_args(fa, fb, c_dtype, M, N, K, alpha, A, lda, SA, ldsa, B, ldb, SB, ldsb,
                          beta, C0, ldc, order_c, stride_a, stride_b, stride_sa, stride_sb,
                          stride_c)
    ref = np.empty((batch, M, N), np.float64)
    den = np.empty((batch, M, N), np.float64)
    _load().orc_mx_gemm(*args, batch, ref.ctypes.data, den.ctypes.data)
    del keep
    return ref, den


def mx_gemm_at(fa, fb, c_dtype, M, N, K, alpha, A, lda, SA, ldsa, B, ldb, SB, ldsb, beta, C0,
               ldc, order_c, idx, stride_a=0, stride_b=0, stride_sa=0, stride_sb=0, stride_c=0):
    """Only the elements listed in ``idx`` (an (n, 3) array of (b, i, j))."""
    idx = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 3)
    args, keep = _mx_args(fa, fb, c_dtype, M, N, K, alpha, A, lda, SA, ldsa, B, ldb, SB, ldsb,
                          beta, C0, ldc, order_c, stride_a, stride_b, stride_sa, stride_sb,
                          stride_c)
    n = idx.shape[0]
    ref = np.empty(n, np.float64)
    den = np.empty(n, np.float64)
    _load().orc_mx_gemm_at(*args, n, idx.ctypes.data, ref.ctypes.data, den.ctypes.data)
    del keep
    return ref, den


def mx_element(fmt, packed, idx) -> float:
    """Element ``idx`` of a packed MX stream, decoded (unscaled)."""
    a = np.ascontiguousarray(packed, dtype=np.uint8)
    return float(_load().orc_mx_element(_TYPES[fmt], a.ctypes.data, int(idx)))
