"""Seeded synthetic inputs for the GEMM workloads.

This module is the one piece that both the GPU tests and the CPU oracle
consume.  It holds no GEMM arithmetic: it draws random numbers, rounds them to
the stored element type and describes each problem (shapes, scalars, layouts).

Recipe (the pages fix shapes but not distributions or seeds beyond what is
listed here, so the reading taken is stated once, here):

* random numbers come from numpy's PCG64 (``np.random.default_rng(seed)``),
  seed 0 unless a workload states another, drawn in the order A, B, then C0
  (P for the attention product), each in row-major element order of the
  matrix as a mathematical object (independent of how it is then stored);
* fp32 entries: ``uniform(-1, 1)`` in float64, rounded to float32;
* bf16/fp16 entries: ``sigma * standard_normal()`` in float64, rounded to
  float32, then to the 16-bit type with round-to-nearest-even (torch's CPU
  conversion);
* 8-bit float entries (OCP E4M3 "e4m3", E5M2 "e5m2"): drawn like bf16 ones,
  then converted by torch's float8_e4m3fn / float8_e5m2 (nearest-even); A and
  B may have different 8-bit types (``b_dtype``);
* softmax rows (the attention probabilities): logits uniform(-1, 1), a
  row-wise softmax in float64, then rounded like any bf16 entry;
* block-scaled (MX) problems (``MxProblem``): element bit patterns drawn
  uniformly from the format's finite patterns (every pattern of the 6- and
  4-bit formats; the 8-bit ones without their NaN and infinity patterns), in
  row-major order of A (M x K) then of B^T (N x K), packed as the library's
  little-endian bit stream with zero elements as padding; the E8M0 scales
  uniform integers in [scale_lo, scale_hi] (2^-4 .. 2^4 by default) for the
  ceil(K/32) blocks of each row, the row padding up to ldsa filled with the
  NaN pattern 0xFF (never used); then C0 as for the other problems;
* the bias of a problem with a fused epilogue comes from a second stream,
  ``np.random.default_rng([seed, 1])``, N entries per batch entry (one vector
  when ``stride_bias`` is 0), drawn like an entry of A with ``sigma_bias``.

Shapes follow the pages: the square 4096 problem of "CUDA GEMM 矩阵乘法优化指南"
section 2.1 and of the hgemm sm120 article's benchmark; the transformer-layer
shapes listed in section 1 of "第4章：经典算子实现 —— GEMM" (QKV projection,
FFN up/down, batched QK^T and PV).
"""
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

ROW, COL = 0, 1


@dataclass
class Problem:
    """One (possibly batched) GEMM: C = alpha * op(A) @ op(B) + beta * C.

    Element (i, k) of A lives at ``A[b*stride_a + i*lda + k]`` when
    ``order_a == ROW`` and at ``A[b*stride_a + k*lda + i]`` when COL; likewise
    B (K x N) and C (M x N).  ``in_dtype`` is the type of A and B, ``c_dtype``
    the type of C (both its initial value and the result).
    """
    name: str
    in_dtype: str                    # type of A (and B unless b_dtype is set)
    c_dtype: str
    M: int
    N: int
    K: int
    alpha: float = 1.0
    beta: float = 0.0
    order_a: int = ROW
    order_b: int = ROW
    order_c: int = ROW
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    batch: int = 1
    stride_a: Optional[int] = None
    stride_b: Optional[int] = None
    stride_c: Optional[int] = None
    sigma_a: float = 1.0
    sigma_b: float = 1.0
    sigma_c: float = 1.0
    a_kind: str = "default"          # "default" or "softmax" (rows of P)
    seed: int = 0
    note: str = ""
    # fused epilogue: C = act(alpha*A@B + beta*C + bias_j)
    bias: bool = False               # add a per-column bias vector
    stride_bias: Optional[int] = None  # elements between batch entries' vectors
    sigma_bias: float = 1.0
    act: int = 0                     # 0 none, 1 ReLU, 2 GELU
    b_dtype: Optional[str] = None    # type of B when it differs from A's (8-bit floats)
    entry: str = ""                  # "valu": gemm_f32_valu; "bf16x3": gemm_f32_bf16x3;
                                     # "quant": gemm_bf16_quant / gemm_f16_quant (8-bit C)
    c_scale: float = 1.0             # "quant": the scale applied before the 8-bit store

    def __post_init__(self):
        M, N, K = self.M, self.N, self.K
        if self.lda is None:
            self.lda = max(1, K if self.order_a == ROW else M)
        if self.ldb is None:
            self.ldb = max(1, N if self.order_b == ROW else K)
        if self.ldc is None:
            self.ldc = max(1, N if self.order_c == ROW else M)
        if self.stride_a is None:
            self.stride_a = self.footprint("a")
        if self.stride_b is None:
            self.stride_b = self.footprint("b")
        if self.stride_c is None:
            self.stride_c = self.footprint("c")
        if self.stride_bias is None:
            self.stride_bias = N if self.batch > 1 else 0
        if self.b_dtype is None:
            self.b_dtype = self.in_dtype

    def dims(self, which):
        return {"a": (self.M, self.K, self.order_a, self.lda),
                "b": (self.K, self.N, self.order_b, self.ldb),
                "c": (self.M, self.N, self.order_c, self.ldc)}[which]

    def footprint(self, which) -> int:
        """Elements one matrix of the batch spans (0 if it is empty)."""
        r, c, order, ld = self.dims(which)
        if r == 0 or c == 0:
            return 0
        outer, inner = (r, c) if order == ROW else (c, r)
        return (outer - 1) * ld + inner

    def buffer_elems(self, which) -> int:
        stride = {"a": self.stride_a, "b": self.stride_b, "c": self.stride_c}[which]
        fp = self.footprint(which)
        if self.batch == 0 or fp == 0:
            return 0
        return (self.batch - 1) * stride + fp

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    def with_(self, **kw) -> "Problem":
        return replace(self, **kw)


def _f32(x64: np.ndarray) -> np.ndarray:
    return x64.astype(np.float32)


EIGHT_BIT = ("e4m3", "e5m2")


def storage(dtype: str):
    """numpy type of a stored element."""
    if dtype == "f32":
        return np.float32
    return np.uint8 if dtype in EIGHT_BIT else np.uint16


def to_8bit(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to OCP 8-bit float bit patterns (uint8), nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    tdt = torch.float8_e4m3fn if dtype == "e4m3" else torch.float8_e5m2
    return t.to(tdt).view(torch.uint8).numpy()


def to_16bit(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to bf16/fp16 bit patterns (uint16), nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return t.to(tdt).view(torch.int16).numpy().view(np.uint16)


def _draw(rng, dtype, rows, cols, sigma, kind="default"):
    """Draw a rows x cols matrix (row-major element order) in its stored type."""
    if kind == "softmax":
        logits = rng.uniform(-1.0, 1.0, size=(rows, cols))
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        return to_16bit(_f32(p), dtype) if dtype != "f32" else _f32(p)
    if dtype == "f32":
        return _f32(rng.uniform(-1.0, 1.0, size=(rows, cols)) * sigma)
    x = _f32(rng.standard_normal(size=(rows, cols)) * sigma)
    return to_8bit(x, dtype) if dtype in EIGHT_BIT else to_16bit(x, dtype)


def _store(mat: np.ndarray, order: int, ld: int, batch_stride: int, b: int,
           out: np.ndarray):
    rows, cols = mat.shape
    if rows == 0 or cols == 0:
        return
    base = b * batch_stride
    if order == ROW:
        view = np.lib.stride_tricks.as_strided(
            out[base:], shape=(rows, cols), strides=(ld * out.itemsize, out.itemsize))
    else:
        view = np.lib.stride_tricks.as_strided(
            out[base:], shape=(rows, cols), strides=(out.itemsize, ld * out.itemsize))
    view[...] = mat


def generate(p: Problem, seed: Optional[int] = None):
    """Host buffers (flat numpy arrays) for A, B and the initial C.

    Padding elements (beyond the matrix inside ld, or between batch slices)
    are zero.  C0 is drawn even when beta == 0, so the draws of a workload do
    not depend on its scalars.  A stride of 0 for A or B (one matrix shared
    by the whole batch) draws that matrix once.
    """
    rng = np.random.default_rng(p.seed if seed is None else seed)
    bufs = {}
    for which, dt, sig, kind in (("a", p.in_dtype, p.sigma_a, p.a_kind),
                                 ("b", p.b_dtype, p.sigma_b, "default"),
                                 ("c", p.c_dtype, p.sigma_c, "default")):
        r, c, order, ld = p.dims(which)
        stride = {"a": p.stride_a, "b": p.stride_b, "c": p.stride_c}[which]
        out = np.zeros(p.buffer_elems(which), storage(dt))
        nb = 1 if stride == 0 else p.batch
        for b in range(nb):
            _store(_draw(rng, dt, r, c, sig, kind), order, ld, stride, b, out)
        bufs[which] = out
    return bufs["a"], bufs["b"], bufs["c"]


def bias_vector(p: Problem, seed: Optional[int] = None):
    """The bias of a fused-epilogue problem as a flat stored-type buffer of
    (batch - 1) * stride_bias + N elements, or None when p has no bias."""
    if not p.bias:
        return None
    rng = np.random.default_rng([p.seed if seed is None else seed, 1])
    n = (p.batch - 1) * p.stride_bias + p.N if p.batch > 0 else 0
    out = np.zeros(n, np.float32 if p.in_dtype == "f32" else np.uint16)
    for b in range(1 if p.stride_bias == 0 else p.batch):
        out[b * p.stride_bias:b * p.stride_bias + p.N] = _draw(rng, p.in_dtype, 1, p.N,
                                                               p.sigma_bias)[0]
    return out


# ---------------------------------------------------------------- block-scaled (MX)

MX_WIDTH = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}


@dataclass
class MxProblem:
    """A block-scaled GEMM C = alpha * A @ B + beta * C (gemm_mx).

    A is M x K and B is K x N, both contiguous along K: row i of A is
    elements b*stride_a + i*lda + (0 .. K-1) of A's packed stream, column j
    of B elements b*stride_b + j*ldb + (0 .. K-1) of B's; E8M0 scales
    SA[b*stride_sa + i*ldsa + k//32] and SB[b*stride_sb + j*ldsb + k//32]
    (bytes).  C as in Problem (c_dtype, order_c, ldc, stride_c).
    """
    name: str
    fa: str
    fb: str
    c_dtype: str
    M: int
    N: int
    K: int
    alpha: float = 1.0
    beta: float = 0.0
    order_c: int = ROW
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    ldsa: Optional[int] = None
    ldsb: Optional[int] = None
    batch: int = 1
    stride_a: Optional[int] = None
    stride_b: Optional[int] = None
    stride_sa: Optional[int] = None
    stride_sb: Optional[int] = None
    stride_c: Optional[int] = None
    scale_lo: int = 123
    scale_hi: int = 131
    sigma_c: float = 1.0
    seed: int = 0
    note: str = ""

    def __post_init__(self):
        M, N, K = self.M, self.N, self.K
        k64 = max(64, -(-K // 64) * 64)
        sbytes = max(4, 4 * -(-K // 128))
        self.lda = k64 if self.lda is None else self.lda
        self.ldb = k64 if self.ldb is None else self.ldb
        self.ldsa = sbytes if self.ldsa is None else self.ldsa
        self.ldsb = sbytes if self.ldsb is None else self.ldsb
        if self.ldc is None:
            self.ldc = max(1, N if self.order_c == ROW else M)
        if self.stride_a is None:
            self.stride_a = M * self.lda
        if self.stride_b is None:
            self.stride_b = N * self.ldb
        if self.stride_sa is None:
            self.stride_sa = M * self.ldsa
        if self.stride_sb is None:
            self.stride_sb = N * self.ldsb
        if self.stride_c is None:
            outer, inner = (M, N) if self.order_c == ROW else (N, M)
            self.stride_c = (outer - 1) * self.ldc + inner if M and N else 0

    # C as a Problem sees it (for the parity harness's C handling)
    def dims(self, which):
        assert which == "c"
        return (self.M, self.N, self.order_c, self.ldc)

    def buffer_elems(self, which) -> int:
        assert which == "c"
        if self.batch == 0 or self.stride_c == 0 and self.M * self.N == 0:
            return 0
        outer, inner = (self.M, self.N) if self.order_c == ROW else (self.N, self.M)
        return (self.batch - 1) * self.stride_c + (outer - 1) * self.ldc + inner

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    def with_(self, **kw) -> "MxProblem":
        return replace(self, **kw)


def finite_patterns(fmt: str) -> np.ndarray:
    """Bit patterns of a format's finite values."""
    n = 1 << MX_WIDTH[fmt]
    p = np.arange(n, dtype=np.uint16)
    if fmt == "e4m3":
        p = p[(p & 0x7F) != 0x7F]
    elif fmt == "e5m2":
        p = p[(p & 0x7C) != 0x7C]
    return p.astype(np.uint8)


def mx_pack(patterns: np.ndarray, width: int) -> np.ndarray:
    """Pack a rows x cols array of element patterns (cols * width a multiple
    of 8) row by row into the little-endian bit stream: rows x cols*width/8."""
    p = np.ascontiguousarray(patterns, dtype=np.uint32)
    rows, cols = p.shape
    if width == 8:
        return p.astype(np.uint8)
    if width == 4:
        return (p[:, 0::2] | (p[:, 1::2] << 4)).astype(np.uint8)
    assert width == 6 and cols % 4 == 0
    w = p[:, 0::4] | (p[:, 1::4] << 6) | (p[:, 2::4] << 12) | (p[:, 3::4] << 18)
    out = np.empty((rows, cols // 4, 3), np.uint8)
    out[:, :, 0] = w & 0xFF
    out[:, :, 1] = (w >> 8) & 0xFF
    out[:, :, 2] = (w >> 16) & 0xFF
    return out.reshape(rows, cols * 3 // 4)


def generate_mx(p: MxProblem, seed: Optional[int] = None, patterns=None):
    """Host buffers (flat uint8 arrays) A, SA, B, SB and the initial C.

    patterns: optional (A, B) pattern arrays of shape (batch, M, K) and
    (batch, N, K) used instead of random ones (scales are still drawn).
    """
    rng = np.random.default_rng(p.seed if seed is None else seed)
    nblk = -(-p.K // 32)
    out = {}
    for which, fmt, rows, ld, stride, lds, sstride in (
            ("a", p.fa, p.M, p.lda, p.stride_a, p.ldsa, p.stride_sa),
            ("b", p.fb, p.N, p.ldb, p.stride_b, p.ldsb, p.stride_sb)):
        w = MX_WIDTH[fmt]
        nb = 1 if stride == 0 else p.batch
        total = ((p.batch - 1) * stride + rows * ld) if p.batch and rows else 0
        data = np.zeros(total * w // 8, np.uint8)
        ns = ((p.batch - 1) * sstride + rows * lds) if p.batch and rows else 0
        scales = np.full(ns, 0xFF, np.uint8)
        fin = finite_patterns(fmt)
        for b in range(nb):
            if patterns is not None:
                pat = np.asarray(patterns[0 if which == "a" else 1][b], np.uint8)
            else:
                pat = fin[rng.integers(0, fin.size, (rows, p.K))]
            full = np.zeros((rows, ld), np.uint8)
            full[:, :p.K] = pat
            packed = mx_pack(full, w).ravel()
            data[b * stride * w // 8:b * stride * w // 8 + packed.size] = packed
        for b in range(1 if sstride == 0 else p.batch):
            sc = rng.integers(p.scale_lo, p.scale_hi + 1, (rows, nblk)).astype(np.uint8)
            view = scales[b * sstride:b * sstride + rows * lds].reshape(rows, lds)
            view[:, :nblk] = sc
        out[which], out["s" + which] = data, scales
    c = np.zeros(p.buffer_elems("c"), storage(p.c_dtype))
    for b in range(p.batch):
        _store(_draw(rng, p.c_dtype, p.M, p.N, p.sigma_c), p.order_c, p.ldc, p.stride_c, b, c)
    return out["a"], out["sa"], out["b"], out["sb"], c


def _configs():
    cfgs = [
        Problem("f32_256", "f32", "f32", 256, 256, 256,
                note="fp32 SGEMM 256^3, row-major, alpha=1 beta=0, U[-1,1], seed 0"),
        Problem("f32_4096", "f32", "f32", 4096, 4096, 4096,
                note="fp32 SGEMM 4096^3, row-major, alpha=1 beta=0, U[-1,1]"),
        Problem("f32_4096_valu", "f32", "f32", 4096, 4096, 4096, entry="valu",
                note="fp32 SGEMM 4096^3 on the vector-ALU kernel (gemm_f32_valu), U[-1,1]"),
        Problem("f32_4096_bf16x3", "f32", "f32", 4096, 4096, 4096, entry="bf16x3",
                note="fp32 SGEMM 4096^3 as three bf16 products of split operands "
                     "(gemm_f32_bf16x3), U[-1,1]"),
        Problem("bf16_4096", "bf16", "bf16", 4096, 4096, 4096,
                note="bf16 HGEMM 4096^3, fp32 accumulate, bf16 out, N(0,1)"),
        Problem("f16_4096", "f16", "f16", 4096, 4096, 4096,
                note="fp16 HGEMM 4096^3, fp32 accumulate, fp16 out, N(0,1)"),
        Problem("bf16_qkv", "bf16", "bf16", 4096, 12288, 4096, beta=1.0, sigma_b=0.02,
                note="QKV projection X(4096x4096) W(4096x12288), beta=1, C0 N(0,1)"),
        Problem("bf16_ffn_up", "bf16", "bf16", 4096, 16384, 4096, beta=1.0, sigma_b=0.02,
                note="FFN up X(4096x4096) W1(4096x16384), beta=1, C0 N(0,1)"),
        Problem("bf16_ffn_down", "bf16", "bf16", 4096, 4096, 16384, beta=1.0, sigma_b=0.02,
                note="FFN down H(4096x16384) W2(16384x4096), beta=1, C0 N(0,1)"),
        Problem("f32_edge", "f32", "f32", 4095, 4097, 1001, alpha=0.5, beta=2.0,
                note="unaligned fp32 4095x4097x1001, alpha=0.5 beta=2, C0 U[-1,1]"),
        Problem("bf16_edge", "bf16", "bf16", 4095, 4097, 1001, alpha=0.5, beta=2.0,
                note="unaligned bf16 4095x4097x1001, alpha=0.5 beta=2, C0 N(0,1)"),
        # aligned, but 16 x 17 = 272 tiles of 256 x 256: one wave of 256
        # compute units and 16 tiles more (the stream-K case of the fast path)
        Problem("bf16_tail", "bf16", "bf16", 4096, 4352, 4096,
                note="aligned bf16 4096x4352x4096 (272 tiles: one wave plus 16)"),
        Problem("bf16_skinny", "bf16", "bf16", 16, 4096, 4096,
                note="skinny bf16 16x4096x4096 (bandwidth-bound)"),
        # Q (2048x128) times K^T: K is stored 2048x128 row-major, which is the
        # 128x2048 operand B in column-major order with ldb = 128.
        Problem("bf16_attn_qk", "bf16", "bf16", 2048, 2048, 128, order_b=COL, ldb=128,
                batch=32, note="batched QK^T, 32 x (2048x128)(128x2048)"),
        Problem("bf16_attn_pv", "bf16", "bf16", 2048, 128, 2048, a_kind="softmax",
                batch=32, note="batched PV, 32 x (2048x2048)(2048x128), P softmax rows"),
        # the FFN up projection with its bias and activation fused into the
        # GEMM's epilogue (the "GEMM + bias + activation" case of the pages)
        Problem("bf16_ffn_up_gelu", "bf16", "bf16", 4096, 16384, 4096, sigma_b=0.02,
                bias=True, act=2,
                note="FFN up X(4096x4096) W1(4096x16384) + b1 then GELU, fused epilogue"),
        # the same layer with its output quantised to E4M3 in the epilogue
        # (scale 16: GELU outputs of N(0, 0.02^2 * 4096) sums land well inside
        # the format's range)
        Problem("bf16_ffn_up_gelu_e4m3", "bf16", "e4m3", 4096, 16384, 4096, sigma_b=0.02,
                bias=True, act=2, entry="quant", c_scale=16.0,
                note="FFN up X(4096x4096) W1(4096x16384) + b1, GELU, x16 and E4M3 output, "
                     "fused epilogue"),
        # 8-bit float inputs in the layout 8-bit GEMMs take: A row-major and B
        # column-major (both contiguous along K), output bf16
        # block-scaled formats (one E8M0 scale per 32 k), K contiguous in
        # both operands as the format requires
        MxProblem("mxfp4_4096", "e2m1", "e2m1", "bf16", 4096, 4096, 4096,
                  note="MXFP4 4096^3 (E2M1 elements, E8M0 scale per 32 k), bf16 out"),
        MxProblem("mxfp6_4096", "e2m3", "e2m3", "bf16", 4096, 4096, 4096,
                  note="MXFP6 4096^3 (E2M3 elements, E8M0 scale per 32 k), bf16 out"),
        MxProblem("mxfp8_4096", "e4m3", "e4m3", "bf16", 4096, 4096, 4096,
                  note="MXFP8 4096^3 (E4M3 elements, E8M0 scale per 32 k), bf16 out"),
        Problem("fp8_4096", "e4m3", "bf16", 4096, 4096, 4096, order_b=COL,
                note="E4M3 GEMM 4096^3, A row-major, B column-major, fp32 accumulate, bf16 out"),
        # 16 x 17 = 272 tiles of 256 x 256 again: the stream-K case of the
        # narrow-float kernel (through the workspace entry points)
        Problem("fp8_tail", "e4m3", "bf16", 4096, 4352, 4096, order_b=COL,
                note="E4M3 4096x4352x4096 TN, bf16 out (272 tiles: one wave plus 16)"),
        MxProblem("mxfp4_tail", "e2m1", "e2m1", "bf16", 4096, 4352, 4096,
                  note="MXFP4 4096x4352x4096, bf16 out (272 tiles: one wave plus 16)"),
    ]
    return {c.name: c for c in cfgs}


CONFIGS = _configs()


def config(name: str):
    """The workload of that name (a Problem, or an MxProblem for the
    block-scaled ones)."""
    return CONFIGS[name]
