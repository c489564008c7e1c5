"""Run one GEMM through libgemm on the GPU and compare it with the CPU oracle.

Tolerances (the bar the tests hold every result to):
  * fp32 inputs, fp32 output: max |C - ref| / den <= 1e-4;
  * bf16/fp16 inputs, fp32 output: the same bound <= 1e-3;
  * bf16/fp16 output: within 2 units in the last place of the oracle result
    rounded (nearest-even, directly from double) to the output type.  An
    element further away is accepted only where the result is a genuine
    cancellation, |ref| <= 2^-8 * den, and the difference stays inside the
    fp32-accumulation bound 2 ulp + 1e-3 * den; such elements are counted;
  * wherever den == 0 the result must equal ref exactly;
  * memory outside C (guard bands around the buffer, padding inside the
    leading dimension and between batch slices) must be bit-unchanged, and
    A and B must be unchanged.

``den`` is the oracle's magnitude scale |alpha| * sum_k |A_ik B_kj| +
|beta| * |C0_ij|.  For alpha = 1 and beta = 0 it is (|A| |B|)_ij.

8-bit float inputs: the gfx950 8-bit matrix instruction does not add its
products at fp32 precision.  Measured on the hardware (one-element probes of
1 + x with x at every position of a 64-deep instruction): within each group
of 8 consecutive k, a product smaller than 2^-13 of the group's largest is
cut off below that point, while products in different groups combine at
fp32 precision.  The error this adds is below 7 * 2^-13 * (largest |product|
of each group), summed over the groups, hence below 7 * 2^-13 * den =
8.5e-4 * den; with the fp32 additions on top, the bound used is F8_DOT =
1e-3 * den.  So an 8-bit GEMM with fp32 output is held to the same 1e-3
normalised bound as bf16/fp16 inputs, and every element of a 16-bit output
must lie within 2 ulp + F8_DOT * den of the oracle (no condition on
|ref|: the truncation does not depend on cancellation).  Products of small
integers fall inside the window, so integer data must still be bit-exact.
"""
import sys
from dataclasses import dataclass

import numpy as np
import torch

import oracle
import workloads
from dense_gemm_optimisation_amd import binding

# 8-bit products, like bf16/fp16 ones, are exact in fp32: the same bound.
TOL = {("f32", "f32"): 1e-4, ("bf16", "f32"): 1e-3, ("f16", "f32"): 1e-3,
       ("e4m3", "f32"): 1e-3, ("e5m2", "f32"): 1e-3}
F8_DOT = 1e-3  # bound on the 8-bit instruction's dot-product error, relative to den
GUARD = 96  # guard elements before and after each buffer (keeps data 16-byte aligned)
CANARY = {"f32": np.uint32(0x7FC0DEAD), "bf16": np.uint16(0x7FC1), "f16": np.uint16(0x7E1D),
          "e4m3": np.uint8(0x7F), "e5m2": np.uint8(0x7E)}
STORE = {"f32": np.uint32, "bf16": np.uint16, "f16": np.uint16, "e4m3": np.uint8,
         "e5m2": np.uint8}
SIGNED = {np.uint32: np.int32, np.uint16: np.int16, np.uint8: np.int8}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def offsets(p: workloads.Problem, which: str, b, i, j) -> np.ndarray:
    """Flat element offsets of entries (b, i, j) of a batched operand."""
    r, c, order, ld = p.dims(which)
    stride = {"a": p.stride_a, "b": p.stride_b, "c": p.stride_c}[which]
    b, i, j = (np.asarray(x, np.int64) for x in (b, i, j))
    return b * stride + (i * ld + j if order == workloads.ROW else j * ld + i)


def matrix_mask(p: workloads.Problem, which: str, size: int) -> np.ndarray:
    """Boolean mask of the buffer elements that belong to the matrix."""
    r, c, order, ld = p.dims(which)
    mask = np.zeros(size, bool)
    outer, inner = (r, c) if order == workloads.ROW else (c, r)
    stride = {"a": p.stride_a, "b": p.stride_b, "c": p.stride_c}[which]
    for b in range(p.batch):
        base = b * stride
        if inner == ld:
            mask[base:base + outer * inner] = True
        else:
            for o in range(outer):
                mask[base + o * ld:base + o * ld + inner] = True
    return mask


def _bits(arr, dtype):
    return arr.view(STORE[dtype])


def _device(host, dtype, shift=0):
    """Device buffer: GUARD canary elements, the host data, GUARD canaries.

    The data starts `shift` elements before the end of the leading guard band
    so that a caller can hand the library a base pointer that is not 16-byte
    aligned.  Returns (device tensor, host image of the buffer, data start).
    """
    store = STORE[dtype]
    full = np.empty(host.size + 2 * GUARD, store)
    full[:] = CANARY[dtype]
    start = GUARD - shift
    full[start:start + host.size] = _bits(host, dtype)
    t = torch.from_numpy(full.view(SIGNED[store])).to("cuda")
    return t, full, start


@dataclass
class Result:
    name: str
    max_err: float = 0.0          # max normalised error (fp32 output)
    max_ulp: int = 0              # max ulp distance (16-bit output)
    strict_fail: int = 0          # 16-bit elements beyond 2 ulp
    exempt: int = 0               # ... of which accepted as cancellations
    checked: int = 0
    kernel: str = ""              # the kernel the library launched
    ok: bool = True
    why: str = ""


def ulp_keys(bits16: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns to integers ordered like their values (+0 == -0)."""
    b = bits16.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def compare(p, got_bits: np.ndarray, ref: np.ndarray, den: np.ndarray, name: str) -> Result:
    """got_bits: output patterns at the compared elements; ref, den from the oracle.
    A block-scaled problem (workloads.MxProblem) runs on the 8-bit matrix
    instruction and is held to its rule."""
    res = Result(name=name, checked=int(ref.size))
    out = p.c_dtype
    narrow = isinstance(p, workloads.MxProblem) or p.in_dtype in workloads.EIGHT_BIT
    if out == "f32":
        got = got_bits.view(np.float32).astype(np.float64)
        tol = F8_DOT if narrow else TOL[(p.in_dtype, "f32")]
        zero = den == 0
        if np.any(zero & (got != ref)):
            res.ok, res.why = False, "den == 0 but result differs from ref"
        with np.errstate(divide="ignore", invalid="ignore"):
            err = np.where(zero, 0.0, np.abs(got - ref) / np.where(zero, 1.0, den))
        err = np.where(np.isnan(got) & ~np.isnan(ref), np.inf, err)
        res.max_err = float(np.max(err)) if err.size else 0.0
        if not res.max_err <= tol:
            res.ok = False
            k = int(np.argmax(err))
            res.why = f"max normalised error {res.max_err:.3e} > {tol:g} at flat {k}: " \
                      f"got {got.ravel()[k]!r} ref {ref.ravel()[k]!r} den {den.ravel()[k]!r}"
        return res
    if out in workloads.EIGHT_BIT:
        return compare8(p, got_bits, ref, den, name, res)
    ref_q = oracle.round_bits(out, ref)
    d = np.abs(ulp_keys(got_bits) - ulp_keys(ref_q))
    res.max_ulp = int(d.max()) if d.size else 0
    bad = d > 2
    res.strict_fail = int(bad.sum())
    if res.strict_fail:
        got = oracle.decode(out, got_bits)
        qv = oracle.decode(out, ref_q)
        ulp = np.abs(oracle.decode(out, (ref_q.astype(np.int64) + 1).astype(np.uint16)) - qv)
        if narrow:
            ok_exempt = np.abs(got - ref) <= 2 * ulp + F8_DOT * den
        else:
            ok_exempt = (np.abs(got - ref) <= 2 * ulp + 1e-3 * den) & \
                (np.abs(ref) <= 2.0 ** -8 * den)
        res.exempt = int((bad & ok_exempt).sum())
        if res.exempt != res.strict_fail:
            res.ok = False
            k = int(np.argmax(bad & ~ok_exempt))
            res.why = (f"{res.strict_fail - res.exempt} elements beyond 2 ulp; e.g. flat {k}: "
                       f"got {got.ravel()[k]!r} ref {ref.ravel()[k]!r} den {den.ravel()[k]!r}")
    zero = den == 0
    if np.any(zero & (ulp_keys(got_bits) != ulp_keys(ref_q))):
        res.ok, res.why = False, "den == 0 but result differs from ref"
    return res


def keys8(bits):
    """8-bit sign-magnitude patterns as integers that step by one per
    representable value (+0 and -0 both 0)."""
    b = np.asarray(bits).astype(np.int64) & 0xFF
    return np.where(b & 0x80, -(b & 0x7F), b & 0x7F)


def compare8(p, got_bits, ref, den, name, res):
    """8-bit (quantised) output against the oracle's exact value ref (already
    scaled).  The kernel rounds its fp32 value, which is within the 16-bit
    inputs' fp32 error of ref; rounding that to the format can differ from
    rounding ref only where ref lies near the middle of two neighbours: at
    most one step (ulp) apart, and NaN exactly where ref is NaN.  As for
    16-bit outputs, an element under cancellation (|ref| <= 2^-8 den) may
    instead be within one ulp plus 1e-3 den of ref."""
    out = p.c_dtype
    got_bits = np.asarray(got_bits).astype(np.uint8)
    got = oracle.decode(out, got_bits)
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    if np.any(nan_ref != nan_got):
        k = int(np.argmax(nan_ref != nan_got))
        res.ok, res.why = False, f"NaN mismatch at flat {k}: got {got.ravel()[k]!r} ref {ref.ravel()[k]!r}"
        return res
    ok = ~nan_ref
    ref_q = oracle.round_bits(out, ref[ok])
    d = np.abs(keys8(got_bits[ok]) - keys8(ref_q))
    res.max_ulp = int(d.max()) if d.size else 0
    bad = d > 1
    res.strict_fail = int(bad.sum())
    if res.strict_fail:
        qv = oracle.decode(out, ref_q)
        step = np.abs(oracle.decode(out, (ref_q.astype(np.int64) + 1).astype(np.uint8)) - qv)
        ok_exempt = (np.abs(got[ok] - ref[ok]) <= step + 1e-3 * den[ok]) & \
            (np.abs(ref[ok]) <= 2.0 ** -8 * den[ok])
        res.exempt = int((bad & ok_exempt).sum())
        if res.exempt != res.strict_fail:
            res.ok = False
            k = int(np.argmax(bad & ~ok_exempt))
            res.why = (f"{res.strict_fail - res.exempt} elements beyond 1 ulp; e.g. flat {k}: "
                       f"got {got[ok][k]!r} ref {ref[ok][k]!r} den {den[ok][k]!r}")
    return res


def default_sample(p: workloads.Problem, rng, n_random=4096):
    """Elements checked at full size: whole first/last rows and columns of the
    first and last batch, tile-boundary rows/columns, and random elements."""
    idx = []
    for b in sorted({0, p.batch - 1}):
        for i in sorted({0, p.M - 1, p.M // 2}):
            js = np.arange(p.N)
            idx.append(np.stack([np.full_like(js, b), np.full_like(js, i), js], 1))
        for j in sorted({0, p.N - 1, p.N // 3}):
            is_ = np.arange(p.M)
            idx.append(np.stack([np.full_like(is_, b), is_, np.full_like(is_, j)], 1))
        for t in (127, 128, 255, 256):
            if t < p.M and t < p.N:
                idx.append(np.array([[b, t, t], [b, t, p.N - 1], [b, p.M - 1, t]]))
    idx.append(np.stack([rng.integers(0, p.batch, n_random), rng.integers(0, p.M, n_random),
                         rng.integers(0, p.N, n_random)], 1))
    idx = np.unique(np.concatenate(idx).astype(np.int64), axis=0)
    return idx


_WORKSPACE = []


def workspace():
    """One device workspace of gemm_workspace_size() bytes, shared by the
    tests (each call reuses it, as a caller would), filled with NaN patterns
    so that a partial tile read before it was written shows up."""
    if not _WORKSPACE:
        n = binding.workspace_size()
        _WORKSPACE.append(torch.full((n // 4,), -1, dtype=torch.int32, device="cuda"))
    return _WORKSPACE[0]


def run(p: workloads.Problem, *, seed=None, host=None, sample=None, c_init=None,
        base_offset=(0, 0, 0), repeat=1, bias_host=None, use_workspace=False, workspace_bytes=None):
    """Run p on the GPU (optionally `repeat` times) and compare with the oracle.

    host: (A, B, C0) host buffers, else generated from the workload recipe.
    bias_host: the bias buffer of a fused-epilogue problem, else generated.
    sample: None for every element, "auto" for default_sample, or an index array.
    c_init: a value written over the whole initial C (e.g. NaN when beta == 0).
    base_offset: elements by which each device base pointer is shifted (to
    test misaligned bases).
    use_workspace: call the workspace entry point (gemm_f32_ws, gemm_bf16_ws,
    gemm_f16_ws, gemm_f8_ws) with the shared workspace, of workspace_bytes
    bytes (default: all of it).
    Returns (Result, output bits of the whole C buffer including guards).
    """
    log(f"[parity] {p.name} {p.in_dtype}->{p.c_dtype} M={p.M} N={p.N} K={p.K} "
        f"batch={p.batch} orders={p.order_a}{p.order_b}{p.order_c} "
        f"ld={p.lda},{p.ldb},{p.ldc} alpha={p.alpha} beta={p.beta} bias={p.bias} act={p.act}")
    a, b, c0 = host if host is not None else workloads.generate(p, seed)
    if c_init is not None:
        c0 = np.full_like(c0, c_init)
    bias = bias_host if bias_host is not None else workloads.bias_vector(p, seed)
    da, fa, sa = _device(a, p.in_dtype, base_offset[0])
    db, fb, sb = _device(b, p.b_dtype, base_offset[1])
    dc, fc, sc = _device(c0, p.c_dtype, base_offset[2])
    if bias is not None:
        dbias, fbias, sbias = _device(bias, p.in_dtype)
    esz_in = np.dtype(STORE[p.in_dtype]).itemsize
    esz_b = np.dtype(STORE[p.b_dtype]).itemsize
    esz_out = {"f32": 4, "e4m3": 1, "e5m2": 1}.get(p.c_dtype, 2)
    pa, pb, pc = (da.data_ptr() + sa * esz_in, db.data_ptr() + sb * esz_b,
                  dc.data_ptr() + sc * esz_out)
    pbias = dbias.data_ptr() + sbias * esz_in if bias is not None else None
    c_dt = binding.DTYPE_F32 if (p.c_dtype == "f32" and p.in_dtype != "f32") else binding.DTYPE_SAME
    ws = {}
    if use_workspace:
        w = workspace()
        ws = dict(workspace=w.data_ptr(),
                  workspace_bytes=w.numel() * 4 if workspace_bytes is None else workspace_bytes)
    cview = {"f32": np.int32, "e4m3": np.int8, "e5m2": np.int8}.get(p.c_dtype, np.int16)
    kernel = binding.kernel_name(p.in_dtype, p.M, p.N, p.K, p.alpha, pa, p.lda, p.order_a, pb,
                                 p.ldb, p.order_b, p.beta, pc, p.ldc, p.order_c, c_dt, p.batch,
                                 p.stride_a, p.stride_b, p.stride_c, b_dtype=p.b_dtype,
                                 out_dtype=p.c_dtype, **ws)
    valu = p.entry == "valu"  # gemm_f32_valu runs the vector-ALU kernel whatever the shape
    if valu and kernel not in ("", "scale", None):
        kernel = "sgemm_valu"
    quant = p.entry == "quant"
    if quant:
        kernel = binding.kernel_name_quant(p.in_dtype, p.M, p.N, p.K, p.alpha, pa, p.lda,
                                           p.order_a, pb, p.ldb, p.order_b, pc, p.ldc, p.order_c,
                                           p.c_dtype, p.batch, p.stride_a, p.stride_b,
                                           p.stride_c)
    x3 = {}
    if p.entry == "bf16x3":  # gemm_f32_bf16x3, with a workspace of its own
        n = binding.bf16x3_workspace_size(p.M, p.N, p.K, p.batch)
        w3 = torch.empty(max(n, 256) // 4 + 64, dtype=torch.int32, device="cuda")
        x3 = dict(workspace=w3.data_ptr(), workspace_bytes=n if workspace_bytes is None
                  else workspace_bytes)
        kernel = binding.kernel_name_bf16x3(p.M, p.N, p.K, p.alpha, pa, p.lda, p.order_a, pb,
                                            p.ldb, p.order_b, p.beta, pc, p.ldc, p.order_c,
                                            p.batch, p.stride_a, p.stride_b, p.stride_c, **x3)
    outs = []
    for r in range(repeat):
        if r:
            dc.copy_(torch.from_numpy(fc.view(cview)))
        if quant:
            binding.gemm_quant(p.in_dtype, p.M, p.N, p.K, p.alpha, pa, p.lda, p.order_a, pb, p.ldb,
                               p.order_b, pc, p.ldc, p.order_c, p.c_dtype, p.c_scale, p.batch,
                               p.stride_a, p.stride_b, p.stride_c, bias=pbias,
                               stride_bias=p.stride_bias or 0, act=p.act)
        elif x3:
            binding.gemm_f32_bf16x3(p.M, p.N, p.K, p.alpha, pa, p.lda, p.order_a, pb, p.ldb,
                                    p.order_b, p.beta, pc, p.ldc, p.order_c, p.batch,
                                    p.stride_a, p.stride_b, p.stride_c, **x3)
        else:
            binding.gemm(p.in_dtype, p.M, p.N, p.K, p.alpha, pa, p.lda, p.order_a, pb, p.ldb,
                         p.order_b, p.beta, pc, p.ldc, p.order_c, c_dt, p.batch, p.stride_a,
                         p.stride_b, p.stride_c, bias=pbias, stride_bias=p.stride_bias,
                         act=p.act, b_dtype=p.b_dtype, out_dtype=p.c_dtype, valu=valu, **ws)
        torch.cuda.synchronize()
        outs.append(dc.cpu().numpy().view(fc.dtype).copy())
    out = outs[0]
    res = Result(name=p.name, kernel=kernel)
    if any(not np.array_equal(o, out) for o in outs[1:]):
        res.ok, res.why = False, "repeated runs differ"
        return res, out
    if not (np.array_equal(da.cpu().numpy().view(fa.dtype), fa)
            and np.array_equal(db.cpu().numpy().view(fb.dtype), fb)
            and (bias is None or np.array_equal(dbias.cpu().numpy().view(fbias.dtype), fbias))):
        res.ok, res.why = False, "A, B or the bias was modified"
        return res, out
    # everything outside the matrix C is bit-unchanged
    outside = np.ones(out.size, bool)
    outside[sc:sc + c0.size] = ~matrix_mask(p, "c", c0.size)
    if not np.array_equal(out[outside], fc[outside]):
        k = int(np.flatnonzero(outside & (out != fc))[0])
        res.ok, res.why = False, f"write outside C at buffer element {k} (data starts at {sc})"
        log(f"[parity]   -> FAIL {res.why}")
        return res, out
    kw = dict(stride_a=p.stride_a, stride_b=p.stride_b, stride_c=p.stride_c, bias=bias,
              stride_bias=p.stride_bias, act=p.act, b_dtype=p.b_dtype)
    odt, oc0 = p.c_dtype, c0
    if quant:  # no beta: the oracle's fp64 value, scaled, against the 8-bit rounding
        odt, oc0 = "f32", np.zeros(c0.size, np.float32)
    if sample is None:
        ref, den = oracle.gemm(p.in_dtype, odt, p.M, p.N, p.K, p.alpha, a, p.lda, p.order_a,
                               b, p.ldb, p.order_b, 0.0 if quant else p.beta, oc0, p.ldc,
                               p.order_c, batch=p.batch, **kw)
        bb, ii, jj = np.meshgrid(np.arange(p.batch), np.arange(p.M), np.arange(p.N),
                                 indexing="ij")
    else:
        idx = default_sample(p, np.random.default_rng(1234)) if isinstance(sample, str) else sample
        ref, den = oracle.gemm_at(p.in_dtype, odt, p.M, p.N, p.K, p.alpha, a, p.lda,
                                  p.order_a, b, p.ldb, p.order_b, 0.0 if quant else p.beta, oc0,
                                  p.ldc, p.order_c, idx, **kw)
        bb, ii, jj = idx[:, 0], idx[:, 1], idx[:, 2]
    got = out[sc + offsets(p, "c", bb, ii, jj)]
    if quant:
        ref, den = p.c_scale * ref, abs(p.c_scale) * den
    res = compare(p, got, ref, den, p.name)
    res.kernel = kernel
    log(f"[parity]   -> {kernel} ok={res.ok} max_err={res.max_err:.3e} max_ulp={res.max_ulp} "
        f"strict_fail={res.strict_fail} exempt={res.exempt} checked={res.checked} {res.why}")
    return res, out


# Element patterns of small integers (magnitudes 0, 1, 2, 3, 4, 6) in each MX
# element format, and the sign bit: products of two of them times scales of
# 2^-1 .. 2^1 are multiples of 2^-2 below 2^8, exact in the 8-bit matrix
# instruction's window and in fp32.
MX_INT = {"e2m1": ({0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 6: 7}, 8),
          "e2m3": ({0: 0, 1: 8, 2: 16, 3: 20, 4: 24, 6: 28}, 32),
          "e3m2": ({0: 0, 1: 12, 2: 16, 3: 18, 4: 20, 6: 22}, 32),
          "e4m3": ({0: 0, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 6: 0x4C}, 128),
          "e5m2": ({0: 0, 1: 0x3C, 2: 0x40, 3: 0x42, 4: 0x44, 6: 0x46}, 128)}


def mx_int_patterns(rng, fmt, batch, rows, K):
    table, sign = MX_INT[fmt]
    mags = np.array(sorted(table))
    v = rng.choice(mags, (batch, rows, K))
    neg = rng.integers(0, 2, (batch, rows, K)).astype(bool)
    lut = np.zeros(7, np.uint8)
    for m, code in table.items():
        lut[m] = code
    return (lut[v] | np.where(neg, sign, 0)).astype(np.uint8)


def run_mx(p: "workloads.MxProblem", *, seed=None, sample=None, repeat=1, patterns=None,
           use_workspace=False):
    """Run a block-scaled problem through gemm_mx (gemm_mx_ws with the shared
    workspace when use_workspace) and compare with the oracle (every element,
    or `sample` as in run()).  patterns: optional element patterns for A and
    B (see workloads.generate_mx)."""
    log(f"[parity] {p.name} mx {p.fa}x{p.fb}->{p.c_dtype} M={p.M} N={p.N} K={p.K} "
        f"batch={p.batch} orderC={p.order_c} ld={p.lda},{p.ldb},{p.ldc} lds={p.ldsa},{p.ldsb} "
        f"alpha={p.alpha} beta={p.beta}")
    a, sa, b, sb, c0 = workloads.generate_mx(p, seed, patterns)
    ins = [torch.from_numpy(x.view(np.int8)).to("cuda") if x.size else
           torch.zeros(16, dtype=torch.int8, device="cuda") for x in (a, sa, b, sb)]
    da, dsa, db, dsb = ins
    dc, fc, sc = _device(c0, p.c_dtype)
    esz_out = 4 if p.c_dtype == "f32" else 2
    pc = dc.data_ptr() + sc * esz_out
    out_t = {"f32": binding.OUTPUT_F32, "bf16": binding.OUTPUT_BF16, "f16": binding.OUTPUT_F16}
    args = (p.M, p.N, p.K, p.alpha, da.data_ptr(), p.lda, binding.MX_FORMAT[p.fa], dsa.data_ptr(),
            p.ldsa, db.data_ptr(), p.ldb, binding.MX_FORMAT[p.fb], dsb.data_ptr(), p.ldsb, p.beta,
            pc, p.ldc, p.order_c, out_t[p.c_dtype], p.batch, p.stride_a, p.stride_b, p.stride_sa,
            p.stride_sb, p.stride_c)
    ws = {}
    if use_workspace:
        w = workspace()
        ws = dict(workspace=w.data_ptr(), workspace_bytes=w.numel() * 4)
    kernel = binding.mx_kernel_name(*args, **ws)
    cview = np.int32 if p.c_dtype == "f32" else np.int16
    outs = []
    for r in range(repeat):
        if r:
            dc.copy_(torch.from_numpy(fc.view(cview)))
        if use_workspace:
            binding.gemm_mx_ws(*args, ws["workspace"], ws["workspace_bytes"])
        else:
            binding.gemm_mx(*args)
        torch.cuda.synchronize()
        outs.append(dc.cpu().numpy().view(fc.dtype).copy())
    out = outs[0]
    res = Result(name=p.name, kernel=kernel or "")
    if any(not np.array_equal(o, out) for o in outs[1:]):
        res.ok, res.why = False, "repeated runs differ"
        return res, out
    for t, h in zip(ins, (a, sa, b, sb)):
        if h.size and not np.array_equal(t.cpu().numpy().view(np.uint8), h):
            res.ok, res.why = False, "an operand or a scale array was modified"
            return res, out
    outside = np.ones(out.size, bool)
    outside[sc:sc + c0.size] = ~matrix_mask(p, "c", c0.size)
    if not np.array_equal(out[outside], fc[outside]):
        k = int(np.flatnonzero(outside & (out != fc))[0])
        res.ok, res.why = False, f"write outside C at buffer element {k} (data starts at {sc})"
        log(f"[parity]   -> FAIL {res.why}")
        return res, out
    okw = dict(stride_a=p.stride_a, stride_b=p.stride_b, stride_sa=p.stride_sa,
               stride_sb=p.stride_sb, stride_c=p.stride_c)
    oargs = (p.fa, p.fb, p.c_dtype, p.M, p.N, p.K, p.alpha, a, p.lda, sa, p.ldsa, b, p.ldb, sb,
             p.ldsb, p.beta, c0, p.ldc, p.order_c)
    if sample is None:
        ref, den = oracle.mx_gemm(*oargs, batch=p.batch, **okw)
        bb, ii, jj = np.meshgrid(np.arange(p.batch), np.arange(p.M), np.arange(p.N),
                                 indexing="ij")
    else:
        idx = default_sample(p, np.random.default_rng(1234)) if isinstance(sample, str) else sample
        ref, den = oracle.mx_gemm_at(*oargs, idx, **okw)
        bb, ii, jj = idx[:, 0], idx[:, 1], idx[:, 2]
    got = out[sc + offsets(p, "c", bb, ii, jj)]
    res = compare(p, got, ref, den, p.name)
    res.kernel = kernel or ""
    log(f"[parity]   -> {kernel} ok={res.ok} max_err={res.max_err:.3e} max_ulp={res.max_ulp} "
        f"strict_fail={res.strict_fail} exempt={res.exempt} checked={res.checked} {res.why}")
    return res, out
