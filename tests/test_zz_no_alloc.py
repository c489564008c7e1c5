"""gemm_bf16_noalloc (the entry point that allocates nothing: the library's
per-device scratch array in place of a caller workspace) against gemm_bf16_ws
with a full workspace, through the C ABI: the same plan runs, so the outputs
must be bit-identical; both are also held to the oracle's tolerance.  Two
calls in a row, the second with a smaller input, so the second reuses the
scratch the first left behind."""
import numpy as np
import pytest
import torch

import workloads
from dense_gemm_optimisation_amd import binding
from workloads import COL, ROW, Problem

from parity import _device, compare, log, workspace
import oracle

pytestmark = pytest.mark.gpu


def _run_both(p, seed):
    a, b, c0 = workloads.generate(p, seed)
    outs = []
    for which in ("ws", "noalloc"):
        da, _, sa = _device(a, p.in_dtype)
        db, _, sb = _device(b, p.in_dtype)
        dc, fc, sc = _device(c0, p.c_dtype)
        esz_c = 4 if p.c_dtype == "f32" else 2
        pa, pb, pc = da.data_ptr() + 2 * sa, db.data_ptr() + 2 * sb, dc.data_ptr() + esz_c * sc
        c_dt = binding.DTYPE_F32 if p.c_dtype == "f32" else binding.DTYPE_SAME
        args = (p.M, p.N, p.K, p.alpha, pa, p.lda, p.order_a, pb, p.ldb, p.order_b, p.beta, pc,
                p.ldc, p.order_c, c_dt, p.batch, p.stride_a, p.stride_b, p.stride_c)
        if which == "ws":
            w = workspace()
            kernel = binding.kernel_name(p.in_dtype, *args, workspace=w.data_ptr(),
                                         workspace_bytes=w.numel() * 4)
            binding.gemm_bf16_ws(*args, workspace=w.data_ptr(), workspace_bytes=w.numel() * 4)
        else:
            binding.gemm_bf16_noalloc(*args)
        torch.cuda.synchronize()
        outs.append(dc.cpu().numpy().view(fc.dtype).copy())
    log(f"[noalloc] {p.name} M={p.M} N={p.N} K={p.K} batch={p.batch}: {kernel}")
    assert np.array_equal(outs[0], outs[1]), f"{p.name}: gemm_bf16_noalloc differs from gemm_bf16_ws"
    # and the result is the product, to the oracle's tolerance
    bb, ii, jj = np.meshgrid(np.arange(p.batch), np.arange(p.M), np.arange(p.N), indexing="ij")
    ref, den = oracle.gemm(p.in_dtype, p.c_dtype, p.M, p.N, p.K, p.alpha, a, p.lda, p.order_a, b,
                           p.ldb, p.order_b, p.beta, c0, p.ldc, p.order_c, batch=p.batch,
                           stride_a=p.stride_a, stride_b=p.stride_b, stride_c=p.stride_c)
    from parity import offsets
    got = outs[1][sc + offsets(p, "c", bb, ii, jj)]
    res = compare(p, got, ref, den, p.name)
    assert res.ok, res.why
    return kernel


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 65 batches of 300 x 290 x 501, operands copied into the
    # scratch, then the direct-load stream-K schedule with its partial tiles
    # there too (about 49 MB of the 64 MiB); second, smaller: unaligned
    # 2047 x 2049 x 1001, copied for the direct-load kernel (8 MB)
    k1 = _run_both(Problem("noalloc-1", "bf16", "bf16", 300, 290, 501, beta=0.5, batch=65,
                           order_b=COL), seed=201)
    k2 = _run_both(Problem("noalloc-2", "bf16", "bf16", 2047, 2049, 1001, alpha=0.75, beta=0.5),
                   seed=202)
    assert k1 == "hgemm_mfma_dma_streamk_packed" and k2 == "hgemm_mfma_dma_packed"


def test_noalloc_refusal_leaves_c_untouched():
    # 65 batches of 300 x 290 x 1001 would use 92 MB: refused, nothing launched
    p = Problem("noalloc-big", "bf16", "bf16", 300, 290, 1001, beta=0.5, batch=65, order_b=COL)
    a, b, c0 = workloads.generate(p, 205)
    da, _, sa = _device(a, "bf16")
    db, _, sb = _device(b, "bf16")
    dc, fc, sc = _device(c0, "bf16")
    st = binding.gemm_bf16_noalloc(p.M, p.N, p.K, p.alpha, da.data_ptr() + 2 * sa, p.lda,
                                   p.order_a, db.data_ptr() + 2 * sb, p.ldb, p.order_b, p.beta,
                                   dc.data_ptr() + 2 * sc, p.ldc, p.order_c, binding.DTYPE_SAME,
                                   p.batch, p.stride_a, p.stride_b, p.stride_c,
                                   raise_on_error=False)
    torch.cuda.synchronize()
    assert st == binding.ERR_SCRATCH
    assert np.array_equal(dc.cpu().numpy().view(fc.dtype), fc)


def test_noalloc_without_scratch_use_and_fp32_output():
    # aligned whole waves: no scratch needed; then fp32 output on the
    # general kernel's stream-K schedule (4 tiles of 47 k-steps)
    k1 = _run_both(Problem("noalloc-3", "bf16", "bf16", 512, 512, 512, beta=0.5), seed=203)
    k2 = _run_both(Problem("noalloc-4", "bf16", "f32", 300, 290, 3001, beta=1.0), seed=204)
    assert k1 == "hgemm_splitk" and k2 == "hgemm_mfma_streamk"
