"""Throughput of libgemm on one MI355X: TFLOPS = 2*M*N*K / t.

A step is one pass of the whole path over the headline workload: one fp32
SGEMM, one bf16 HGEMM and one fp16 HGEMM, each 4096 x 4096 x 4096, row-major,
alpha = 1, beta = 0 (the square 4096 problem the pages benchmark; inputs
U[-1, 1] for fp32 and N(0, 1) rounded to bf16/fp16, generated on the host and
resident in HBM before timing starts).  `value` is the step's whole-job
throughput (three GEMMs' FLOPs over the step's wall time); `per_kernel` gives
each GEMM's own TFLOPS and fraction of MI355X's dense peak for its dtype,
from HIP events recorded on the stream the kernels run on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--no-context] [--no-rotate] [--no-clocks]
                       [--copy-calibration MiB] [--workspace] [--results FILE]
Each kernel cycles through at least three copies of its buffers, enough that
their footprint exceeds twice the 256 MB MALL, so inputs come from HBM;
--no-rotate reuses one set (the warm-cache figure).
--workload runs the named workload, or a comma-separated list of them (see
workloads.CONFIGS), instead of the headline step, for profiling.  --workspace
runs the workloads without a fused epilogue through the workspace entry
points, which use the stream-K schedule where it applies.  --copy-calibration runs only a plain
device-to-device copy of the given size (the reference kernel against which
the HBM byte counters FETCH_SIZE / WRITE_SIZE are scaled).

Besides the back-to-back mean that `value` uses, each kernel is also timed
launch by launch (its own event pair around each of --launch-samples
launches) for the median and the minimum.  With amd-smi present, the gfx
clock, power and temperatures are read before the run, while each kernel runs
in a loop, and after.  The CPU baseline runs the oracle once per workload
(all rows, or the first rows that fit the time budget, as stated in its
`sample`), the 256^3 problem as the median of 10 and once on one thread, and
records the CPU model; the same oracle values give the error statistics of
the GPU result on those rows.

The roofline's `traffic` is the dominant kernel's HBM bytes per launch, read
from profiles/hbm_traffic.txt (counters taken with rocprofv3 --pmc, scaled by
the copy calibration).  Each entry records a hash of the kernel source it was
measured on; when the source has changed since, `traffic` is null.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense peaks, published (8-bit floats: twice the 16-bit rate; the
# block-scaled 6- and 4-bit formats twice the 8-bit one)
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2,
               "mxfp8": 5033.2, "mxfp6": 10066.3, "mxfp4": 10066.3,
               # fp32 through three bf16 products: the bf16 peak over three, in
               # fp32-equivalent flops (2MNK)
               "f32_bf16x3": 2516.6 / 3}
ESIZE = {"f32": 4, "bf16": 2, "f16": 2, "e4m3": 1, "e5m2": 1}
VIEW = {"f32": np.float32, "bf16": np.int16, "f16": np.int16, "e4m3": np.int8, "e5m2": np.int8}
HBM_GBS = 8000.0

HEADLINE = ["f32_4096", "bf16_4096", "f16_4096"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
# kernel family -> the source file that defines it (hashed to detect changes)
KERNEL_SOURCE = {"sgemm_mfma_dma": "sgemm_mfma.hip", "sgemm_mfma": "sgemm_mfma.hip",
                 "sgemm_valu": "sgemm_valu.hip", "hgemm_mfma_dma": "hgemm_mfma_dma.hip",
                 "hgemm_mfma": "hgemm_mfma.hip", "hgemm_splitk": "hgemm_splitk.hip",
                 "sgemm_splitk": "sgemm_splitk.hip", "gemm_skinny": "gemm_skinny.hip",
                 "f8gemm_mfma_dma": "f8gemm_mfma.hip", "f8gemm_mfma": "f8gemm_mfma.hip",
                 "hgemm_mfma_streamk": "hgemm_mfma.hip", "hgemm_mfma_dma_streamk": "hgemm_mfma_dma.hip",
                 "sgemm_mfma_streamk": "sgemm_mfma.hip",
                 "hgemm_mfma_dma_packed": "hgemm_mfma_dma.hip",
                 "hgemm_mfma_dma_streamk_packed": "hgemm_mfma_dma.hip",
                 "sgemm_mfma_dma_packed": "sgemm_mfma.hip",
                 "sgemm_mfma_dma_streamk": "sgemm_mfma.hip",
                 "sgemm_mfma_dma_streamk_packed": "sgemm_mfma.hip",
                 "mxgemm_mfma_dma": "mxgemm.hip",
                 "f8gemm_mfma_dma_streamk": "f8gemm_mfma.hip",
                 "mxgemm_mfma_dma_streamk": "mxgemm.hip",
                 "gemm_skinny_splitk": "gemm_skinny.hip",
                 "scale": "scale.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def is_mx(p):
    import workloads
    return isinstance(p, workloads.MxProblem)


def dtype_key(p):
    """The key of PEAK_TFLOPS for a workload: its input type, mxfp8/6/4, or
    f32_bf16x3 for fp32 through split bf16 products."""
    import workloads
    if is_mx(p):
        return f"mxfp{workloads.MX_WIDTH[p.fa]}"
    return "f32_bf16x3" if p.entry == "bf16x3" else p.in_dtype


def algorithmic_bytes(p):
    """Bytes a launch must move at least: A and B once (with their scales),
    C written once and, when beta != 0, read once."""
    import workloads
    c = p.M * p.N * ESIZE[p.c_dtype] * p.batch * (2 if p.beta else 1)
    if is_mx(p):
        wa, wb = workloads.MX_WIDTH[p.fa], workloads.MX_WIDTH[p.fb]
        return (p.M * p.K * wa // 8 + p.N * p.K * wb // 8 + (p.M + p.N) * (p.K // 32)) * p.batch + c
    return (p.M * p.K * ESIZE[p.in_dtype] + p.K * p.N * ESIZE[p.b_dtype]) * p.batch + c


def device_buffers(p, torch):
    import workloads
    if is_mx(p):
        a, sa, b, sb, c = workloads.generate_mx(p)
        return tuple(torch.from_numpy(x.view(np.int8)).to("cuda") for x in (a, sa, b, sb)) + \
            (torch.from_numpy(c.view(VIEW[p.c_dtype])).to("cuda"),)
    a, b, c = workloads.generate(p)
    return (torch.from_numpy(a.view(VIEW[p.in_dtype])).to("cuda"),
            torch.from_numpy(b.view(VIEW[p.b_dtype])).to("cuda"),
            torch.from_numpy(c.view(VIEW[p.c_dtype])).to("cuda"))


def device_bias(p, torch):
    """The bias vector of a fused-epilogue workload on the device, or None."""
    import workloads
    bias = workloads.bias_vector(p)
    if bias is None:
        return None
    return torch.from_numpy(bias.view(np.float32 if p.in_dtype == "f32" else np.int16)).to("cuda")


# Each kernel cycles through enough copies of its buffers that their combined
# footprint exceeds twice the 256 MB Infinity Cache (MALL), so a launch finds
# its inputs in HBM rather than left in the MALL by the previous launch.
ROTATE_BYTES = 600_000_000
MIN_SETS, MAX_SETS = 3, 16


def buffer_sets(bufs, n):
    """`bufs` plus n - 1 device copies of it (same values, other addresses)."""
    return [bufs] + [tuple(t.clone() for t in bufs) for _ in range(n - 1)]


def sets_needed(bufs, rotate):
    if not rotate:
        return 1
    nbytes = sum(t.numel() * t.element_size() for t in bufs)
    return min(MAX_SETS, max(MIN_SETS, -(-ROTATE_BYTES // nbytes)))


def make_launch(p, sets, stream, bias=None, workspace=None):
    """A callable that runs the GEMM on the next buffer set in turn (with the
    workload's fused bias and activation, if it has them; through the
    workspace entry point when a workspace tensor is given)."""
    from dense_gemm_optimisation_amd import binding
    if is_mx(p):
        return make_mx_launch(p, sets, stream, workspace)
    c_dt = binding.DTYPE_F32 if (p.c_dtype == "f32" and p.in_dtype != "f32") else binding.DTYPE_SAME
    argsets = [(p.in_dtype, p.M, p.N, p.K, p.alpha, da.data_ptr(), p.lda, p.order_a, db.data_ptr(),
                p.ldb, p.order_b, p.beta, dc.data_ptr(), p.ldc, p.order_c, c_dt, p.batch,
                p.stride_a, p.stride_b, p.stride_c, stream.cuda_stream) for da, db, dc in sets]
    epi = dict(bias=None if bias is None else bias.data_ptr(), stride_bias=p.stride_bias,
               act=p.act, b_dtype=p.b_dtype, out_dtype=p.c_dtype, valu=p.entry == "valu")
    if workspace is not None:
        epi.update(workspace=workspace.data_ptr(), workspace_bytes=workspace.numel() * 4)
    turn = [0]
    if p.entry == "quant":
        def launch():
            a = argsets[turn[0]]
            binding.gemm_quant(p.in_dtype, *a[1:11], *a[12:15], p.c_dtype, p.c_scale, p.batch,
                               p.stride_a, p.stride_b, p.stride_c, bias=epi["bias"],
                               stride_bias=p.stride_bias or 0, act=p.act, stream=a[-1])
            turn[0] = (turn[0] + 1) % len(argsets)
        launch.turn = lambda: turn[0]
        return launch
    if p.entry == "bf16x3":
        def launch():
            a = argsets[turn[0]]
            binding.gemm_f32_bf16x3(*a[1:15], batch=p.batch, stride_a=p.stride_a,
                                    stride_b=p.stride_b, stride_c=p.stride_c,
                                    workspace=workspace.data_ptr(),
                                    workspace_bytes=workspace.numel() * 4, stream=a[-1])
            turn[0] = (turn[0] + 1) % len(argsets)
        launch.turn = lambda: turn[0]
        return launch

    def launch():
        binding.gemm(*argsets[turn[0]], **epi)
        turn[0] = (turn[0] + 1) % len(argsets)
    launch.turn = lambda: turn[0]
    return launch


def mx_args(p, bufs, stream=0):
    from dense_gemm_optimisation_amd import binding
    da, dsa, db, dsb, dc = bufs
    out = {"f32": binding.OUTPUT_F32, "bf16": binding.OUTPUT_BF16, "f16": binding.OUTPUT_F16}
    return (p.M, p.N, p.K, p.alpha, da.data_ptr(), p.lda, binding.MX_FORMAT[p.fa], dsa.data_ptr(),
            p.ldsa, db.data_ptr(), p.ldb, binding.MX_FORMAT[p.fb], dsb.data_ptr(), p.ldsb, p.beta,
            dc.data_ptr(), p.ldc, p.order_c, out[p.c_dtype], p.batch, p.stride_a, p.stride_b,
            p.stride_sa, p.stride_sb, p.stride_c)


def make_mx_launch(p, sets, stream, workspace=None):
    """make_launch for a block-scaled workload (gemm_mx, or gemm_mx_ws with
    a workspace tensor)."""
    from dense_gemm_optimisation_amd import binding
    argsets = [mx_args(p, bufs) for bufs in sets]
    turn = [0]

    def launch():
        if workspace is None:
            binding.gemm_mx(*argsets[turn[0]], stream=stream.cuda_stream)
        else:
            binding.gemm_mx_ws(*argsets[turn[0]], workspace.data_ptr(), workspace.numel() * 4,
                               stream=stream.cuda_stream)
        turn[0] = (turn[0] + 1) % len(argsets)
    launch.turn = lambda: turn[0]
    return launch


def kernel_family(p, bufs, workspace=None):
    """The kernel libgemm launches for workload p on these device buffers
    (asked of the library itself, so the answer follows its dispatch rules
    and the buffers' actual alignment)."""
    from dense_gemm_optimisation_amd import binding
    if is_mx(p):
        if workspace is None:
            return binding.mx_kernel_name(*mx_args(p, bufs))
        return binding.mx_kernel_name(*mx_args(p, bufs), workspace=workspace.data_ptr(),
                                      workspace_bytes=workspace.numel() * 4)
    if p.entry == "valu":
        return "sgemm_valu"
    da, db, dc = bufs
    if p.entry == "quant":
        return binding.kernel_name_quant(p.in_dtype, p.M, p.N, p.K, p.alpha, da.data_ptr(), p.lda,
                                         p.order_a, db.data_ptr(), p.ldb, p.order_b, dc.data_ptr(),
                                         p.ldc, p.order_c, p.c_dtype, p.batch, p.stride_a,
                                         p.stride_b, p.stride_c)
    if p.entry == "bf16x3":
        name = binding.kernel_name_bf16x3(p.M, p.N, p.K, p.alpha, da.data_ptr(), p.lda, p.order_a,
                                          db.data_ptr(), p.ldb, p.order_b, p.beta, dc.data_ptr(),
                                          p.ldc, p.order_c, p.batch, p.stride_a, p.stride_b,
                                          p.stride_c, workspace.data_ptr(), workspace.numel() * 4)
        return f"f32_bf16x3 ({name})"
    c_dt = binding.DTYPE_F32 if (p.c_dtype == "f32" and p.in_dtype != "f32") else binding.DTYPE_SAME
    return binding.kernel_name(p.in_dtype, p.M, p.N, p.K, p.alpha, da.data_ptr(), p.lda, p.order_a,
                               db.data_ptr(), p.ldb, p.order_b, p.beta, dc.data_ptr(), p.ldc,
                               p.order_c, c_dt, p.batch, p.stride_a, p.stride_b, p.stride_c,
                               b_dtype=p.b_dtype, out_dtype=p.c_dtype,
                               workspace=None if workspace is None else workspace.data_ptr(),
                               workspace_bytes=0 if workspace is None else workspace.numel() * 4)


def source_hash(family):
    """Hash of the source file that defines the kernel family and of every
    header of the package it includes, directly or not (the kernel's code
    lives in both)."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "dense_gemm_optimisation_amd", "csrc")
    h = hashlib.sha256()
    if family not in KERNEL_SOURCE:
        return None
    todo, seen = [KERNEL_SOURCE[family]], set()
    while todo:
        name = todo.pop(0)
        path = os.path.join(csrc, name)
        if name in seen or not os.path.exists(path):
            continue
        seen.add(name)
        with open(path, "rb") as f:
            data = f.read()
        h.update(name.encode() + b"\0" + data)
        todo += [m.decode() for m in re.findall(rb'#include "([^"]+)"', data)]
    return h.hexdigest()[:16]


def measured_traffic(family, workload):
    """HBM bytes per launch from profiles/hbm_traffic.txt, or None when the
    entry is missing or was measured on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = source_hash(family)
    if want is None:
        return None
    for ln in open(TRAFFIC_FILE):
        f = ln.split()
        # family  source-sha  workload  fetch_bytes  write_bytes  (scaled, per launch)
        if len(f) >= 5 and not ln.startswith("#") and f[0] == family and f[2] == workload:
            return int(float(f[3]) + float(f[4])) if f[1] == want else None
    return None


def copy_calibration(mib, torch):
    """A plain copy of `mib` MiB, five times: the counters' reference kernel."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4}))


def cpu_model():
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for ln in out.splitlines():
        if ln.startswith("Model name:"):
            return ln.split(":", 1)[1].strip()
    return None


def error_stats(p, got_bits, ref, den):
    """Error of GPU results (stored bit patterns) against oracle values, by
    the tolerances the parity tests apply: fp32 output |C - ref| / den; 16-bit
    output the distance in units in the last place from the oracle rounded
    to that type, where an element beyond 2 ulp is accepted only as a genuine
    cancellation (|ref| <= 2^-8 den and |C - ref| <= 2 ulp + 1e-3 den; for
    8-bit inputs, whose instruction truncates small products, only the
    second condition)."""
    import oracle
    import workloads
    if p.c_dtype in workloads.EIGHT_BIT:  # quantised output: steps of the 8-bit format
        q = oracle.round_bits(p.c_dtype, ref).astype(np.int64)
        g = got_bits.view(np.uint8).astype(np.int64)
        key = lambda b: np.where(b & 0x80, -(b & 0x7F), b & 0x7F)
        both_nan = np.isnan(oracle.decode(p.c_dtype, g.astype(np.uint8))) & np.isnan(ref)
        d = np.where(both_nan, 0, np.abs(key(g) - key(q)))
        return {"max_ulp": int(d.max()), "beyond_1ulp": int((d > 1).sum()),
                "elements": int(ref.size)}
    with np.errstate(divide="ignore", invalid="ignore"):
        if p.c_dtype == "f32":
            got = got_bits.view(np.float32).astype(np.float64)
            err = np.where(den > 0, np.abs(got - ref) / np.where(den > 0, den, 1.0),
                           np.where(got == ref, 0.0, np.inf))
            return {"max_norm_err": float(err.max()), "elements": int(ref.size)}
        q = oracle.round_bits(p.c_dtype, ref).astype(np.int64)
        g = got_bits.view(np.uint16).astype(np.int64)
        key = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
        d = np.abs(key(g) - key(q))
        gv = oracle.decode(p.c_dtype, g.astype(np.uint16))
        qv = oracle.decode(p.c_dtype, q.astype(np.uint16))
        ulp = np.abs(oracle.decode(p.c_dtype, (q + 1).astype(np.uint16)) - qv)
        near = np.abs(gv - ref) <= 2 * ulp + 1e-3 * den
        if not is_mx(p) and p.in_dtype not in ("e4m3", "e5m2"):
            near &= np.abs(ref) <= 2.0 ** -8 * den
        bad = d > 2
        norm = np.where(den > 0, np.abs(gv - ref) / np.where(den > 0, den, 1.0), 0.0)
    return {"max_ulp": int(d.max()), "beyond_2ulp": int(bad.sum()),
            "accepted_cancellations": int((bad & near).sum()),
            "violations": int((bad & ~near).sum()), "max_norm_err": float(norm.max()),
            "elements": int(ref.size)}


def cpu_baseline(problems, budget_s, gpu_results):
    """The CPU oracle, as it stands, on each workload (a bounded sample of its
    rows), timed on this host; its values also give the error statistics of
    the GPU result on the same rows (gpu_results[name] = C bits as stored)."""
    import oracle
    import workloads
    threads = oracle.max_threads()
    total_flop, total_t, parts, per, errs = 0.0, 0.0, [], {}, {}
    share = budget_s / max(1, len(problems))
    for p in problems:
        if is_mx(p):
            a, sa, b, sb, c = workloads.generate_mx(p)
        else:
            a, b, c = workloads.generate(p)
        # rows [0, r) of C for the first batch entry: a sub-problem with
        # M = r when A is row-major (rows contiguous), else listed elements
        r = p.M
        est = 2.0 * p.M * p.N * p.K / 50e9  # ~50-65 GFLOP/s with 16 threads
        if est > share:
            r = max(1, int(p.M * share / est))
        t0 = time.perf_counter()
        if is_mx(p):  # A rows are contiguous; C row-major in every MX workload
            ref, den = oracle.mx_gemm(p.fa, p.fb, p.c_dtype, r, p.N, p.K, p.alpha, a, p.lda, sa,
                                      p.ldsa, b, p.ldb, sb, p.ldsb, p.beta, c, p.ldc, p.order_c)
            ref, den = ref[0].ravel(), den[0].ravel()
        elif p.order_a == workloads.ROW and p.order_c == workloads.ROW:
            ref, den = oracle.gemm(p.in_dtype, p.c_dtype, r, p.N, p.K, p.alpha, a, p.lda,
                                   p.order_a, b, p.ldb, p.order_b, p.beta, c, p.ldc, p.order_c,
                                   stride_a=p.stride_a, stride_b=p.stride_b, stride_c=p.stride_c,
                                   bias=workloads.bias_vector(p), stride_bias=p.stride_bias,
                                   act=p.act, b_dtype=p.b_dtype)
            ref, den = ref[0].ravel(), den[0].ravel()
        else:
            idx = np.stack([np.zeros(r * p.N, np.int64), np.repeat(np.arange(r), p.N),
                            np.tile(np.arange(p.N), r)], 1)
            ref, den = oracle.gemm_at(p.in_dtype, p.c_dtype, p.M, p.N, p.K, p.alpha, a, p.lda,
                                      p.order_a, b, p.ldb, p.order_b, p.beta, c, p.ldc,
                                      p.order_c, idx, stride_a=p.stride_a, stride_b=p.stride_b,
                                      stride_c=p.stride_c, bias=workloads.bias_vector(p),
                                      stride_bias=p.stride_bias, act=p.act, b_dtype=p.b_dtype)
        dt = time.perf_counter() - t0
        if getattr(p, "entry", "") == "quant":  # stored: the epilogue's value times the scale
            ref, den = p.c_scale * ref, abs(p.c_scale) * den
        flop = 2.0 * r * p.N * p.K
        total_flop += flop
        total_t += dt
        per[p.name] = {"rows": r, "of_rows": p.M, "seconds": round(dt, 3),
                       "gflops": round(flop / dt / 1e9, 3)}
        parts.append(f"{p.name}: rows 0..{r - 1} of {p.M} (batch entry 0), {dt:.1f} s")
        got = gpu_results.get(p.name)
        if got is not None:
            if p.order_c == workloads.ROW:
                sel = (np.arange(r)[:, None] * p.ldc + np.arange(p.N)[None, :]).ravel()
            else:
                sel = (np.arange(p.N)[None, :] * p.ldc + np.arange(r)[:, None]).ravel()
            errs[p.name] = error_stats(p, got[sel], ref, den)
    # the 256^3 problem whole: median of 10 with every thread, and once on one
    small = workloads.config("f32_256")
    a, b, c = workloads.generate(small)
    args = (small.in_dtype, small.c_dtype, small.M, small.N, small.K, small.alpha, a, small.lda,
            small.order_a, b, small.ldb, small.order_b, small.beta, c, small.ldc, small.order_c)
    ts = []
    for _ in range(10):
        t0 = time.perf_counter()
        oracle.gemm(*args)
        ts.append(time.perf_counter() - t0)
    oracle.set_threads(1)
    t0 = time.perf_counter()
    oracle.gemm(*args)
    t1 = time.perf_counter() - t0
    oracle.set_threads(threads)
    out = {"value": total_flop / total_t / 1e12, "unit": "TFLOPS", "cores": threads,
           "kind": "oracle",
           "sample": "; ".join(parts) + " -- the oracle's full-matrix path (double "
                     "accumulation, increasing k per element), perf_counter around the call",
           "cpu_model": cpu_model(), "per_config": per,
           "f32_256": {"median_s": round(float(np.median(ts)), 5), "threads": threads,
                       "gflops": round(small.flops / float(np.median(ts)) / 1e9, 3),
                       "single_thread_s": round(t1, 5),
                       "single_thread_gflops": round(small.flops / t1 / 1e9, 3)}}
    if errs:
        out["gpu_error_on_sampled_rows"] = errs
    return out


def smi():
    """gfx clock (mean over the dies), memory clock, power and temperatures
    from amd-smi, or None when it is unavailable."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--temperature", "--power",
                            "--json"], capture_output=True, text=True, timeout=30)
        g = json.loads(r.stdout)["gpu_data"][0]
    except (OSError, subprocess.SubprocessError, ValueError, KeyError, IndexError):
        return None

    def val(x):
        return x.get("value") if isinstance(x, dict) else None
    clocks = g.get("clock", {})
    gfx = [val(v.get("clk")) for k, v in clocks.items() if k.startswith("gfx_")]
    gfx = [x for x in gfx if isinstance(x, (int, float))]
    temp = g.get("temperature", {})
    return {"gfx_mhz": round(sum(gfx) / len(gfx), 1) if gfx else None,
            "mem_mhz": val(clocks.get("mem_0", {}).get("clk")),
            "power_w": val(g.get("power", {}).get("socket_power")),
            "hotspot_c": val(temp.get("hotspot")), "mem_c": val(temp.get("mem"))}


def clocks_under_load(fn, torch, seconds=3.0):
    """amd-smi readings taken while `fn` runs back to back for `seconds`
    (amd-smi reports values that trail the hardware by up to a second, so two
    readings are taken after the load has run a while, and the one drawing
    more power is kept)."""
    import threading
    stop = threading.Event()

    def loop():
        while not stop.is_set():
            for _ in range(256):
                fn()
            torch.cuda.synchronize()
    th = threading.Thread(target=loop)
    th.start()
    time.sleep(seconds * 0.4)
    first = smi()
    time.sleep(seconds * 0.3)
    second = smi()
    stop.set()
    th.join()
    readings = [r for r in (first, second) if r]
    return max(readings, key=lambda r: r.get("power_w") or 0) if readings else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-rotate", action="store_true",
                    help="reuse one buffer set per kernel (inputs may stay in the MALL)")
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=24.0)
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--no-clocks", action="store_true")
    ap.add_argument("--launch-samples", type=int, default=50,
                    help="launches timed one by one for the median and minimum")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB")
    ap.add_argument("--workspace", action="store_true",
                    help="workloads without a fused epilogue through the workspace entry "
                         "points (stream-K)")
    ap.add_argument("--results", default=None, help="append the JSON line to this file")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the GEMM path has no multi-GPU "
              "sharding (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from dense_gemm_optimisation_amd import binding
    binding.library()  # fails loudly if libgemm.so is missing
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, torch)
        return
    names = HEADLINE if args.workload == "headline" else args.workload.split(",")
    problems = [workloads.config(n) for n in names]
    stream = torch.cuda.Stream()  # default priority
    ws = None
    if args.workspace:
        ws = torch.empty(binding.workspace_size() // 4, dtype=torch.int32, device="cuda")
    clocks = {"before": None if args.no_clocks else smi()}
    launches, nsets, families = [], {}, {}
    with torch.cuda.stream(stream):
        for p in problems:
            log(f"[bench] preparing {p.name}: {p.note}")
            bufs = device_buffers(p, torch)
            sets = buffer_sets(bufs, sets_needed(bufs, not args.no_rotate))
            nsets[p.name] = len(sets)
            takes_ws = is_mx(p) or (not p.bias and not p.act and not p.entry)
            pws = ws if (ws is not None and takes_ws) else None
            if getattr(p, "entry", "") == "bf16x3":  # its own workspace, for the split copies
                pws = torch.empty(binding.bf16x3_workspace_size(p.M, p.N, p.K, p.batch) // 4,
                                  dtype=torch.int32, device="cuda")
            families[p.name] = kernel_family(p, bufs, pws)
            bias = None if is_mx(p) else device_bias(p, torch)
            launches.append((p, sets, make_launch(p, sets, stream, bias, pws)))
    torch.cuda.synchronize()

    # warmup
    for _ in range(args.warmup):
        for _, _, fn in launches:
            fn()
    torch.cuda.synchronize()

    # Timed region: the step's kernels, each launched `steps` times back to
    # back between one pair of HIP events on the stream they run on (an event
    # pair around every launch would add its own gap to each launch's time).
    # A kernel's mean launch duration is its event interval / steps; the
    # step's wall time is the whole region / steps.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in launches]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k, (_, _, fn) in enumerate(launches):
        ev[k][0].record(stream)
        for _ in range(args.steps):
            fn()
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Launch by launch (outside the timed region): each launch between its
    # own event pair, for the median and the minimum.
    one_by_one = {}
    for p, _, fn in launches:
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.launch_samples)]
        for e0, e1 in pairs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        one_by_one[p.name] = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)

    if not args.no_clocks:
        clocks["under_load"] = {p.name: clocks_under_load(fn, torch) for p, _, fn in launches}
        clocks["after"] = smi()

    per_kernel = {}
    flops_step = 0
    for k, (p, _, _) in enumerate(launches):
        ms = ev[k][0].elapsed_time(ev[k][1]) / args.steps
        tfl = p.flops / (ms * 1e-3) / 1e12
        flops_step += p.flops
        alg_bytes = algorithmic_bytes(p)
        key = dtype_key(p)
        t1 = one_by_one[p.name]
        med, mn = t1[len(t1) // 2], t1[0]
        per_kernel[p.name] = {
            "kernel": families[p.name],
            "dtype": key, "M": p.M, "N": p.N, "K": p.K, "batch": p.batch,
            "mean_us": round(ms * 1e3, 2), "tflops": round(tfl, 2),
            "frac_of_peak": round(tfl / PEAK_TFLOPS[key], 4),
            "alg_gbs": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
            "alg_frac_of_hbm": round(alg_bytes / (ms * 1e-3) / 1e9 / HBM_GBS, 4),
            "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2),
            "tflops_median": round(p.flops / (med * 1e-3) / 1e12, 2),
            "frac_of_peak_median": round(p.flops / (med * 1e-3) / 1e12 / PEAK_TFLOPS[key], 4),
            "tflops_best": round(p.flops / (mn * 1e-3) / 1e12, 2)}
    ms_step = wall / args.steps * 1e3
    value = flops_step / (wall / args.steps) / 1e12

    def roof(name):
        k = per_kernel[name]
        p = workloads.config(name)
        fam = families[name]
        peak = PEAK_TFLOPS[dtype_key(p)]
        traffic = measured_traffic(fam, name)
        # below the ridge point (peak flop rate / HBM bandwidth) the problem
        # is bound by HBM: its algorithmic bytes against 8 TB/s; above it by
        # the matrix cores' rate for its dtype, or for the vector-ALU fp32
        # kernel by the vector units' FMA rate (MI355X publishes the same
        # 157.3 TF/s for both fp32 units)
        if p.flops / algorithmic_bytes(p) < peak * 1e12 / (HBM_GBS * 1e9):
            return {"kernel": f"{fam} {name}", "bound": "hbm", "achieved": k["alg_gbs"],
                    "peak": HBM_GBS, "unit": "GB/s", "frac": round(k["alg_gbs"] / HBM_GBS, 4),
                    "traffic": traffic}
        bound = "alu" if fam == "sgemm_valu" else "mfma"
        return {"kernel": f"{fam} {name}", "bound": bound, "achieved": k["tflops"],
                "peak": peak, "unit": "TFLOP/s", "frac": round(k["tflops"] / peak, 4),
                "traffic": traffic}

    dominant = max(per_kernel, key=lambda n: per_kernel[n]["mean_us"])
    out = {
        "metric": "TFLOPS (2MNK/t) at 4096^3 fp32 and bf16; % of MI355X dense peak per dtype",
        "value": round(value, 3), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "+".join(dtype_key(p) for p in problems),
        "data": "synthetic",
        "config": {"workload": " + ".join(f"{p.name} ({p.note})" for p in problems),
                   "global_batch": 1, "parallelism": "none (1 GPU)",
                   "buffer_sets": nsets},
        "per_kernel": per_kernel,
        "roofline": roof(dominant),
        "roofline_all": [roof(n) for n in per_kernel],
        "clocks": None if args.no_clocks else clocks,
    }
    if not args.no_context:
        out["context_torch_matmul"] = torch_context(problems, stream, torch)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(problems, args.cpu_budget,
                                           single_results(launches, torch))
    line = json.dumps(out)
    print(line, flush=True)
    if args.results:
        with open(args.results, "a") as f:
            f.write(line + "\n")


def single_results(launches, torch):
    """C of one clean launch per workload (C0 restored first), as stored bits,
    for the error statistics of the CPU-baseline leg."""
    import workloads
    res = {}
    for p, sets, fn in launches:
        c0 = workloads.generate_mx(p)[4] if is_mx(p) else workloads.generate(p)[2]
        dc = sets[0][-1]
        dc.copy_(torch.from_numpy(c0.view(VIEW[p.c_dtype])).to(dc.device))
        torch.cuda.synchronize()
        # the launcher cycles through the buffer sets: run until set 0 comes round
        for _ in range(len(sets)):
            turn = fn.turn()
            fn()
            if turn == 0:
                break
        torch.cuda.synchronize()
        res[p.name] = dc.cpu().numpy().view(workloads.storage(p.c_dtype))
    return res


def torch_context(problems, stream, torch):
    """torch.matmul (the vendor BLAS) on the same shapes: context only, not the path."""
    res = {}
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
          "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
    with torch.cuda.stream(stream):
        for p in problems:
            if p.batch != 1 or is_mx(p):
                continue
            a = torch.randn(p.M, p.K, device="cuda").to(dt[p.in_dtype])
            b = torch.randn(p.K, p.N, device="cuda").to(dt[p.b_dtype])
            if p.in_dtype in ("e4m3", "e5m2"):
                # torch's scaled 8-bit product (row-major A, column-major B)
                one = torch.ones((), device="cuda")
                bt = b.t().contiguous().t()
                out_dt = dt[p.c_dtype]

                def fn():
                    torch._scaled_mm(a, bt, scale_a=one, scale_b=one, out_dtype=out_dt)
            else:
                def fn():
                    torch.matmul(a, b)
            try:
                for _ in range(3):
                    fn()
            except RuntimeError as e:  # not every torch build has the 8-bit product
                res[p.name] = f"unavailable: {str(e).splitlines()[0][:80]}"
                continue
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            res[p.name] = round(p.flops / (ms * 1e-3) / 1e12, 2)
    return {"unit": "TFLOPS", "note": "torch.matmul on identical shapes; context only", **res}


if __name__ == "__main__":
    main()
