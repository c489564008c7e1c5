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
                       [--no-cpu-baseline] [--no-context] [--no-rotate]
                       [--copy-calibration MiB] [--workspace]
Each kernel cycles through at least three copies of its buffers, enough that
their footprint exceeds twice the 256 MB MALL, so inputs come from HBM;
--no-rotate reuses one set (the warm-cache figure).
--workload runs the named workload, or a comma-separated list of them (see
workloads.CONFIGS), instead of the headline step, for profiling.  --workspace runs fp32/bf16/fp16 workloads
through the workspace entry points, which use the stream-K schedule where
it applies.  --copy-calibration runs only a plain
device-to-device copy of the given size (the reference kernel against which
the HBM byte counters FETCH_SIZE / WRITE_SIZE are scaled).

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

# MI355X dense peaks, published (8-bit floats: twice the 16-bit rate)
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2}
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
                 "scale": "scale.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_buffers(p, torch):
    import workloads
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
    c_dt = binding.DTYPE_F32 if (p.c_dtype == "f32" and p.in_dtype != "f32") else binding.DTYPE_SAME
    argsets = [(p.in_dtype, p.M, p.N, p.K, p.alpha, da.data_ptr(), p.lda, p.order_a, db.data_ptr(),
                p.ldb, p.order_b, p.beta, dc.data_ptr(), p.ldc, p.order_c, c_dt, p.batch,
                p.stride_a, p.stride_b, p.stride_c, stream.cuda_stream) for da, db, dc in sets]
    epi = dict(bias=None if bias is None else bias.data_ptr(), stride_bias=p.stride_bias,
               act=p.act, b_dtype=p.b_dtype, out_dtype=p.c_dtype)
    if workspace is not None:
        epi.update(workspace=workspace.data_ptr(), workspace_bytes=workspace.numel() * 4)
    turn = [0]

    def launch():
        binding.gemm(*argsets[turn[0]], **epi)
        turn[0] = (turn[0] + 1) % len(argsets)
    return launch


def kernel_family(p, bufs, workspace=None):
    """The kernel libgemm launches for workload p on these device buffers
    (asked of the library itself, so the answer follows its dispatch rules
    and the buffers' actual alignment)."""
    from dense_gemm_optimisation_amd import binding
    da, db, dc = bufs
    c_dt = binding.DTYPE_F32 if (p.c_dtype == "f32" and p.in_dtype != "f32") else binding.DTYPE_SAME
    return binding.kernel_name(p.in_dtype, p.M, p.N, p.K, p.alpha, da.data_ptr(), p.lda, p.order_a,
                               db.data_ptr(), p.ldb, p.order_b, p.beta, dc.data_ptr(), p.ldc,
                               p.order_c, c_dt, p.batch, p.stride_a, p.stride_b, p.stride_c,
                               b_dtype=p.b_dtype, out_dtype=p.c_dtype,
                               workspace=None if workspace is None else workspace.data_ptr(),
                               workspace_bytes=0 if workspace is None else workspace.numel() * 4)


def source_hash(family):
    import hashlib
    path = os.path.join(ROOT, "dense_gemm_optimisation_amd", "csrc", KERNEL_SOURCE[family])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(family, workload):
    """HBM bytes per launch from profiles/hbm_traffic.txt, or None when the
    entry is missing or was measured on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = source_hash(family)
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


def cpu_baseline(problems, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    import workloads
    total_flop, total_t, parts = 0.0, 0.0, []
    per = budget_s / len(problems)
    for p in problems:
        a, b, c = workloads.generate(p)
        rows = 1
        while True:  # calibrate on one row, then size the sample to the budget
            idx = np.stack([np.zeros(rows * p.N, np.int64), np.repeat(np.arange(rows), p.N),
                            np.tile(np.arange(p.N), rows)], 1)
            t0 = time.perf_counter()
            oracle.gemm_at(p.in_dtype, p.c_dtype, p.M, p.N, p.K, p.alpha, a, p.lda, p.order_a, b,
                           p.ldb, p.order_b, p.beta, c, p.ldc, p.order_c, idx, b_dtype=p.b_dtype)
            dt = time.perf_counter() - t0
            if dt >= 0.5 * per or rows >= p.M:
                break
            rows = min(p.M, max(rows * 2, int(rows * per / max(dt, 1e-3))))
        flop = 2.0 * rows * p.N * p.K
        total_flop += flop
        total_t += dt
        parts.append(f"{p.name}: first {rows} rows x {p.N} cols ({dt:.1f} s)")
    return {"value": total_flop / total_t / 1e12, "unit": "TFLOPS", "cores": oracle.max_threads(),
            "kind": "oracle", "sample": "; ".join(parts) +
            " -- double-accumulating triple loop, timed with perf_counter"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-rotate", action="store_true",
                    help="reuse one buffer set per kernel (inputs may stay in the MALL)")
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB")
    ap.add_argument("--workspace", action="store_true",
                    help="fp32/bf16/fp16 workloads through the workspace entry points (stream-K)")
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
    launches, nsets, families = [], {}, {}
    with torch.cuda.stream(stream):
        for p in problems:
            log(f"[bench] preparing {p.name}: {p.note}")
            bufs = device_buffers(p, torch)
            sets = buffer_sets(bufs, sets_needed(bufs, not args.no_rotate))
            nsets[p.name] = len(sets)
            pws = ws if (ws is not None and p.in_dtype in ("f32", "bf16", "f16") and not p.bias
                         and not p.act) else None
            families[p.name] = kernel_family(p, bufs, pws)
            bias = device_bias(p, torch)
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

    per_kernel = {}
    flops_step = 0
    for k, (p, _, _) in enumerate(launches):
        ms = ev[k][0].elapsed_time(ev[k][1]) / args.steps
        tfl = p.flops / (ms * 1e-3) / 1e12
        flops_step += p.flops
        alg_bytes = (p.M * p.K * ESIZE[p.in_dtype] + p.K * p.N * ESIZE[p.b_dtype]) * p.batch + \
            p.M * p.N * ESIZE[p.c_dtype] * p.batch * (2 if p.beta else 1)
        per_kernel[p.name] = {
            "dtype": p.in_dtype, "M": p.M, "N": p.N, "K": p.K, "batch": p.batch,
            "mean_us": round(ms * 1e3, 2), "tflops": round(tfl, 2),
            "frac_of_peak": round(tfl / PEAK_TFLOPS[p.in_dtype], 4),
            "alg_gbs": round(alg_bytes / (ms * 1e-3) / 1e9, 1)}
    ms_step = wall / args.steps * 1e3
    value = flops_step / (wall / args.steps) / 1e12

    def roof(name):
        k = per_kernel[name]
        p = workloads.config(name)
        fam = families[name]
        # the vector-ALU fp32 kernel is bound by the FMA rate of the vector
        # units; every other kernel by the matrix cores' rate for its dtype
        # (MI355X publishes the same 157.3 TF/s for both fp32 units)
        bound = "alu" if fam == "sgemm_valu" else "mfma"
        peak = PEAK_TFLOPS[p.in_dtype]
        return {"kernel": f"{fam} {name}", "bound": bound, "achieved": k["tflops"],
                "peak": peak, "unit": "TFLOP/s", "frac": round(k["tflops"] / peak, 4),
                "traffic": measured_traffic(fam, name)}

    dominant = max(per_kernel, key=lambda n: per_kernel[n]["mean_us"])
    out = {
        "metric": "TFLOPS (2MNK/t) at 4096^3 fp32 and bf16; % of MI355X dense peak per dtype",
        "value": round(value, 3), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "+".join(p.in_dtype for p in problems),
        "data": "synthetic",
        "config": {"workload": " + ".join(f"{p.name} ({p.note})" for p in problems),
                   "global_batch": 1, "parallelism": "none (1 GPU)",
                   "buffer_sets": nsets},
        "per_kernel": per_kernel,
        "roofline": roof(dominant),
        "roofline_all": [roof(n) for n in per_kernel],
    }
    if not args.no_context:
        out["context_torch_matmul"] = torch_context(problems, stream, torch)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(problems[:2], args.cpu_budget)
    print(json.dumps(out), flush=True)


def torch_context(problems, stream, torch):
    """torch.matmul (the vendor BLAS) on the same shapes: context only, not the path."""
    res = {}
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
          "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
    with torch.cuda.stream(stream):
        for p in problems:
            if p.batch != 1:
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
