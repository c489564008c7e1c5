"""Build libgemm.so for gfx950 with hipcc.

Each source compiles to an object in ``_build/`` (in parallel), then one
shared library is linked into this package directory, where the Python
binding loads it.  The compiler's per-kernel resource report (VGPRs, AGPRs,
LDS, scratch) is saved to ``_build/resource_usage.txt``; a kernel that spills
to scratch memory is reported, since a spill in the inner loop costs far more
than it saves.

Packed fp32 instructions are switched off (``-packed-fp32-ops``): the fp32
kernel's fused multiply-adds are issued one lane-value per instruction.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "scale.hip", "pack.hip", "noalloc.hip", "sgemm_valu.hip", "sgemm_mfma.hip", "sgemm_splitk.hip", "hgemm_mfma.hip", "hgemm_mfma_dma.hip",
           "hgemm_splitk.hip", "gemm_skinny.hip", "f8gemm_mfma.hip", "mxgemm.hip", "split_bf16.hip"]
# Sources compiled once per part (-D<macro>=k, one object each), so that
# their many kernel instantiations build in parallel: source -> (macro, parts).
PARTS = {"hgemm_mfma.hip": ("LIBGEMM_HGEMM_PART", 4), "mxgemm.hip": ("LIBGEMM_MX_PART", 3)}


def units():
    """(source, part or None) for every object of the library."""
    out = []
    for s in SOURCES:
        n = PARTS.get(s)
        out += [(s, None)] if n is None else [(s, k) for k in range(n[1])]
    return out


def object_path(src: str, part=None) -> str:
    suffix = "" if part is None else f".p{part}"
    return os.path.join(BUILD_DIR, os.path.basename(src) + suffix + ".o")

FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool, part=None):
    obj = object_path(src, part)
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if part is not None:
        cmd.insert(1, f"-D{PARTS[src][0]}={part}")
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj, r.stderr


def _resource_report(logs):
    lines, spills = [], []
    kernel = None
    for log in logs:
        for ln in log.splitlines():
            m = re.search(r"Function Name: (\S+)", ln)
            if m:
                kernel = m.group(1)
            m = re.search(r"remark: .*?(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy "
                          r"\[waves/SIMD\]|LDS Size \[bytes/block\]|SGPRs): (\d+)", ln)
            if m and kernel:
                lines.append(f"{kernel}\t{m.group(1)}\t{m.group(2)}")
                if m.group(1).startswith("ScratchSize") and int(m.group(2)) > 0:
                    spills.append((kernel, int(m.group(2))))
    return lines, spills


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        # longest compilations first, so they do not start last
        todo = sorted(units(), key=lambda u: u[0] not in PARTS)
        results = list(ex.map(lambda u: _compile(u[0], verbose, u[1]), todo))
    objs = [o for o, _ in results]
    lines, spills = _resource_report([log for _, log in results])
    with open(os.path.join(BUILD_DIR, "resource_usage.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    for k, n in spills:
        print(f"warning: kernel {k} uses {n} bytes/lane of scratch (register spill)",
              file=sys.stderr)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
