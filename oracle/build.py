"""Build the CPU oracle library (test infrastructure).

Compiles ``gemm_oracle.c`` with gcc and OpenMP into ``liboracle.so`` next to
this file.  ``-ffp-contract=off`` keeps every multiply and add a separately
rounded double operation, as the oracle's definition requires.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
