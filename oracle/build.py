"""Compile the C oracle into ``oracle/liboracle_gemm.so`` (gcc, OpenMP).

Test infrastructure only: see the package docstring.  The flags keep the
arithmetic plain: no fast-math, no fused multiply-add contraction, no
auto-vectorised reassociation (fp64 sums stay in k order).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_gemm.c")
LIB = os.path.join(HERE, "liboracle_gemm.so")

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fno-tree-vectorize",
          "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile unconditionally and return the library path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Build only if the library is missing or older than its source."""
    if (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
