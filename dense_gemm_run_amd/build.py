"""Compile the HIP sources into ``dense_gemm_run_amd/libdense_gemm_run_amd.so``.

gfx950 only.  Every translation unit goes through hipcc with packed-fp32
instruction selection switched off; the host pass prints a harmless warning
that it does not know that (device-only) feature.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdense_gemm_run_amd.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["gemm_api.cpp", "gemm_generic.hip", "gemm_mfma32x32.hip", "gemm_mfma16x16.hip", "gemm_gemv.hip",
           "gemm_fp8.hip", "gemm_skinny.hip", "gemm_splitk.hip", "gemm_fp32.hip",
           "gemm_shortk.hip", "gemm_fewrow.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# The pipelined kernels unroll whole K-steps (hundreds of MFMAs with their
# loads and LDS operations); the pragma-unroll size limit is raised so that
# every such loop unrolls and the per-slot register arrays never fall back to
# scratch memory (tests/test_codegen_cpu.py checks for scratch use).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-pragma-unroll-threshold=1000000",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    # a library with unresolved symbols (e.g. a kernel whose host stub was not
    # emitted) must fail here, not at first use
    import ctypes
    ctypes.CDLL(tmp)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
