"""ctypes binding of the plain C oracle (``oracle_gemm.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Functions and what pins them (tests/test_oracle_pins.py):

``gemm_f64``         the three-loop fp64 product, written from the definition
                     C[row,col] = sum_inner A[row,inner]*B[inner,col] (lesson
                     "Matrix multiplication: reuse the inputs", section "The
                     three dimensions have different jobs").  Pinned by the
                     worked 2x3·3x2 example printed there, by exact rational
                     brute force on every shape up to 6x6x6, by integer closed
                     forms (identity, all-ones) and by numpy's float64 matmul
                     within its rounding bound.
``gemm_points_f64``  the same sum for chosen (row, col) pairs, for sampling a
                     product too large to form whole.  Pinned against
                     ``gemm_f64`` entries and against exact integer sums.
``gemm_batched_f64`` C[i] = A[i]·B[i] for every i of an outer batch
                     dimension (notebook "Triton tiled matmul", the
                     exercises: the same product with a third program axis
                     over the batch), one ``gemm_f64`` per matrix; a 2-D
                     operand is the same matrix for every i.  Pinned against
                     numpy's batched matmul on integer inputs (exact), with
                     each operand shared in turn and with an empty batch.
``round_to_bits``    fp64 -> fp16 / bf16 / fp32 round-to-nearest-even (the
                     reading of the final cast in "Connect to the real
                     implementation" and the Triton kernel of chapter "Fast
                     matrix multiplication").  Pinned against numpy's and
                     CPython's binary16 conversion, torch's fp32 -> bf16
                     conversion on fp32-exact values, an exact rational RNE,
                     and hand-checked ties, overflow and subnormal values.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_DBL_P = ctypes.POINTER(ctypes.c_double)
_I64_P = ctypes.POINTER(ctypes.c_int64)


def default_threads() -> int:
    """Threads the oracle uses: OMP_NUM_THREADS if set, else the CPUs this
    process may run on."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        L = ctypes.CDLL(path)
        L.oracle_gemm_f64.argtypes = [_DBL_P, _DBL_P, _DBL_P, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
        L.oracle_gemm_f64.restype = None
        L.oracle_gemm_rows_f64.argtypes = [_DBL_P, _DBL_P, _DBL_P, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int]
        L.oracle_gemm_rows_f64.restype = None
        L.oracle_time_gemm_rows_f64.argtypes = L.oracle_gemm_rows_f64.argtypes
        L.oracle_time_gemm_rows_f64.restype = ctypes.c_double
        L.oracle_gemm_points_f64.argtypes = [_DBL_P, _DBL_P, _I64_P, _I64_P,
                                             ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, _DBL_P, ctypes.c_int]
        L.oracle_gemm_points_f64.restype = None
        for name, ct in (("oracle_round_f16", ctypes.c_uint16),
                         ("oracle_round_bf16", ctypes.c_uint16),
                         ("oracle_round_f32", ctypes.c_uint32)):
            f = getattr(L, name)
            f.argtypes = [_DBL_P, ctypes.POINTER(ct), ctypes.c_int64]
            f.restype = None
        _lib = L
    return _lib


def _f64(x) -> np.ndarray:
    """Exact widening to a C-contiguous float64 array (fp16/bf16/fp32 -> fp64
    is exact).  Accepts numpy arrays or CPU torch tensors."""
    if not isinstance(x, np.ndarray):  # torch tensor
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray, t=_DBL_P):
    return a.ctypes.data_as(t)


def gemm_f64(A, B, nthreads: int | None = None) -> np.ndarray:
    """Full fp64 product of A [M,K] and B [K,N]."""
    A = _f64(A)
    B = _f64(B)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("oracle expects [M, K] @ [K, N]")
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), dtype=np.float64)
    if M and N:
        lib().oracle_gemm_f64(_ptr(A), _ptr(B), _ptr(C), M, N, K,
                              nthreads or default_threads())
    return C


def gemm_rows_f64(A, B, row0: int, nrows: int, nthreads: int | None = None):
    """Rows [row0, row0+nrows) of the fp64 product."""
    A = _f64(A)
    B = _f64(B)
    M, K = A.shape
    N = B.shape[1]
    if not (0 <= row0 and row0 + nrows <= M):
        raise ValueError("row block out of range")
    C = np.empty((nrows, N), dtype=np.float64)
    if nrows and N:
        lib().oracle_gemm_rows_f64(_ptr(A), _ptr(B), _ptr(C), row0, nrows, N, K,
                                   nthreads or default_threads())
    return C


def time_rows_f64(A64: np.ndarray, B64: np.ndarray, row0: int, nrows: int,
                  nthreads: int) -> tuple[float, np.ndarray]:
    """Seconds spent computing rows [row0, row0+nrows), and those rows."""
    M, K = A64.shape
    N = B64.shape[1]
    C = np.empty((nrows, N), dtype=np.float64)
    t = lib().oracle_time_gemm_rows_f64(_ptr(A64), _ptr(B64), _ptr(C), row0, nrows,
                                        N, K, nthreads)
    return t, C


def gemm_points_f64(A, B, rows, cols, nthreads: int | None = None) -> np.ndarray:
    """C[rows[t], cols[t]] for each t, each one fp64 dot product."""
    A = _f64(A)
    B = _f64(B)
    M, K = A.shape
    N = B.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and the same length")
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise ValueError("point out of range")
    out = np.empty(rows.size, dtype=np.float64)
    if rows.size:
        lib().oracle_gemm_points_f64(_ptr(A), _ptr(B), _ptr(rows, _I64_P),
                                     _ptr(cols, _I64_P), rows.size, N, K,
                                     _ptr(out), nthreads or default_threads())
    return out


def gemm_batched_f64(A, B, nthreads: int | None = None) -> np.ndarray:
    """C[i] = A[i] @ B[i] for i in range(batch): A is [batch, M, K] or [M, K]
    (shared by every i), B is [batch, K, N] or [K, N]."""
    A = _f64(A)
    B = _f64(B)
    if A.ndim not in (2, 3) or B.ndim not in (2, 3) or (A.ndim == 2 and B.ndim == 2):
        raise ValueError("batched oracle expects [batch, M, K] @ [batch, K, N]")
    if A.shape[-1] != B.shape[-2]:
        raise ValueError("batched oracle expects [..., M, K] @ [..., K, N]")
    batch = A.shape[0] if A.ndim == 3 else B.shape[0]
    if (A.ndim == 3 and A.shape[0] != batch) or (B.ndim == 3 and B.shape[0] != batch):
        raise ValueError("batch sizes differ")
    M, N = A.shape[-2], B.shape[-1]
    C = np.empty((batch, M, N), dtype=np.float64)
    for i in range(batch):
        C[i] = gemm_f64(A[i] if A.ndim == 3 else A, B[i] if B.ndim == 3 else B, nthreads)
    return C


_ROUNDERS = {
    "f16": ("oracle_round_f16", np.uint16, ctypes.c_uint16),
    "bf16": ("oracle_round_bf16", np.uint16, ctypes.c_uint16),
    "f32": ("oracle_round_f32", np.uint32, ctypes.c_uint32),
}


def round_to_bits(x, dtype: str) -> np.ndarray:
    """Round fp64 values to ``dtype`` ("f16", "bf16", "f32") with
    round-to-nearest-even; returns the bit patterns."""
    name, npt, ct = _ROUNDERS[dtype]
    x = _f64(x)
    flat = np.ascontiguousarray(x.reshape(-1))
    out = np.empty(flat.size, dtype=npt)
    if flat.size:
        getattr(lib(), name)(_ptr(flat), out.ctypes.data_as(ctypes.POINTER(ct)), flat.size)
    return out.reshape(x.shape)


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode bit patterns of ``dtype`` to the exact fp64 values."""
    bits = np.asarray(bits)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def reference(A, B, dtype: str, nthreads: int | None = None):
    """The oracle's answer for inputs already held in ``dtype``: the fp64
    product rounded once to ``dtype``.  Returns (rounded values as fp64, the
    unrounded fp64 product)."""
    C64 = gemm_f64(A, B, nthreads)
    return bits_to_f64(round_to_bits(C64, dtype), dtype), C64


def reference_batched(A, B, dtype: str, nthreads: int | None = None):
    """As ``reference``, for the batched product."""
    C64 = gemm_batched_f64(A, B, nthreads)
    return bits_to_f64(round_to_bits(C64, dtype), dtype), C64
