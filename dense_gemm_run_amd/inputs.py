"""Seeded synthetic operands for the dense matrix product.

This module draws random inputs and nothing else: it holds none of the
product's arithmetic, and it is the only code shared by the GPU path's tests
and benchmark and the CPU oracle's callers.

Recipe (every workload): a CPU ``torch.Generator`` seeded with the workload's
seed draws A first, then B, in fp32; each is then cast to the workload's dtype
with torch's round-to-nearest-even (for the 8-bit dtypes, torch's conversion
to ``float8_e4m3fn`` / ``float8_e5m2``, the OCP formats; the distributions
used with them stay far inside both formats' ranges).  The seeding convention (a fixed seed
before drawing both operands) follows the correctness cell of the notebook
"Triton tiled matmul".  Distributions:

``uniform``        U[-1, 1): ``rand * 2 - 1`` for A and B.
``normal``         N(0, 1): ``randn`` for A and B.
``normal_sqrtk``   N(0, 1)/sqrt(K) for both A and B.
``prefill``        activations A ~ N(0, 1), weights B [K, N] ~ N(0, 0.02)
                   (``0.02 * randn``), as a transformer projection with
                   tokens along M.
``decode``         weights A [M, K] ~ N(0, 0.02) and activations B [K, N] ~
                   N(0, 1): the matrix-vector product y = W·x of one decode
                   step (few columns N).
``integers``       integers drawn uniformly from [-4, 4] for A and B (every
                   product and partial sum is then an exact small integer).
``fp32_fine``      values 1 + j·2^-23 with j uniform in [0, 2^23): fp32 numbers
                   in [1, 2) whose low significand bits are all in use, so any
                   shortening of fp32 inputs (a 10- or 7-bit significand)
                   moves the product by far more than 1e-5 relative.

Batched workloads draw the same way with one generator: all of A's matrices
([batch, M, K], in order), then all of B's ([batch, K, N], or one [K, N] when
B is shared by every product).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
          "fp8_e4m3": torch.float8_e4m3fn, "fp8_e5m2": torch.float8_e5m2}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str
    dist: str
    seed: int
    about: str
    batch: int = 1

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch


# The workloads the product is checked and measured on, with their seeds.
WORKLOADS: dict[str, Workload] = {w.name: w for w in [
    Workload("f32_64x64x64", 64, 64, 64, "f32", "uniform", 0,
             "fp32 64^3, U[-1,1)"),
    Workload("f16_127x255x65", 127, 255, 65, "f16", "normal", 1,
             "ragged fp16 127x255x65, N(0,1): every edge masked"),
    Workload("f16_4096x4096x4096", 4096, 4096, 4096, "f16", "normal_sqrtk", 2,
             "square fp16 4096^3, N(0,1)/sqrt(K)"),
    Workload("bf16_8192x8192x8192", 8192, 8192, 8192, "bf16", "uniform", 3,
             "square bf16 8192^3, U[-1,1)"),
    Workload("bf16_prefill_qkv_8192x12288x4096", 8192, 12288, 4096, "bf16", "prefill", 4,
             "prefill QKV projection, 8192 tokens"),
    Workload("bf16_prefill_out_8192x4096x4096", 8192, 4096, 4096, "bf16", "prefill", 5,
             "prefill output projection, 8192 tokens"),
    Workload("bf16_prefill_up_8192x14336x4096", 8192, 14336, 4096, "bf16", "prefill", 6,
             "prefill MLP up projection, 8192 tokens"),
    Workload("bf16_prefill_down_8192x4096x14336", 8192, 4096, 14336, "bf16", "prefill", 7,
             "prefill MLP down projection, 8192 tokens"),
    Workload("bf16_batched_16x2048x2048x2048", 2048, 2048, 2048, "bf16", "uniform", 8,
             "16 independent bf16 2048^3 products in one launch", batch=16),
    Workload("bf16_batched_64x2048x2048x128", 2048, 2048, 128, "bf16", "normal_sqrtk", 9,
             "attention-score shaped batch: 64 heads of [2048 x 128] @ [128 x 2048]", batch=64),
    Workload("bf16_gemv_14336x1x4096", 14336, 1, 4096, "bf16", "decode", 10,
             "decode GEMV y = W x, W [14336, 4096] (MLP up, one token)"),
    Workload("bf16_gemv_4096x1x14336", 4096, 1, 14336, "bf16", "decode", 11,
             "decode GEMV y = W x, W [4096, 14336] (MLP down, one token)"),
    Workload("bf16_gemv_12288x4x4096", 12288, 4, 4096, "bf16", "decode", 12,
             "decode GEMV with 4 vectors, W [12288, 4096] (QKV, 4 tokens)"),
    Workload("fp8_e4m3_4096x4096x4096", 4096, 4096, 4096, "fp8_e4m3", "normal", 13,
             "square 4096^3 with E4M3 inputs, N(0,1) rounded to E4M3, bf16 output"),
    Workload("fp8_e5m2_4096x4096x4096", 4096, 4096, 4096, "fp8_e5m2", "normal", 14,
             "square 4096^3 with E5M2 inputs, N(0,1) rounded to E5M2, bf16 output"),
    Workload("fp8_e4m3_8192x8192x8192", 8192, 8192, 8192, "fp8_e4m3", "normal", 15,
             "square 8192^3 with E4M3 inputs, N(0,1) rounded to E4M3, bf16 output"),
    Workload("bf16_tokens16_16x4096x4096", 16, 4096, 4096, "bf16", "prefill", 16,
             "16 tokens through a 4096 x 4096 projection (weights B [K, N])"),
    Workload("bf16_tokens128_128x4096x4096", 128, 4096, 4096, "bf16", "prefill", 17,
             "128 tokens through a 4096 x 4096 projection (weights B [K, N])"),
    Workload("bf16_3072x3072x3072", 3072, 3072, 3072, "bf16", "normal_sqrtk", 18,
             "square bf16 3072^3, N(0,1)/sqrt(K): 144 tiles of 256 x 256, a partial wave of the 256 CUs"),
    Workload("f32_4096x4096x4096", 4096, 4096, 4096, "f32", "uniform", 19,
             "square fp32 4096^3, U[-1,1): the fp32 path at a size where it is compute-bound"),
]}

# Order in which the four prefill projections of one layer run.
PREFILL_SWEEP = [
    "bf16_prefill_qkv_8192x12288x4096",
    "bf16_prefill_out_8192x4096x4096",
    "bf16_prefill_up_8192x14336x4096",
    "bf16_prefill_down_8192x4096x14336",
]


def _draw(shape, dist: str, K: int, gen: torch.Generator, role: str) -> torch.Tensor:
    if dist == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2 - 1
    if dist == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32)
    if dist == "normal_sqrtk":
        return torch.randn(shape, generator=gen, dtype=torch.float32) / math.sqrt(max(K, 1))
    if dist == "prefill":
        z = torch.randn(shape, generator=gen, dtype=torch.float32)
        return z if role == "A" else 0.02 * z
    if dist == "decode":
        z = torch.randn(shape, generator=gen, dtype=torch.float32)
        return 0.02 * z if role == "A" else z
    if dist == "integers":
        return torch.randint(-4, 5, shape, generator=gen).to(torch.float32)
    if dist == "fp32_fine":
        j = torch.randint(0, 1 << 23, shape, generator=gen, dtype=torch.int64)
        return (1.0 + j.to(torch.float64) * 2.0 ** -23).to(torch.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_operands(M: int, N: int, K: int, dtype: str, dist: str, seed: int):
    """(A [M,K], B [K,N]) as contiguous CPU tensors of ``dtype``."""
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {sorted(DTYPES)}")
    gen = torch.Generator().manual_seed(seed)
    A = _draw((M, K), dist, K, gen, "A").to(DTYPES[dtype]).contiguous()
    B = _draw((K, N), dist, K, gen, "B").to(DTYPES[dtype]).contiguous()
    return A, B


def make_batched_operands(batch: int, M: int, N: int, K: int, dtype: str, dist: str,
                          seed: int, share_b: bool = False):
    """(A [batch,M,K], B [batch,K,N] or [K,N] when ``share_b``) as contiguous
    CPU tensors of ``dtype``."""
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {sorted(DTYPES)}")
    gen = torch.Generator().manual_seed(seed)
    A = _draw((batch, M, K), dist, K, gen, "A").to(DTYPES[dtype]).contiguous()
    B = _draw((K, N) if share_b else (batch, K, N), dist, K, gen, "B").to(DTYPES[dtype]).contiguous()
    return A, B


def workload_operands(name: str):
    w = WORKLOADS[name]
    if w.batch > 1:
        return make_batched_operands(w.batch, w.M, w.N, w.K, w.dtype, w.dist, w.seed)
    return make_operands(w.M, w.N, w.K, w.dtype, w.dist, w.seed)
