"""8-bit floating-point inputs for the oracle: decoding and the product.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages ask for an FP8 input path whose accumulator stays FP32, compared
against FP16 (notebook "Triton tiled matmul", the exercises).  They do not
define the 8-bit formats; the two in use on current GPUs are the OCP 8-bit
floating-point formats (the Open Compute Project "OCP 8-bit Floating Point
Specification (OFP8)"), and this module decodes them from that definition:

``E4M3``  1 sign bit, 4 exponent bits (bias 7), 3 significand bits.  Exponent
          field 0 is subnormal: (-1)^s * m/8 * 2^-6.  Otherwise
          (-1)^s * (1 + m/8) * 2^(e-7), except S.1111.111, which is NaN; the
          format has no infinities, so 448 (0.1111.110) is the largest value.
``E5M2``  1 sign bit, 5 exponent bits (bias 15), 2 significand bits, laid out
          like IEEE binary16 with its low 8 bits cut off: exponent 0 is
          subnormal ((-1)^s * m/4 * 2^-14), exponent 31 is infinity (m = 0) or
          NaN, the largest finite value is 57344.

Functions and what pins them (tests/test_oracle_pins.py):

``decode``          bit patterns -> exact fp64 values.  Pinned by hand-checked
                    codes from the definitions above (largest, smallest
                    subnormal, smallest normal, one, NaN and infinities), by
                    torch's own float8_e4m3fn / float8_e5m2 conversion on all
                    256 codes, by E5M2 being binary16 with 8 low zero bits
                    (numpy's binary16 decode), and by the ordering invariant
                    (codes 0 .. largest finite decode strictly increasing; the
                    sign bit mirrors them).
``decoded_max_abs``  the largest finite magnitude among decoded codes (it
                    sets the absolute floor of the 8-bit comparisons).
                    Pinned by hand-checked sets of codes: every code gives the
                    format's largest finite value (448 / 57344), a negative
                    code of larger magnitude beats a positive one whose raw
                    code is smaller, NaN and infinity codes are ignored, an
                    empty set gives 0 (``test_fp8_decoded_max_abs``, with
                    planted mistakes in ``test_oracle_mutants.py``).
``reference_fp8``   the product of decoded inputs in fp64 (``gemm64``) rounded
                    once to bf16, the output type of the 8-bit path.  Pinned
                    by exact integer products (small integers are exact in
                    both formats) and by the decoded values fed through the
                    pinned fp64 product.
"""
from __future__ import annotations

import numpy as np

from . import gemm64

FORMATS = ("e4m3", "e5m2")


def decode(bits, fmt: str) -> np.ndarray:
    """Exact fp64 value of every 8-bit code in ``bits`` (any integer array)."""
    b = np.asarray(bits).astype(np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    if fmt == "e4m3":
        e = (b >> 3) & 0xF
        m = (b & 0x7).astype(np.float64)
        mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
        mag = np.where((e == 0xF) & (m == 7), np.nan, mag)
    elif fmt == "e5m2":
        e = (b >> 2) & 0x1F
        m = (b & 0x3).astype(np.float64)
        mag = np.where(e == 0, m / 4.0 * 2.0 ** -14, (1.0 + m / 4.0) * np.exp2(e - 15.0))
        mag = np.where(e == 0x1F, np.where(m == 0, np.inf, np.nan), mag)
    else:
        raise ValueError(f"unknown 8-bit format {fmt!r}")
    return sign * mag


def _bits(x) -> np.ndarray:
    """uint8 codes of a numpy array or a CPU torch float8 / uint8 tensor."""
    if isinstance(x, np.ndarray):
        return x.astype(np.uint8)
    import torch
    return x.detach().to("cpu").contiguous().view(torch.uint8).numpy()


def reference_fp8(A, B, fmt: str, nthreads: int | None = None):
    """The oracle's answer for 8-bit inputs A [M,K] and B [K,N] (or batched
    [batch, M, K] / [batch, K, N], one side may be 2-D and shared), given as
    codes: the fp64 product of the decoded values rounded once to bf16.
    Returns (rounded values as fp64, the unrounded fp64 product)."""
    a = decode(_bits(A), fmt)
    b = decode(_bits(B), fmt)
    if a.ndim == 2 and b.ndim == 2:
        C64 = gemm64.gemm_f64(a, b, nthreads)
    else:
        C64 = gemm64.gemm_batched_f64(a, b, nthreads)
    return gemm64.bits_to_f64(gemm64.round_to_bits(C64, "bf16"), "bf16"), C64


def decoded_max_abs(x, fmt: str) -> float:
    """Largest magnitude among the finite decoded inputs (0 when empty)."""
    v = decode(_bits(x), fmt)
    v = v[np.isfinite(v)]
    return float(np.abs(v).max()) if v.size else 0.0
