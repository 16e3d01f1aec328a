"""Acceptance rule for comparing a GPU product with the rounded oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The oracle's fp64 product is rounded once to the output type; the GPU value
g and that reference r are compared in fp64.  An element passes when

    |g - r| <= max(rtol * |r|, floor),   floor = 1e-3 * sqrt(K) * max|A| * max|B|

with rtol 2e-3 for fp16 output, 1e-2 for bf16 and 1e-5 for fp32, max|A| and
max|B| taken over the rounded inputs.  A NaN where the reference is finite
fails, and a non-finite reference must be matched exactly.

Why these bounds hold for a correct kernel: fp16/bf16 products are exact in
fp32, and an fp32 sum of K terms in any order is within about K·2^-24·sum|a·b|
of the exact sum, far below the floor for the configured shapes; the single
rounding to the output then adds at most half an output ulp, and the GPU's
two roundings (fp32 sum, then fp32 -> output) can differ from the oracle's one
by one output ulp in rare double-rounding cases, which is 2^-10 relative for
fp16 (< 2e-3) and 2^-7 for bf16 (< 1e-2).
"""
from __future__ import annotations

import math

import numpy as np

RTOL = {"f16": 2e-3, "bf16": 1e-2, "f32": 1e-5}


def abs_floor(K: int, amax: float, bmax: float) -> float:
    return 1e-3 * math.sqrt(max(K, 0)) * amax * bmax


def compare(gpu: np.ndarray, ref: np.ndarray, dtype: str, K: int,
            amax: float, bmax: float, use_floor: bool = True) -> dict:
    """Element-wise check; returns a report dict with ``ok``."""
    g = np.asarray(gpu, dtype=np.float64).reshape(-1)
    r = np.asarray(ref, dtype=np.float64).reshape(-1)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    rtol = RTOL[dtype]
    fl = abs_floor(K, amax, bmax) if use_floor else 0.0
    finite = np.isfinite(r)
    err = np.where(finite, np.abs(g - r), 0.0)
    err = np.where(np.isnan(g) & finite, np.inf, err)
    bound = np.maximum(rtol * np.abs(r), fl)
    bad = finite & ~(err <= bound)
    nonfinite_bad = ~finite & ~((g == r) | (np.isnan(g) & np.isnan(r)))
    bad = bad | nonfinite_bad
    nb = int(bad.sum())
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(finite & (r != 0), err / np.abs(r), 0.0)
    rep = {
        "ok": nb == 0,
        "n": int(g.size),
        "n_bad": nb,
        "max_abs_err": float(err.max()) if g.size else 0.0,
        "max_rel_err": float(rel.max()) if g.size else 0.0,
        "floor": fl,
        "max_err_over_floor": float((err / fl).max()) if (g.size and fl > 0) else None,
        "n_not_bitequal": int((finite & (g != r)).sum()),
    }
    if nb:
        i = int(np.flatnonzero(bad)[0])
        rep["first_bad"] = {"flat_index": i, "gpu": float(g[i]), "ref": float(r[i]),
                            "bound": float(bound[i])}
    return rep
