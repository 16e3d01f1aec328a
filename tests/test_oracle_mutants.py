"""The oracle's pins catch plausible mistakes.

Each mutant below is a copy of the oracle's three-loop algorithm with one
planted mistake (on the CPU, in Python).  The same pin checks used on the real
oracle - the printed worked example, exact brute force on tiny shapes and the
identity closed form - must reject every mutant and accept the unmutated
copy.
"""
import json
import os

import numpy as np
import pytest

from oracle import exact

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def three_loop(A, B, mutant=None):
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    M, K = A.shape
    N = B.shape[1]
    C = np.zeros((M, N))
    for i in range(M):
        for k in range(K):
            if mutant == "drop_last_k" and k == K - 1:
                continue
            if mutant == "reset_each_k_step" and k % 2 == 0:
                C[i, :] = 0.0                       # accumulator cleared per BK=2 step
            a = A[(i + 1) % M if mutant == "wrong_row" else i, k]
            for j in range(N):
                if mutant == "transposed_b":
                    b = B[j % K, k % N]
                elif mutant == "wrong_k_in_b":
                    b = B[(k + 1) % K, j]
                else:
                    b = B[k, j]
                term = a * b
                if mutant == "wrong_sign" and k == 1:
                    term = -term
                C[i, j] += term
    if mutant == "swapped_output":
        C = C[::-1, :].copy()
    return C


def pins_pass(fn) -> bool:
    g = GOLD["worked_example"]
    try:
        if fn(g["A"], g["B"]).tolist() != g["C"]:
            return False
        rng = np.random.default_rng(0)
        for M, N, K in [(2, 3, 4), (3, 2, 5), (4, 4, 3), (1, 5, 2)]:
            A = rng.integers(-4, 5, (M, K))
            B = rng.integers(-4, 5, (K, N))
            want = np.array(exact.exact_gemm(A.tolist(), B.tolist()), dtype=np.float64)
            if not np.array_equal(fn(A, B), want):
                return False
        B = rng.integers(-4, 5, (5, 5))
        if not np.array_equal(fn(np.eye(5), B), B.astype(np.float64)):
            return False
    except IndexError:
        return False
    return True


def test_unmutated_copy_passes():
    assert pins_pass(lambda A, B: three_loop(A, B))


@pytest.mark.parametrize("mutant", ["drop_last_k", "reset_each_k_step", "wrong_row",
                                    "transposed_b", "wrong_k_in_b", "wrong_sign",
                                    "swapped_output"])
def test_mutant_is_caught(mutant):
    assert not pins_pass(lambda A, B: three_loop(A, B, mutant))


# ---------------------------------------------------------------- batched
def batched_loop(A, B, mutant=None):
    """A copy of the batched oracle's loop over matrices, with a planted
    mistake."""
    batch = A.shape[0]
    out = []
    for i in range(batch):
        ia = 0 if mutant == "first_a_everywhere" else i
        ib = (i + 1) % batch if mutant == "shifted_b" else i
        out.append(three_loop(A[ia], B[ib]))
    return np.stack(out)


@pytest.mark.parametrize("mutant", [None, "first_a_everywhere", "shifted_b"])
def test_batched_pin_catches(mutant):
    rng = np.random.default_rng(3)
    A = rng.integers(-4, 5, (4, 3, 5)).astype(np.float64)
    B = rng.integers(-4, 5, (4, 5, 2)).astype(np.float64)
    ok = np.array_equal(batched_loop(A, B, mutant), np.matmul(A, B))
    assert ok == (mutant is None)


# ---------------------------------------------------------------- 8-bit decode
def decode_mutant(bits, fmt, mutant=None):
    """A copy of the oracle's 8-bit decode with one planted mistake."""
    b = np.asarray(bits).astype(np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    if fmt == "e4m3":
        ebits, mbits, bias = 4, 3, 7
    else:
        ebits, mbits, bias = 5, 2, 15
    if mutant == "wrong_bias":
        bias += 1
    e = (b >> mbits) & ((1 << ebits) - 1)
    m = (b & ((1 << mbits) - 1)).astype(np.float64)
    frac = m / (1 << mbits)
    if mutant == "subnormal_as_normal":
        sub = (1.0 + frac) * np.exp2(1.0 - bias - 1)
    else:
        sub = frac * 2.0 ** (1 - bias)
    mag = np.where(e == 0, sub, (1.0 + frac) * np.exp2(e - float(bias)))
    top = (1 << ebits) - 1
    if fmt == "e4m3":
        if mutant == "ieee_specials":
            mag = np.where(e == top, np.where(m == 0, np.inf, np.nan), mag)
        else:
            mag = np.where((e == top) & (m == 7), np.nan, mag)
    else:
        mag = np.where(e == top, np.where(m == 0, np.inf, np.nan), mag)
    if mutant == "sign_dropped":
        sign = np.ones_like(sign)
    return sign * mag


def decode_pins_pass(fn) -> bool:
    from test_oracle_pins import FP8_HAND, FP8_MAXCODE, FP8_NAN
    import math
    for fmt in ("e4m3", "e5m2"):
        for code, want in FP8_HAND[fmt].items():
            got = float(fn(np.array([code]), fmt)[0])
            if not (got == want and math.copysign(1, got) == math.copysign(1, want)):
                return False
        if not np.isnan(fn(np.array(FP8_NAN[fmt]), fmt)).all():
            return False
        pos = fn(np.arange(0, FP8_MAXCODE[fmt] + 1), fmt)
        if not (np.diff(pos) > 0).all():
            return False
    return True


def test_unmutated_decode_passes():
    assert decode_pins_pass(lambda b, f: decode_mutant(b, f))


@pytest.mark.parametrize("mutant", ["wrong_bias", "subnormal_as_normal", "ieee_specials",
                                    "sign_dropped"])
def test_decode_mutant_is_caught(mutant):
    assert not decode_pins_pass(lambda b, f: decode_mutant(b, f, mutant))


# ---------------------------------------------------------------- 8-bit input magnitude
def max_abs_mutant(x, fmt, mutant):
    """A copy of the oracle's decoded-max-abs with one planted mistake."""
    from oracle import fp8
    codes = fp8._bits(x)
    v = fp8.decode(codes, fmt)
    if mutant == "raw_codes":
        v = codes.astype(np.float64)
    elif mutant == "signed_max":
        v = v[np.isfinite(v)]
        return float(v.max()) if v.size else 0.0
    elif mutant == "specials_kept":   # infinities count (NaN still dropped)
        v = v[~np.isnan(v)]
        return float(np.abs(v).max()) if v.size else 0.0
    elif mutant == "first_only":
        v = v.reshape(-1)[:1]
    v = v[np.isfinite(v)]
    return float(np.abs(v).max()) if v.size else 0.0


@pytest.mark.parametrize("mutant", ["raw_codes", "signed_max", "specials_kept", "first_only"])
def test_max_abs_mutant_is_caught(mutant):
    import torch
    from test_oracle_pins import fp8_max_abs_checks
    caught = 0
    for fmt, tdt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        try:
            fp8_max_abs_checks(lambda x, f: max_abs_mutant(x, f, mutant), fmt, tdt)
        except AssertionError:
            caught += 1
    assert caught >= 1, mutant


def test_unmutated_max_abs_passes():
    import torch
    from test_oracle_pins import fp8_max_abs_checks
    for fmt, tdt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        fp8_max_abs_checks(lambda x, f: max_abs_mutant(x, f, None), fmt, tdt)
