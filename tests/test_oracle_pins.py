"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check uses a value the
pages print (tests/golden/pages_values.json, each entry cited), a closed form,
an exact rational brute force, or a library routine (numpy, CPython struct,
torch's own dtype conversions).
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import exact, gemm64, tolerance
from dense_gemm_run_amd.inputs import make_operands

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


# ---------------------------------------------------------------- worked example
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_worked_example_c_oracle(dtype):
    g = GOLD["worked_example"]
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    C = gemm64.gemm_f64(A, B)
    assert C.tolist() == g["C"]
    ref, _ = gemm64.reference(A, B, dtype)
    assert ref.tolist() == g["C"]          # integers <= 256: exact in every dtype


def test_worked_example_exact():
    g = GOLD["worked_example"]
    assert exact.exact_gemm(g["A"], g["B"]) == [[Fraction(v) for v in r] for r in g["C"]]


def test_worked_example_orientation():
    # B·A is a different (3x3) product; a transposed operand would not match.
    g = GOLD["worked_example"]
    BA = gemm64.gemm_f64(np.array(g["B"], float), np.array(g["A"], float))
    assert BA.shape == (3, 3)
    with pytest.raises(ValueError):
        gemm64.gemm_f64(np.array(g["A"], float), np.array(g["A"], float))


# ---------------------------------------------------------------- split-K walk
def test_split_k_contributions():
    g = GOLD["worked_example"]
    s = GOLD["split_k"]
    C, loads, steps = exact.tiled_walk(g["A"], g["B"], 2, 2, s["BK"])
    assert steps[(0, 0)] == s["C00_step_contributions"]
    assert C[0][0] == sum(s["C00_step_contributions"]) == g["C"][0][0]
    # an accumulator cleared at every K-step would keep only the last part
    assert steps[(0, 0)][-1] == s["C00_if_accumulator_reset_each_step"]
    assert C == exact.exact_gemm(g["A"], g["B"])


# ---------------------------------------------------------------- tile_ranges
def test_tile_ranges_printed():
    t = GOLD["tile_ranges"]
    assert exact.tile_ranges(t["n"], t["t"]) == [tuple(r) for r in t["ranges"]]


def test_tile_ranges_properties():
    for n in range(0, 60):
        for t in range(1, 14):
            rs = exact.tile_ranges(n, t)
            assert len(rs) == -(-n // t)
            covered = [i for a, b in rs for i in range(a, b)]
            assert covered == list(range(n))          # disjoint, ordered, complete
            assert all(b - a == t for a, b in rs[:-1])
            assert all(0 < b - a <= t for a, b in rs)


# ---------------------------------------------------------------- exit check
def test_exit_check_counts():
    e = GOLD["exit_check"]
    M, N, K, BM, BN, BK = (e[k] for k in ("M", "N", "K", "BM", "BN", "BK"))
    assert exact.program_count(M, N, BM, BN) == e["programs"]
    assert exact.k_steps(K, BK) == e["k_steps"]
    assert exact.needs_mask(M, N, K, BM, BN, BK) == e["masks"]
    # the same counts fall out of the tiled walk itself
    A = [[(3 * r + i) % 7 - 3 for i in range(K)] for r in range(M)]
    B = [[(5 * i + c) % 9 - 4 for c in range(N)] for i in range(K)]
    C, loads, steps = exact.tiled_walk(A, B, BM, BN, BK)
    assert C == exact.exact_gemm(A, B)
    assert all(len(v) == e["k_steps"] for v in steps.values())
    tiles = {(r // BM, c // BN) for r in range(M) for c in range(N)}
    assert len(tiles) == e["programs"]


# ---------------------------------------------------------------- traffic
def test_naive_waste_count_at_4096():
    w = GOLD["waste_count"]
    M, N, K = w["M"], w["N"], w["K"]
    loads = exact.naive_loads(M, N, K)
    assert loads == 2 * 4096 ** 3 == 137_438_953_472
    assert abs(loads - w["naive_loads_approx"]) / w["naive_loads_approx"] < 0.005
    assert abs(M * N - w["outputs_approx"]) / w["outputs_approx"] < 0.005
    distinct = M * K + K * N + M * N
    assert abs(distinct - w["distinct_values_approx"]) / w["distinct_values_approx"] < 0.01
    # every A element is read once per output column, every B element once per row
    assert (loads // 2) // (M * K) == w["fetches_per_element"]
    assert (loads // 2) // (K * N) == w["fetches_per_element"]


def test_tiled_traffic_is_one_over_t_at_64():
    t = GOLD["tiled_traffic_64"]
    M, N, K = t["M"], t["N"], t["K"]
    rng = np.random.default_rng(0)
    A = rng.integers(-3, 4, (M, K)).tolist()
    B = rng.integers(-3, 4, (K, N)).tolist()
    naive = exact.naive_loads(M, N, K)
    for T in t["tiles"]:
        _, loads, _ = exact.tiled_walk(A, B, T, T, T)
        assert loads * T == naive, T
        assert exact.tiled_loads(M, N, K, T, T) * T == naive


def test_tiled_traffic_closed_form_brute_force():
    # the closed form against the walk's own count, including ragged tiles
    rng = np.random.default_rng(1)
    for M, N, K, BM, BN, BK in [(5, 7, 5, 2, 3, 2), (7, 3, 4, 3, 3, 3), (6, 6, 6, 4, 5, 6),
                                (9, 4, 3, 2, 4, 1), (1, 8, 5, 3, 3, 4), (8, 1, 7, 8, 2, 5)]:
        A = rng.integers(-2, 3, (M, K)).tolist()
        B = rng.integers(-2, 3, (K, N)).tolist()
        C, loads, _ = exact.tiled_walk(A, B, BM, BN, BK)
        assert loads == exact.tiled_loads(M, N, K, BM, BN)
        assert C == exact.exact_gemm(A, B)
    # ragged example: the 1/T statement needs T to divide M and N
    assert exact.tiled_loads(64, 64, 64, 48, 48) == 16384 != 2 * 64 ** 3 // 48


# ---------------------------------------------------------------- intensity
def test_tile_reuse_ratio():
    t = GOLD["tile_reuse"]
    bm, bn, bk, s = t["BM"], t["BN"], t["BK"], t["dtype_bytes"]
    assert bm * bk + bk * bn == t["input_elements"]
    assert (bm * bk + bk * bn) * s == t["input_bytes"]
    assert 2 * bm * bn * bk == t["flops"]
    assert round(exact.tile_intensity(bm, bn, bk, s), 2) == t["flop_per_byte_approx"]


def test_whole_problem_intensity():
    w = GOLD["whole_problem_intensity"]
    ai = exact.matmul_intensity(w["m"], w["k"], w["n"], w["dtype_bytes"])
    assert round(ai) == w["approx"]
    assert ai == pytest.approx(4096 / 3)
    assert ai > w["threshold"]


def test_phase_intensity():
    p = GOLD["phase_intensity"]
    assert exact.phase_intensity_fp32(p["T"]) == p["tiled"]
    assert exact.phase_intensity_fp32(1) == p["naive"]
    assert exact.phase_intensity_fp32(p["T"]) / exact.phase_intensity_fp32(1) == p["ratio"]
    for T in (4, 8, 32, 64):
        assert exact.phase_intensity_fp32(T) == T / 4


def test_smem_tile_pair():
    s = GOLD["smem_tile_pair"]
    assert 2 * s["T"] * s["T"] * s["bytes_per_elem"] == s["bytes"]


# ---------------------------------------------------------------- grouped order
def test_grouped_order_bijection_and_row_major():
    for tm in range(1, 12):
        for tn in range(1, 12):
            for g in range(1, 10):
                seen = [exact.grouped_tile(p, tm, tn, g) for p in range(tm * tn)]
                assert sorted(seen) == [(r, c) for r in range(tm) for c in range(tn)]
                if g == 1:
                    assert seen == [(p // tn, p % tn) for p in range(tm * tn)]


def test_grouped_order_walks_down_band_first():
    tm, tn, g = 16, 16, 8
    first = [exact.grouped_tile(p, tm, tn, g) for p in range(g)]
    assert first == [(r, 0) for r in range(g)]
    assert exact.grouped_tile(g, tm, tn, g) == (0, 1)
    assert exact.grouped_tile(g * tn, tm, tn, g) == (g, 0)


# ---------------------------------------------------------------- brute force
def _rand_vals(M, N, K, dtype, seed):
    A, B = make_operands(M, N, K, dtype, "normal", seed)
    return A.to(torch.float64).numpy(), B.to(torch.float64).numpy()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_exact_bruteforce_all_tiny_shapes(dtype):
    for seed in (11, 12):
        for M in range(1, 7):
            for N in range(1, 7):
                for K in range(1, 7):
                    A, B = _rand_vals(M, N, K, dtype, seed * 1000 + M * 100 + N * 10 + K)
                    ex = exact.exact_gemm(A.tolist(), B.tolist())
                    want = np.array([[exact.rne_bits(v, dtype) for v in row] for row in ex])
                    got = gemm64.round_to_bits(gemm64.gemm_f64(A, B), dtype)
                    assert np.array_equal(got, want), (dtype, M, N, K)


def test_integer_closed_forms():
    # identity: I·B = B exactly
    _, B = make_operands(1, 37, 37, "f32", "normal", 3)
    I = np.eye(37)
    assert np.array_equal(gemm64.gemm_f64(I, B.double().numpy()), B.double().numpy())
    # all ones: every entry is K
    for K in (1, 64, 65, 2048, 2049, 4097):
        C = gemm64.gemm_f64(np.ones((3, K)), np.ones((K, 5)))
        assert (C == K).all()
    # fp16 above 2048 rounds to even steps of 2: 2049 is a tie -> 2048, 2051 -> 2052
    assert gemm64.bits_to_f64(gemm64.round_to_bits(np.array([2049.0, 2051.0]), "f16"), "f16").tolist() == [2048.0, 2052.0]
    # bf16 above 256 rounds to steps of 2: 257 -> 256, 259 -> 260
    assert gemm64.bits_to_f64(gemm64.round_to_bits(np.array([257.0, 259.0]), "bf16"), "bf16").tolist() == [256.0, 260.0]


def test_integers_against_exact_integer_matmul():
    for (M, N, K, seed) in [(17, 23, 300, 0), (64, 64, 64, 1), (5, 129, 1000, 2)]:
        A, B = make_operands(M, N, K, "f32", "integers", seed)
        Ai = A.numpy().astype(np.int64)
        Bi = B.numpy().astype(np.int64)
        assert np.array_equal(gemm64.gemm_f64(A, B), (Ai @ Bi).astype(np.float64))


def test_against_numpy_float64_matmul():
    rng = np.random.default_rng(5)
    for M, N, K in [(100, 120, 300), (33, 1, 1000), (1, 77, 513)]:
        A = rng.standard_normal((M, K))
        B = rng.standard_normal((K, N))
        got = gemm64.gemm_f64(A, B)
        want = A @ B
        bound = K * 2.0 ** -52 * (np.abs(A) @ np.abs(B))
        assert (np.abs(got - want) <= bound).all()


def test_points_rows_and_threads_agree():
    A, B = make_operands(70, 90, 130, "bf16", "normal", 9)
    full = gemm64.gemm_f64(A, B, nthreads=1)
    assert np.array_equal(full, gemm64.gemm_f64(A, B, nthreads=4))
    rows = np.array([0, 69, 33, 5, 69])
    cols = np.array([0, 89, 44, 89, 0])
    assert np.array_equal(gemm64.gemm_points_f64(A, B, rows, cols), full[rows, cols])
    assert np.array_equal(gemm64.gemm_rows_f64(A, B, 20, 7), full[20:27])
    t, blk = gemm64.time_rows_f64(A.double().numpy(), B.double().numpy(), 3, 4, 2)
    assert t >= 0 and np.array_equal(blk, full[3:7])


def _int_batch(shape, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(-4, 5, shape).astype(np.float64)


@pytest.mark.parametrize("a_shared,b_shared", [(False, False), (True, False), (False, True)])
def test_batched_against_numpy_batched_matmul(a_shared, b_shared):
    # integer entries with small K: every sum is exact in fp64 and in numpy
    batch, M, N, K = 5, 7, 9, 33
    A = _int_batch((M, K) if a_shared else (batch, M, K), 11)
    B = _int_batch((K, N) if b_shared else (batch, K, N), 12)
    got = gemm64.gemm_batched_f64(A, B)
    assert got.shape == (batch, M, N)
    assert np.array_equal(got, np.matmul(A, B))
    # matrix i of the result depends on matrix i of each 3-D operand only
    if not a_shared:
        A2 = A.copy()
        A2[2] += 1
        d = gemm64.gemm_batched_f64(A2, B) != got
        assert d[2].any() and not d[[0, 1, 3, 4]].any()


def test_batched_degenerate_and_rounded():
    assert gemm64.gemm_batched_f64(np.zeros((0, 3, 4)), np.zeros((0, 4, 5))).shape == (0, 3, 5)
    A = _int_batch((3, 4, 6), 13)
    B = _int_batch((3, 6, 2), 14)
    ref, raw = gemm64.reference_batched(A, B, "bf16")
    assert np.array_equal(raw, np.matmul(A, B))
    assert np.array_equal(ref, raw)          # |sums| <= 96: exact in bf16
    with pytest.raises(ValueError):
        gemm64.gemm_batched_f64(np.zeros((2, 3, 4)), np.zeros((3, 4, 5)))


def test_degenerate_sizes():
    assert gemm64.gemm_f64(np.zeros((0, 4)), np.zeros((4, 3))).shape == (0, 3)
    assert gemm64.gemm_f64(np.zeros((2, 4)), np.zeros((4, 0))).shape == (2, 0)
    C = gemm64.gemm_f64(np.zeros((3, 0)), np.zeros((0, 5)))
    assert C.shape == (3, 5) and (C == 0).all() and not np.signbit(C).any()


# ---------------------------------------------------------------- rounding
def _wide_doubles(n, seed):
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(-160, 140, n)
    sign = rng.choice([-1.0, 1.0], n)
    return sign * np.ldexp(mant, expo)


def test_round_f16_against_numpy_and_struct():
    x = np.concatenate([_wide_doubles(200_000, 1) / 2 ** 100 * 2 ** 80,
                        np.random.default_rng(2).standard_normal(100_000) * 3e4,
                        np.random.default_rng(3).standard_normal(100_000) * 1e-6])
    got = gemm64.round_to_bits(x, "f16")
    assert np.array_equal(got, x.astype(np.float16).view(np.uint16))
    for v in x[:3000]:
        try:
            want = struct.unpack("<H", struct.pack("<e", float(v)))[0]
        except OverflowError:
            want = 0x7C00 | (0x8000 if v < 0 else 0)
        assert int(gemm64.round_to_bits(np.array([v]), "f16")[0]) == want


def test_round_bf16_against_torch_on_fp32_values():
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 2 ** 32, 300_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = gemm64.round_to_bits(f.astype(np.float64), "bf16")
    assert np.array_equal(got, want)


def test_round_f32_against_numpy():
    x = _wide_doubles(300_000, 6)
    got = gemm64.round_to_bits(x, "f32")
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", ["f16", "bf16", "f32"])
def test_round_against_exact_rational(fmt):
    x = _wide_doubles(4000, 7)
    got = gemm64.round_to_bits(x, fmt)
    want = [exact.rne_bits(float(v), fmt) for v in x]
    assert got.tolist() == want


def test_round_hand_checked_cases():
    f16 = {1 + 2 ** -11: 0x3C00, 1 + 3 * 2 ** -11: 0x3C02, 65504.0: 0x7BFF,
           65519.99: 0x7BFF, 65520.0: 0x7C00, 2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000,
           3 * 2.0 ** -25: 0x0002, 2.0 ** -14: 0x0400, -2.0: 0xC000, 1e300: 0x7C00,
           float("inf"): 0x7C00, float("-inf"): 0xFC00}
    for v, b in f16.items():
        assert int(gemm64.round_to_bits(np.array([v]), "f16")[0]) == b, v
        if math.isfinite(v) and v != 0:
            assert exact.rne_bits(v, "f16") == b, v
    bf16 = {1 + 2 ** -8: 0x3F80, 1 + 3 * 2 ** -8: 0x3F82, 1.0: 0x3F80,
            (2 - 2 ** -7) * 2.0 ** 127: 0x7F7F, (2 - 2 ** -8) * 2.0 ** 127: 0x7F80,
            2.0 ** -133: 0x0001, 2.0 ** -126: 0x0080, -1.5: 0xBFC0}
    for v, b in bf16.items():
        assert int(gemm64.round_to_bits(np.array([v]), "bf16")[0]) == b, v
        assert exact.rne_bits(v, "bf16") == b, v
    # signed zeros (a dict cannot hold both: 0.0 == -0.0)
    assert int(gemm64.round_to_bits(np.array([0.0]), "f16")[0]) == 0x0000
    assert int(gemm64.round_to_bits(np.array([-0.0]), "f16")[0]) == 0x8000
    assert int(gemm64.round_to_bits(np.array([-2.0 ** -26]), "f16")[0]) == 0x8000
    assert exact.rne_bits(-2.0 ** -26, "f16") == 0x8000
    assert int(gemm64.round_to_bits(np.array([float("nan")]), "f16")[0]) == 0x7E00
    assert int(gemm64.round_to_bits(np.array([float("nan")]), "bf16")[0]) == 0x7FC0
    assert int(gemm64.round_to_bits(np.array([float("nan")]), "f32")[0]) == 0x7FC00000


def test_bits_roundtrip():
    for fmt in ("f16", "bf16"):
        bits = np.arange(0, 1 << 16, dtype=np.uint32)
        expf = (bits >> (10 if fmt == "f16" else 7)) & (0x1F if fmt == "f16" else 0xFF)
        finite = expf != (0x1F if fmt == "f16" else 0xFF)
        vals = gemm64.bits_to_f64(bits[finite], fmt)
        back = gemm64.round_to_bits(vals, fmt).astype(np.uint32)
        negzero = bits[finite] == 0x8000
        assert np.array_equal(back[~negzero], bits[finite][~negzero])
        for b in bits[finite][::97]:
            assert exact.bits_value(int(b), fmt) == Fraction(float(gemm64.bits_to_f64(np.array([b]), fmt)[0]))


# ---------------------------------------------------------------- fp32 data
def test_fp32_fine_inputs_discriminate_reduced_precision():
    # Shortening fp32 inputs to a 10-bit (or 7-bit) significand before
    # multiplying moves these products far beyond the 1e-5 fp32 tolerance.
    A, B = make_operands(64, 64, 64, "f32", "fp32_fine", 21)
    full = gemm64.gemm_f64(A, B)

    def chop(t, keep):
        b = t.numpy().view(np.uint32) & np.uint32((0xFFFFFFFF << (23 - keep)) & 0xFFFFFFFF)
        return b.view(np.float32).astype(np.float64)

    for keep in (10, 7):
        short = gemm64.gemm_f64(chop(A, keep), chop(B, keep))
        rel = np.abs(short - full) / np.abs(full)
        assert rel.min() > 1e-4, keep
    # and the values really are fp32 values with low bits in use
    low = A.numpy().view(np.uint32) & 0x1FFF
    assert (low != 0).mean() > 0.99


# ---------------------------------------------------------------- tolerance rule
def test_tolerance_rule():
    ref = np.array([1.0, 100.0, 1e-3, 0.0])
    rep = tolerance.compare(ref.copy(), ref, "f16", K=64, amax=1.0, bmax=1.0)
    assert rep["ok"] and rep["n_not_bitequal"] == 0
    fl = tolerance.abs_floor(64, 1.0, 1.0)
    assert fl == pytest.approx(8e-3)
    # within rtol at large magnitude, within floor at small magnitude
    g = ref + np.array([1.9e-3, 0.19, 7e-3, -7e-3])
    assert tolerance.compare(g, ref, "f16", 64, 1.0, 1.0)["ok"]
    g = ref + np.array([0.0, 0.21, 0.0, 0.0])
    assert not tolerance.compare(g, ref, "f16", 64, 1.0, 1.0)["ok"]
    g = ref + np.array([0.0, 0.0, 0.0, 9e-3])
    assert not tolerance.compare(g, ref, "f16", 64, 1.0, 1.0)["ok"]
    g = ref.copy()
    g[0] = np.nan
    assert not tolerance.compare(g, ref, "f16", 64, 1.0, 1.0)["ok"]
    # one fp16 ulp of double rounding at any magnitude passes; bf16 likewise
    for v in (1.0, 37.5, 1000.0):
        assert tolerance.compare(np.array([v * (1 + 2 ** -10)]), np.array([v]), "f16", 1, 1e-9, 1e-9)["ok"]
        assert tolerance.compare(np.array([v * (1 + 2 ** -7)]), np.array([v]), "bf16", 1, 1e-9, 1e-9)["ok"]
    assert not tolerance.compare(np.array([1.0 + 2e-5]), np.array([1.0]), "f32", 1, 1e-9, 1e-9)["ok"]


# ---------------------------------------------------------------- 8-bit inputs
# The 8-bit formats are the OCP FP8 ones (E4M3: bias 7, 3 significand bits,
# S.1111.111 NaN, no infinities; E5M2: bias 15, 2 significand bits, IEEE-style
# infinities and NaNs).  Hand-checked codes from those definitions:
FP8_HAND = {
    "e4m3": {0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0xB8: -1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0,
             0x77: 240.0, 0x3F: 1.875},
    "e5m2": {0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -16, 0x03: 3 * 2.0 ** -16, 0x04: 2.0 ** -14,
             0x3C: 1.0, 0xBC: -1.0, 0x3D: 1.25, 0x7B: 57344.0, 0xFB: -57344.0,
             0x7C: math.inf, 0xFC: -math.inf},
}
FP8_NAN = {"e4m3": [0x7F, 0xFF], "e5m2": [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]}
FP8_MAXCODE = {"e4m3": 0x7E, "e5m2": 0x7B}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decode_hand_values(fmt):
    from oracle import fp8
    for code, want in FP8_HAND[fmt].items():
        got = float(fp8.decode(np.array([code]), fmt)[0])
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (hex(code), got)
    nan = fp8.decode(np.array(FP8_NAN[fmt]), fmt)
    assert np.isnan(nan).all()
    everything = fp8.decode(np.arange(256), fmt)
    assert int(np.isnan(everything).sum()) == len(FP8_NAN[fmt])


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_decode_matches_torch_on_every_code(fmt, tdt):
    from oracle import fp8
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(tdt).to(torch.float64).numpy()
    got = fp8.decode(codes.numpy(), fmt)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_fp8_e5m2_is_binary16_with_low_byte_zero():
    from oracle import fp8
    codes = np.arange(256, dtype=np.uint16)
    want = (codes << 8).view(np.float16).astype(np.float64)
    got = fp8.decode(codes, "e5m2")
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decode_order_and_sign(fmt):
    from oracle import fp8
    top = FP8_MAXCODE[fmt]
    pos = fp8.decode(np.arange(0, top + 1), fmt)
    assert (np.diff(pos) > 0).all()
    neg = fp8.decode(np.arange(0, top + 1) | 0x80, fmt)
    assert np.array_equal(neg, -pos)
    # every value is exact in bf16 and in fp16 (the widenings the GPU path may use)
    v = pos[1:]
    assert np.array_equal(v.astype(np.float16).astype(np.float64), v)
    bf = gemm64.bits_to_f64(gemm64.round_to_bits(v, "bf16"), "bf16")
    assert np.array_equal(bf, v)


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_reference_on_integers(fmt, tdt):
    # integers in [-4, 4] are exact in both formats; with K = 16 every sum
    # is an integer of magnitude <= 256, which bf16 holds exactly
    from oracle import fp8
    rng = np.random.default_rng(21)
    M, N, K = 9, 11, 16
    A = rng.integers(-4, 5, (M, K))
    B = rng.integers(-4, 5, (K, N))
    At = torch.from_numpy(A.astype(np.float32)).to(tdt)
    Bt = torch.from_numpy(B.astype(np.float32)).to(tdt)
    ref, raw = fp8.reference_fp8(At, Bt, fmt)
    exact_c = np.array(exact.exact_gemm(A.tolist(), B.tolist()), dtype=np.float64)
    assert np.array_equal(raw, exact_c)
    assert np.array_equal(ref, exact_c)      # |sums| <= 256: exact in bf16
    # batched, B shared
    A3 = np.stack([A, -A, 2 * A])
    r3, raw3 = fp8.reference_fp8(torch.from_numpy(A3.astype(np.float32)).to(tdt), Bt, fmt)
    assert np.array_equal(raw3, np.stack([exact_c, -exact_c, 2 * exact_c]))


def test_fp8_reference_rounds_once_to_bf16():
    from oracle import fp8
    # [1, 1, 1] . [1, 2^-8, 2^-12] = 1 + 2^-8 + 2^-12 is not a bf16 value; it
    # lies above the half-way point 1 + 2^-8, so it rounds to 1 + 2^-7 (a
    # rounding of the partial sum 1 + 2^-8 first would give the tie and 1.0)
    b5 = np.array([[0x3C], [0x1C], [0x0C]], dtype=np.uint8)   # E5M2: 1, 2^-8, 2^-12
    a5 = np.array([[0x3C, 0x3C, 0x3C]], dtype=np.uint8)
    assert list(fp8.decode(b5.ravel(), "e5m2")) == [1.0, 2.0 ** -8, 2.0 ** -12]
    ref, raw = fp8.reference_fp8(a5, b5, "e5m2")
    assert raw[0, 0] == 1 + 2.0 ** -8 + 2.0 ** -12
    assert ref[0, 0] == 1 + 2.0 ** -7


def fp8_max_abs_checks(fn, fmt, tdt):
    """Checks of a decoded-max-abs function ``fn(codes, fmt)`` (raises
    AssertionError on the first failure).  Expected values come from the OCP
    definitions (E4M3 largest 448, E5M2 largest 57344; NaN and infinity codes
    are not values and are left out)."""
    from oracle import fp8
    # every code: the format's largest finite magnitude
    assert fn(np.arange(256, dtype=np.uint8), fmt) == {"e4m3": 448.0, "e5m2": 57344.0}[fmt]
    # the magnitude counts, not the signed value or the raw code: -4 (0xC8
    # in E4M3, 0xC4 in E5M2) against +1 (0x38 / 0x3C) gives 4, where the
    # largest raw code (0xC8 = 200) or the largest signed value (1) would not
    minus4 = {"e4m3": 0xC8, "e5m2": 0xC4}[fmt]
    one = {"e4m3": 0x38, "e5m2": 0x3C}[fmt]
    assert list(fp8.decode(np.array([minus4, one]), fmt)) == [-4.0, 1.0]
    assert fn(np.array([minus4, one], dtype=np.uint8), fmt) == 4.0
    assert fn(np.array([one, minus4], dtype=np.uint8), fmt) == 4.0
    # the smallest subnormal alone (2^-9 / 2^-16)
    assert fn(np.array([0x81], dtype=np.uint8), fmt) == {"e4m3": 2.0 ** -9, "e5m2": 2.0 ** -16}[fmt]
    # NaN (and, for E5M2, infinity) codes only, or nothing: 0
    specials = np.array(FP8_NAN[fmt] + ([0x7C, 0xFC] if fmt == "e5m2" else []), dtype=np.uint8)
    assert fn(specials, fmt) == 0.0
    assert fn(np.array([], dtype=np.uint8), fmt) == 0.0
    # a special next to a finite value is ignored
    assert fn(np.concatenate([specials, np.array([one], dtype=np.uint8)]), fmt) == 1.0
    # a CPU torch tensor of the format is read by its codes: -3.5 and 1.0 give 3.5
    t = torch.tensor([[-3.5, 1.0], [0.0, 0.5]]).to(tdt)
    assert fn(t, fmt) == 3.5


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_decoded_max_abs(fmt, tdt):
    """The largest finite magnitude of a set of 8-bit codes, which sets the
    absolute floor of the 8-bit comparisons."""
    from oracle import fp8
    fp8_max_abs_checks(fp8.decoded_max_abs, fmt, tdt)
