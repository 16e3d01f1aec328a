"""Exact pure-Python reference pieces for the dense matrix product.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow on purpose: used
on tiny shapes and as the independent check of the C oracle.

Contents and sources
--------------------
``exact_gemm``        C[row,col] = sum_inner A[row,inner]*B[inner,col] in exact
                      rational arithmetic (lesson "Matrix multiplication: reuse
                      the inputs", section "The three dimensions have different
                      jobs").  Pinned by the worked 2x3·3x2 example printed
                      there and by integer closed forms.
``rne_bits``          round-to-nearest-even of an exact rational into binary16,
                      bfloat16 or binary32 (the reading of the final cast; see
                      ``gemm64``).  Pinned against numpy / CPython binary16 and
                      torch fp32->bf16 conversions and hand-checked ties.
``tile_ranges``       the half-open partition of one dimension into tiles
                      (same lesson, section "Tiles are small rectangles of
                      work").  Pinned by the printed tile_ranges(7,3).
``tiled_walk``        the output-tile by K-step walk of that section, with each
                      step's contribution kept and every element copied into a
                      tile counted as one load, as the CPU load counter of
                      chapter "Fast matrix multiplication" (section "Tiling:
                      load once, use many times") counts them.  Pinned by the
                      printed BK=2 split of C[0,0] (25 then 33), the exit-check
                      counts of "Connect to the real implementation", and the
                      1/T traffic statement.
``grouped_tile``      the grouped program ordering (kernels-book chapter
                      "Matrix Multiplication", section "The naive version";
                      lesson section "Connect to the real implementation"):
                      walk down a band of GROUP_M tile-rows, then move right.
                      Pinned by its bijection property and by GROUP_M=1 being
                      plain row-major order, as the lesson states.
``naive_loads`` ...   the traffic and intensity models: naive 2MNK loads
                      (chapter "Matrix Multiplication", "Why this is slow";
                      chapter "Fast matrix multiplication", "Counting the
                      waste"), tiled loads, whole-problem intensity (notebook
                      "Triton tiled matmul", "Correctness check"), tile reuse
                      ratio (lesson, "Why tiling can improve throughput") and
                      phase intensity T/4 (chapter "Fast matrix
                      multiplication", the tiling equation).  Pinned by the
                      numbers printed with each.
"""
from __future__ import annotations

from fractions import Fraction
from math import ceil

# (significand bits incl. hidden bit, minimum normal exponent, maximum exponent,
#  exponent field width, total width)
FORMATS = {
    "f16": (11, -14, 15, 5, 16),
    "bf16": (8, -126, 127, 8, 16),
    "f32": (24, -126, 127, 8, 32),
}


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def exact_gemm(A, B):
    """Exact product of A [M][K] and B [K][N] (lists of lists of ints, floats
    or Fractions); every entry is a Fraction.  Rows are separate lists."""
    M = len(A)
    K = len(B)
    N = len(B[0]) if K else 0
    if M and len(A[0]) != K:
        raise ValueError("A's column count must match B's row count")
    out = []
    for r in range(M):
        row = []
        for c in range(N):
            s = Fraction(0)
            for i in range(K):
                s += Fraction(A[r][i]) * Fraction(B[i][c])
            row.append(s)
        out.append(row)
    return out


def _floor_log2(x: Fraction) -> int:
    """e with 2^e <= x < 2^(e+1), for x > 0."""
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    elif Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def rne_bits(x, fmt: str) -> int:
    """Bit pattern of the exact rational (or float) ``x`` rounded to nearest,
    ties to even, in format ``fmt``.  Overflow gives infinity; an exact zero
    gives +0 (the sign a sum that starts from +0 ends with)."""
    p, emin, emax, ebits, width = FORMATS[fmt]
    sign_bit = 1 << (width - 1)
    mbits = p - 1
    inf_bits = ((1 << ebits) - 1) << mbits
    if isinstance(x, float):
        if x != x:
            return inf_bits | (1 << (mbits - 1))
        if x in (float("inf"), float("-inf")):
            return inf_bits | (sign_bit if x < 0 else 0)
    x = Fraction(x)
    if x == 0:
        return 0
    sign = sign_bit if x < 0 else 0
    ax = abs(x)
    e = max(_floor_log2(ax), emin)
    q = e - mbits                              # quantum is 2^q
    y = ax / Fraction(2) ** q
    r = y.numerator // y.denominator           # floor
    rem = y - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    if r == 0:                                 # rounds to a zero of x's sign
        return sign
    v = r * Fraction(2) ** q
    maxfin = ((1 << p) - 1) * Fraction(2) ** (emax - mbits)
    if v > maxfin:
        return sign | inf_bits
    ev = _floor_log2(v)
    bias = (1 << (ebits - 1)) - 1
    if ev < emin:                              # subnormal: exponent field 0
        mant = v / Fraction(2) ** (emin - mbits)
        return sign | int(mant)
    mant = v / Fraction(2) ** (ev - mbits) - (1 << mbits)
    return sign | ((ev + bias) << mbits) | int(mant)


def bits_value(bits: int, fmt: str) -> Fraction | float:
    """Exact value of a finite bit pattern (inf/nan returned as floats)."""
    p, emin, emax, ebits, width = FORMATS[fmt]
    mbits = p - 1
    sign = -1 if bits >> (width - 1) else 1
    expf = (bits >> mbits) & ((1 << ebits) - 1)
    mant = bits & ((1 << mbits) - 1)
    if expf == (1 << ebits) - 1:
        return float("nan") if mant else sign * float("inf")
    bias = (1 << (ebits - 1)) - 1
    if expf == 0:
        return sign * mant * Fraction(2) ** (emin - mbits)
    return sign * ((1 << mbits) + mant) * Fraction(2) ** (expf - bias - mbits)


def tile_ranges(n: int, t: int) -> list[tuple[int, int]]:
    """Half-open [start, stop) pieces of length t covering [0, n); the last
    piece is shorter when t does not divide n."""
    if t <= 0:
        raise ValueError("tile size must be positive")
    return [(s, min(s + t, n)) for s in range(0, n, t)]


def tiled_walk(A, B, BM: int, BN: int, BK: int):
    """Compute C tile by tile the way one program per output tile does it.

    Each output tile [BM, BN] keeps one accumulator that starts at zero and
    survives every K-step; each K-step adds A_tile·B_tile for its K range.
    Returns (C, loads, steps) where ``loads`` counts every element copied into
    an A or B tile (in-range elements only, as slicing a ragged edge tile
    gives) and ``steps[(r, c)]`` lists the contribution each K-step made to
    C[r][c], in order.
    """
    M, K = len(A), len(B)
    N = len(B[0]) if K else 0
    C = [[Fraction(0)] * N for _ in range(M)]
    steps: dict[tuple[int, int], list[Fraction]] = {}
    loads = 0
    for r0, r1 in tile_ranges(M, BM):
        for c0, c1 in tile_ranges(N, BN):
            acc = {(r, c): Fraction(0) for r in range(r0, r1) for c in range(c0, c1)}
            for k0, k1 in tile_ranges(K, BK):
                loads += (r1 - r0) * (k1 - k0) + (k1 - k0) * (c1 - c0)
                for r in range(r0, r1):
                    for c in range(c0, c1):
                        part = sum((Fraction(A[r][i]) * Fraction(B[i][c])
                                    for i in range(k0, k1)), Fraction(0))
                        acc[(r, c)] += part
                        steps.setdefault((r, c), []).append(part)
            for (r, c), v in acc.items():
                C[r][c] = v
    return C, loads, steps


def grouped_tile(pid: int, tiles_m: int, tiles_n: int, group_m: int) -> tuple[int, int]:
    """Tile (row, col) owned by 1-D program ``pid``: programs fill a band of
    ``group_m`` tile-rows column by column (down the band first, then one
    column right); the last band holds whatever tile-rows remain."""
    band, within = divmod(pid, group_m * tiles_n)
    top = band * group_m
    height = min(group_m, tiles_m - top)
    col, down = divmod(within, height)
    return top + down, col


def program_count(M: int, N: int, BM: int, BN: int) -> int:
    """One program per output tile."""
    return cdiv(M, BM) * cdiv(N, BN)


def k_steps(K: int, BK: int) -> int:
    return cdiv(K, BK)


def needs_mask(M: int, N: int, K: int, BM: int, BN: int, BK: int) -> dict[str, bool]:
    """Which dimensions have a ragged last tile (and so need masking)."""
    return {"M": M % BM != 0, "N": N % BN != 0, "K": K % BK != 0}


def naive_loads(M: int, N: int, K: int) -> int:
    """One program per output element loads K of A and K of B."""
    return 2 * M * N * K


def tiled_loads(M: int, N: int, K: int, BM: int, BN: int) -> int:
    """Elements loaded by the tiled walk: each of the ceil(M/BM)·ceil(N/BN)
    tiles reads its rows of A and its columns of B once across all of K."""
    return K * (M * cdiv(N, BN) + N * cdiv(M, BM))


def matmul_intensity(m: int, k: int, n: int, dtype_bytes: int = 2) -> float:
    """Whole-problem FLOP per compulsory byte: 2mkn over reading A and B and
    writing C once."""
    return 2 * m * k * n / (dtype_bytes * (m * k + k * n + m * n))


def tile_intensity(bm: int, bn: int, bk: int, dtype_bytes: int = 2) -> float:
    """FLOP per input byte of one BM x BN x BK tile step (output excluded)."""
    return 2 * bm * bn * bk / (dtype_bytes * (bm * bk + bk * bn))


def phase_intensity_fp32(T: int) -> float:
    """FLOP per byte of one shared-memory phase with T x T fp32 tiles: 2T^3
    FLOP over two T x T tiles of 4-byte values."""
    return 2 * T ** 3 / (2 * T * T * 4)
