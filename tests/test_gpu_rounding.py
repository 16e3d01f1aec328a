"""Bit-exact GPU check of the one rounding from the fp32 sum to the output
type (round to nearest, ties to even; overflow to infinity; gradual
underflow; NaN and infinity propagation), in every kernel configuration,
the split-K reduction and gemm_run's own choice.

The operation's last step converts the fp32 accumulator to the output type
(lesson "Matrix multiplication: reuse the inputs", section "Connect to the
real implementation"; the Triton kernel of chapter "Fast matrix
multiplication"); the pages do not name the rounding mode, and the reading
here is IEEE round-to-nearest-even.  The inputs below are chosen so that every
fp32 partial sum is exact in any order (sums of few terms, or of equal
powers of two), so the GPU's fp32 sum equals the exact sum and its rounding
must equal the oracle's fp64 -> output rounding bit for bit:

* ties: A[i, k] = 1 for k < c_i (else 0) and B[k, j] = 1 for k >= j (else
  0), so C[i, j] = c_i - j, every integer from 0 to K-1 somewhere: odd sums
  between 2048 and 4096 are fp16 ties (spacing 2), sums from 4096 round to
  multiples of 4 (4097 -> 4096, 4098 -> 4096, 4102 -> 4104); for bf16 the
  ties start at 256.  c_0, c_1, c_2 = 2049, 2051, 4097 are all-ones rows.
* overflow: two or three large terms per row: 32768 + 32736 = 65504 (the
  largest fp16 value) stays, 65519 rounds down to it, 65520 (the tie with
  the first value past the range) and above become +inf; the negated rows
  -inf; bf16 2^127 + 2^127 overflows in fp32 already.
* subnormal outputs (fp16): A = 2^-13 for k < c_i, B = 2^-12, so
  C = c_i * 2^-25: half-integer multiples of the smallest subnormal 2^-24,
  ties to even; c_i up to 2050 reaches the smallest normal 2^-14.
  Subnormal inputs: A = 2^-24 (k < c_i) against B = 1 gives exact subnormal
  sums (input subnormals are not flushed).
* NaN and infinity inputs: a NaN in row 5 makes the whole row NaN, +inf and
  -inf in rows 9 and 11 meet zeros of B (NaN) and signed values (signed
  infinities).
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_run_amd as dg
from oracle import gemm64

pytestmark = pytest.mark.gpu

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
CODE = {"f16": 1, "bf16": 2}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def ties_operands(dtype, M, N, K):
    c = (150 + (np.arange(M, dtype=np.int64) * 2654435761) % (K - 150)).astype(np.int64)
    if dtype == "f16":
        c[:3] = [2049, 2051, 4097]
    else:
        c[:3] = [257, 259, 513]
    k = np.arange(K)
    A = (k[None, :] < c[:, None]).astype(np.float32)
    B = (k[:, None] >= np.arange(N)[None, :]).astype(np.float32)
    return A, B


def overflow_operands(dtype, M, N, K):
    A = np.zeros((M, K), dtype=np.float32)
    if dtype == "f16":
        rows = [(32768, 32736, 0), (32768, 32736, 8), (32768, 32736, 15), (32768, 32752, 0),
                (32768, 32752, 1), (60000, 60000, 60000), (65504, -65504, 1), (16384, 16384, 16384)]
    else:
        # (no cancelling terms: 2^127 - 2^127 + 1 depends on the fp32 order)
        big = 2.0 ** 127
        rows = [(big, big, 0), (big, 2.0 ** 126, 0), (1.5 * big, 1.5 * big, 0),
                (1.5 * 2.0 ** 126, 1.5 * 2.0 ** 126, 1.5 * 2.0 ** 126), (2.0 ** 126, 2.0 ** 126, 0),
                (1.5 * 2.0 ** 126, 2.0 ** 125, 2.0 ** 124)]
    for i in range(M):
        r = rows[i % len(rows)]
        s = -1.0 if (i // len(rows)) % 2 else 1.0
        A[i, :3] = [s * v for v in r]
    B = np.ones((K, N), dtype=np.float32)
    return A, B


def subnormal_operands(M, N, K):
    # rows 0 .. M/2-1: 2^-13 * 2^-12 products; the rest: subnormal inputs
    h = M // 2
    c = np.concatenate([np.arange(h) * 37 % 2051, np.arange(M - h) * 13 % 1030])
    c[:4] = [1, 3, 2047, 2050]
    k = np.arange(K)
    mask = (k[None, :] < c[:, None])
    A = np.where(mask, np.float32(2.0 ** -13), np.float32(0)).astype(np.float32)
    A[h:] = np.where(mask[h:], np.float32(2.0 ** -24), np.float32(0))
    B = np.full((K, N), 2.0 ** -12, dtype=np.float32)
    Bsub = np.ones((K, N), dtype=np.float32)
    return A, B, Bsub, h


def nan_operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rng.integers(-3, 4, (M, K)).astype(np.float32)
    B = rng.integers(-3, 4, (K, N)).astype(np.float32)
    A[5, 7] = np.nan
    A[9, 3] = np.inf
    A[11, 2] = -np.inf
    B[3, ::3] = 0.0
    B[2, ::4] = 0.0
    return A, B


def expect_bits(A, B, dtype):
    """The oracle's answer as output bit patterns."""
    C64 = gemm64.gemm_f64(A.to(torch.float64).numpy(), B.to(torch.float64).numpy())
    return gemm64.round_to_bits(C64, dtype)


def assert_bits(c_gpu, want, dtype, label):
    got = c_gpu.to("cpu").view(torch.int16).numpy().astype(np.uint16)
    gv = gemm64.bits_to_f64(got, dtype)
    wv = gemm64.bits_to_f64(want, dtype)
    nan_g, nan_w = np.isnan(gv), np.isnan(wv)
    assert np.array_equal(nan_g, nan_w), (label, "NaN positions differ", np.argwhere(nan_g != nan_w)[:5])
    ok = ~nan_w
    bad = np.argwhere(ok & (got != want))
    assert bad.size == 0, (label, [(tuple(i), hex(int(got[tuple(i)])), hex(int(want[tuple(i)])))
                                   for i in bad[:5]])


def case_list(dtype, M, N, K):
    """(label, A, B) with A, B torch tensors of `dtype` (exact: every value
    above is representable in both 16-bit formats where used)."""
    t = TDT[dtype]
    cases = []
    A, B = ties_operands(dtype, M, N, K)
    cases.append(("ties", torch.from_numpy(A).to(t), torch.from_numpy(B).to(t)))
    A, B = overflow_operands(dtype, M, N, 8)
    for x in (A, B):   # every value of the construction is exact in the format
        assert np.array_equal(torch.from_numpy(x).to(t).float().numpy(), x)
    cases.append(("overflow", torch.from_numpy(A).to(t), torch.from_numpy(B).to(t)))
    if dtype == "f16":
        A, B, Bsub, h = subnormal_operands(M, N, K)
        At = torch.from_numpy(A).to(t)
        # first half against B = 2^-12, second half (subnormal A) against B = 1
        cases.append(("subnormal_outputs", At[:h].contiguous(), torch.from_numpy(B).to(t)))
        cases.append(("subnormal_inputs", At[h:].contiguous(), torch.from_numpy(Bsub).to(t)))
        # subnormal B (2^-24) against the 0/1 rows of the ties case: c_i * 2^-24
        Aties, _ = ties_operands(dtype, M, N, K)
        cases.append(("subnormal_b", torch.from_numpy(Aties).to(t),
                      torch.from_numpy(np.full((K, N), 2.0 ** -24, dtype=np.float32)).to(t)))
    A, B = nan_operands(M, N, 64, 7)
    cases.append(("nan_inf", torch.from_numpy(A).to(t), torch.from_numpy(B).to(t)))
    return cases


def accepts(cid, a, b, c, M, N, K, dtype):
    h = dg.gemm_create()
    try:
        st = dg._lib.lib().gemm_run_config(h, a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K,
                                           CODE[dtype], cid, None)
        torch.cuda.synchronize()
        assert st in (0, 7), st
        return st == 0
    finally:
        dg.gemm_destroy(h)


def split_configs():
    """Tile configurations with a split-K form (16x16x32: A through
    registers, and the 128 x 128 / 64 x 128 ones with A direct to LDS)."""
    out = []
    for c in range(dg.gemm_config_count()):
        n = dg.gemm_config_info(c)["name"]
        if n.startswith("mfma16x16") and not n.endswith("_apair") and (
                not n.endswith("_adma") or "_128x128x" in n or "_64x128x" in n):
            out.append(c)
    return out


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(264, 136, 4104), (40, 4, 4104)])
def test_output_rounding_is_bit_exact_in_every_configuration(dtype, shape):
    M, N, K = shape
    for label, A, B in case_list(dtype, M, N, K):
        m, k = A.shape
        n = B.shape[1]
        want = expect_bits(A, B, dtype)
        a, b = A.cuda(), B.cuda()
        c = torch.empty((m, n), dtype=TDT[dtype], device="cuda")
        # gemm_run's own choice
        note(f"[rounding] {dtype} {label} {(m, n, k)} gemm_run")
        dg.gemm(a, b, out=c)
        torch.cuda.synchronize()
        assert_bits(c, want, dtype, (label, "gemm_run"))
        for cid in range(dg.gemm_config_count()):
            info = dg.gemm_config_info(cid)
            if not (info["dtype_mask"] >> CODE[dtype]) & 1:
                continue
            if not accepts(cid, a, b, c, m, n, k, dtype):
                continue
            note(f"[rounding] {dtype} {label} {(m, n, k)} config {cid} {info['name']}")
            c.fill_(0)
            dg.gemm(a, b, out=c, config=cid)
            torch.cuda.synchronize()
            assert_bits(c, want, dtype, (label, info["name"]))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_output_rounding_is_bit_exact_after_the_split_k_reduction(dtype):
    M, N, K = 264, 136, 4104
    for label, A, B in case_list(dtype, M, N, K):
        m, k = A.shape
        n = B.shape[1]
        want = expect_bits(A, B, dtype)
        a, b = A.cuda(), B.cuda()
        for cid in split_configs():
            c = torch.empty((m, n), dtype=TDT[dtype], device="cuda")
            if not accepts(cid, a, b, c, m, n, k, dtype):
                continue
            for s in (2, 3, 8):
                note(f"[rounding] {dtype} {label} split {s} config {cid}")
                c.fill_(0)
                dg.gemm(a, b, out=c, config=cid, splits=s)
                torch.cuda.synchronize()
                assert_bits(c, want, dtype, (label, cid, s))
