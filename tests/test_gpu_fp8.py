"""GPU parity of the 8-bit input path (E4M3 / E5M2 inputs, fp32 sums, bf16 C)
against the CPU oracle (oracle/fp8.py: decode from the format definitions,
fp64 product, one rounding to bf16).

Acceptance: ``oracle.tolerance`` with the bf16 output's rtol 1e-2 and the
floor 1e-3*sqrt(K)*max|A|*max|B| over the decoded inputs; integer inputs
(exact in both formats, exact sums) must match bit for bit.  The comparison
the pages ask for, FP8 against FP16, runs the same values through the fp16
path.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_run_amd as dg
from dense_gemm_run_amd.inputs import WORKLOADS, make_batched_operands, make_operands, workload_operands
from oracle import fp8, gemm64, tolerance
from test_gpu_parity import accepts

pytestmark = pytest.mark.gpu

FMT = {"fp8_e4m3": "e4m3", "fp8_e5m2": "e5m2"}
CODE = {"fp8_e4m3": 3, "fp8_e5m2": 4}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def fp8_configs():
    """The MFMA configurations of the 8-bit path (the generic one, which
    takes every dtype, is tested separately as config 0)."""
    return [c for c in range(1, dg.gemm_config_count())
            if (dg.gemm_config_info(c)["dtype_mask"] >> 3) & 1]


def check(A, B, dtype, C_gpu):
    fmt = FMT[dtype]
    ref, _ = fp8.reference_fp8(A, B, fmt)
    got = C_gpu.detach().to("cpu", torch.float64).numpy()
    assert got.shape == ref.shape
    K = A.shape[-1]
    rep = tolerance.compare(got, ref, "bf16", K, fp8.decoded_max_abs(A, fmt), fp8.decoded_max_abs(B, fmt))
    assert rep["ok"], rep
    return rep


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "fp8_e5m2"])
@pytest.mark.parametrize("shape", [(520, 784, 272), (256, 256, 64), (1, 16, 16), (300, 1024, 48),
                                   (777, 528, 1040), (127, 255, 65), (64, 48, 0)])
def test_fp8_every_configuration(dtype, shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, dtype, "normal", 40 + M)
    Ai, Bi = make_operands(M, N, K, dtype, "integers", 41 + M)
    a, b, ai, bi = A.cuda(), B.cuda(), Ai.cuda(), Bi.cuda()
    ref_i, _ = fp8.reference_fp8(Ai, Bi, FMT[dtype])
    ran = []
    for cid in [0] + fp8_configs():
        if not accepts(cid, a, b, M, N, K):
            continue
        note(f"[fp8] config {cid} {dg.gemm_config_info(cid)['name']} {dtype} {shape}")
        c = dg.gemm(a, b, config=cid)
        torch.cuda.synchronize()
        assert c.dtype == torch.bfloat16
        check(A, B, dtype, c)
        ci = dg.gemm(ai, bi, config=cid)
        torch.cuda.synchronize()
        assert np.array_equal(ci.to("cpu", torch.float64).numpy(), ref_i)
        ran.append(cid)
    assert 0 in ran
    if K % 16 == 0 and N % 16 == 0 and K > 0:
        assert len(ran) == 1 + len(fp8_configs()), ran   # the MFMA kernels took the aligned shapes


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "fp8_e5m2"])
def test_fp8_batched(dtype):
    batch, M, N, K = 3, 300, 528, 208
    A, B = make_batched_operands(batch, M, N, K, dtype, "normal", 50)
    a, b = A.cuda(), B.cuda()
    for cid in [None, 0]:
        note(f"[fp8] batched config {cid} {dtype}")
        c = dg.gemm_batched(a, b, config=cid)
        torch.cuda.synchronize()
        check(A, B, dtype, c)
    # B shared by every product
    Bs = B[0].contiguous()
    c = dg.gemm_batched(a, Bs.cuda())
    torch.cuda.synchronize()
    check(A, Bs, dtype, c)


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "fp8_e5m2"])
def test_fp8_against_fp16(dtype):
    """The same input values through the fp16 path: every 8-bit value is an
    fp16 value, both paths form exact products and fp32 sums, so the two
    results differ only by their output roundings (and the sum order)."""
    M, N, K = 1024, 1024, 1024
    A, B = make_operands(M, N, K, dtype, "normal", 60)
    a, b = A.cuda(), B.cuda()
    a16, b16 = a.to(torch.float16), b.to(torch.float16)
    # the widening to fp16 is exact: check it against the oracle's decode
    assert np.array_equal(a16.cpu().to(torch.float64).numpy(), fp8.decode(fp8._bits(A), FMT[dtype]))
    c8 = dg.gemm(a, b)
    c16 = dg.gemm(a16, b16)
    torch.cuda.synchronize()
    note(f"[fp8] vs fp16 {dtype}: configs {dg.gemm_select_config(a.data_ptr(), b.data_ptr(), c8.data_ptr(), M, N, K, CODE[dtype])}")
    g8 = c8.to("cpu", torch.float64).numpy()
    g16 = c16.to("cpu", torch.float64).numpy()
    amax, bmax = fp8.decoded_max_abs(A, FMT[dtype]), fp8.decoded_max_abs(B, FMT[dtype])
    rep = tolerance.compare(g8, g16, "bf16", K, amax, bmax)
    assert rep["ok"], rep
    # and each against the oracle
    check(A, B, dtype, c8)


def test_fp8_nan_and_infinity_propagate():
    M, N, K = 256, 256, 128
    for dtype, special in (("fp8_e4m3", [0x7F]), ("fp8_e5m2", [0x7C, 0x7D])):
        A, B = make_operands(M, N, K, dtype, "normal", 70)
        Ab = A.view(torch.uint8).clone()
        for i, code in enumerate(special):
            Ab[5 + i, 7] = code                  # row 5 (+i) holds a NaN or infinity
        A = Ab.view(A.dtype)
        for cid in [0] + fp8_configs():
            note(f"[fp8] specials {dtype} config {cid}")
            c = dg.gemm(A.cuda(), B.cuda(), config=cid)
            torch.cuda.synchronize()
            check(A, B, dtype, c)


def test_fp8_errors():
    a = torch.zeros((64, 64), dtype=torch.float8_e4m3fn, device="cuda")
    b5 = torch.zeros((64, 64), dtype=torch.float8_e5m2, device="cuda")
    with pytest.raises(TypeError):
        dg.gemm(a, b5)                          # mixed formats
    with pytest.raises(ValueError):
        dg.gemm(a, a, out=torch.empty((64, 64), dtype=torch.float8_e4m3fn, device="cuda"))
    # the fast kernels refuse rows that are not whole 16-byte pieces
    a2 = torch.zeros((64, 72), dtype=torch.float8_e4m3fn, device="cuda")
    b2 = torch.zeros((72, 64), dtype=torch.float8_e4m3fn, device="cuda")
    for cid in fp8_configs():
        with pytest.raises(dg.GemmError) as e:
            dg.gemm(a2, b2, config=cid)
        assert e.value.name == "GEMM_ERR_CONFIG_MISMATCH"
    # ... and an fp16 configuration refuses 8-bit inputs
    with pytest.raises(dg.GemmError):
        dg.gemm(a, a, config=6)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["fp8_e4m3_4096x4096x4096", "fp8_e5m2_4096x4096x4096",
                                  "fp8_e4m3_8192x8192x8192"])
def test_fp8_workloads_sampled(name):
    """The 8-bit workloads at full size in the configuration gemm_run picks
    (the one bench.py times): whole rows, whole columns and random points."""
    w = WORKLOADS[name]
    fmt = FMT[w.dtype]
    note(f"[fp8] full-size {name}")
    A, B = workload_operands(name)
    a, b = A.cuda(), B.cuda()
    c = dg.gemm(a, b)
    torch.cuda.synchronize()
    note(f"  config {dg.gemm_select_config(a.data_ptr(), b.data_ptr(), c.data_ptr(), w.M, w.N, w.K, CODE[w.dtype])}")
    assert not torch.isnan(c).any()
    rng = np.random.default_rng(w.seed)
    rows = [0, w.M - 1, int(rng.integers(0, w.M))]
    cols = [0, w.N - 1, int(rng.integers(0, w.N))]
    pr = np.concatenate([np.full(w.N, r) for r in rows] + [np.arange(w.M) for _ in cols]
                        + [rng.integers(0, w.M, 100000)])
    pc = np.concatenate([np.arange(w.N) for _ in rows] + [np.full(w.M, c_) for c_ in cols]
                        + [rng.integers(0, w.N, 100000)])
    A64 = fp8.decode(fp8._bits(A), fmt)
    B64 = fp8.decode(fp8._bits(B), fmt)
    exact_vals = gemm64.gemm_points_f64(A64, B64, pr, pc)
    ref = gemm64.bits_to_f64(gemm64.round_to_bits(exact_vals, "bf16"), "bf16")
    got = c[torch.from_numpy(pr).cuda(), torch.from_numpy(pc).cuda()].to("cpu", torch.float64).numpy()
    rep = tolerance.compare(got, ref, "bf16", w.K, float(np.abs(A64).max()), float(np.abs(B64).max()))
    note(f"  {rep}")
    assert rep["ok"], rep


@pytest.mark.parametrize("shape", [(2048, 2048, 2048), (256, 14336, 4096), (64, 14336, 4096),
                                   (1000, 3008, 1040)])
def test_fp8_mid_sizes_in_the_selected_configuration(shape):
    """Shapes with fewer than 128 tiles of 256 x 256 (the 128 x 128 tiles, or
    64 x 128 while those fit one wave), in the configuration gemm_run picks,
    on whole rows, whole columns and random points."""
    M, N, K = shape
    A, B = make_operands(M, N, K, "fp8_e4m3", "normal", 700 + M)
    a, b = A.cuda(), B.cuda()
    c = dg.gemm(a, b)
    torch.cuda.synchronize()
    cid = dg.gemm_select_config(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, 3)
    note(f"[fp8] mid size {shape} config {dg.gemm_config_info(cid)['name']}")
    assert dg.gemm_config_info(cid)["name"].startswith(("fp8_128x128", "fp8_64x128"))
    rng = np.random.default_rng(M)
    rows = [0, M - 1, int(rng.integers(0, M))]
    cols = [0, N - 1, int(rng.integers(0, N))]
    pr = np.concatenate([np.full(N, r) for r in rows] + [np.arange(M) for _ in cols]
                        + [rng.integers(0, M, 20000)])
    pc = np.concatenate([np.arange(N) for _ in rows] + [np.full(M, c_) for c_ in cols]
                        + [rng.integers(0, N, 20000)])
    A64 = fp8.decode(fp8._bits(A), "e4m3")
    B64 = fp8.decode(fp8._bits(B), "e4m3")
    ref = gemm64.bits_to_f64(gemm64.round_to_bits(gemm64.gemm_points_f64(A64, B64, pr, pc), "bf16"), "bf16")
    got = c[torch.from_numpy(pr).cuda(), torch.from_numpy(pc).cuda()].to("cpu", torch.float64).numpy()
    rep = tolerance.compare(got, ref, "bf16", K, float(np.abs(A64).max()), float(np.abs(B64).max()))
    assert rep["ok"], rep


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "fp8_e5m2"])
@pytest.mark.parametrize("shape", [(127, 255, 65), (264, 400, 144), (520, 784, 272), (1, 16, 16)])
def test_fp8_masked_store_leaves_guards_untouched(dtype, shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, dtype, "normal", 6)
    guard = 4096
    buf = torch.full((guard + M * N + guard,), 1234.0, dtype=torch.bfloat16, device="cuda")
    pattern = buf.clone()
    out = buf[guard:guard + M * N].view(M, N)
    for cid in [None] + fp8_configs():
        if cid is not None and not accepts(cid, A.cuda(), B.cuda(), M, N, K):
            continue
        note(f"[fp8] guards {dtype} {shape} config {cid}")
        dg.gemm(A.cuda(), B.cuda(), out=out, config=cid)
        torch.cuda.synchronize()
        assert torch.equal(buf[:guard], pattern[:guard])
        assert torch.equal(buf[guard + M * N:], pattern[guard + M * N:])
        check(A, B, dtype, out)


def test_fp8_unaligned_pointers_take_the_generic_kernel():
    M, N, K = 200, 144, 80
    A0, B0 = make_operands(M + 1, N + 1, K + 1, "fp8_e4m3", "normal", 9)
    a = A0.reshape(-1)[: 1 + M * K].cuda()[1:].view(M, K)
    b = B0.reshape(-1)[: 1 + K * N].cuda()[1:].view(K, N)
    c = dg.gemm(a, b)
    torch.cuda.synchronize()
    assert dg.gemm_select_config(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, 3) == 0
    check(a.cpu(), b.cpu(), "fp8_e4m3", c)
