"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every comparison is element by element on the same seeded inputs, with the
acceptance rule of ``oracle.tolerance`` (rtol 2e-3 fp16 / 1e-2 bf16 / 1e-5
fp32, floor 1e-3·sqrt(K)·max|A|·max|B|).  Small and mid shapes and the
4096^3 headline product are compared whole; the 8192-row workloads are
compared on sampled outputs (whole rows and columns plus 100,000 random
points), each computed by the oracle one by one.
"""
import math
import sys

import numpy as np
import pytest
import torch

import dense_gemm_run_amd as dg
from dense_gemm_run_amd.inputs import DTYPES, WORKLOADS, make_operands, workload_operands
from oracle import gemm64, tolerance

pytestmark = pytest.mark.gpu

DT_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(A, B, config=None, out=None):
    a = A.cuda()
    b = B.cuda()
    c = dg.gemm(a, b, out=out, config=config)
    torch.cuda.synchronize()
    return c


def accepts(cid, a, b, M, N, K, batch=1):
    """Whether configuration cid runs these arguments (a forced configuration
    that does not, e.g. a matrix-vector one for many columns, is refused with
    GEMM_ERR_CONFIG_MISMATCH before any launch)."""
    h = dg.gemm_create()
    try:
        # C of the output type (bf16 for 8-bit inputs), M*N elements per matrix
        c = torch.empty((batch, M, N) if batch > 1 else (M, N), dtype=dg.out_dtype(a.dtype),
                        device=a.device)
        st = dg._lib.lib().gemm_run_batched_config(h, a.data_ptr(), b.data_ptr(), c.data_ptr(),
                                                  batch, M, N, K, M * K if a.ndim == 3 else 0,
                                                  K * N if b.ndim == 3 else 0, M * N,
                                                  dg.dtype_code(a.dtype), cid, None)
        torch.cuda.synchronize()
        assert st in (0, 7), st        # ran, or refused as a mismatch
        return st == 0
    finally:
        dg.gemm_destroy(h)


def check_full(A, B, dtype, C_gpu, use_floor=True):
    K = A.shape[1]
    ref, _ = gemm64.reference(A, B, dtype)
    got = C_gpu.detach().to("cpu", torch.float64).numpy()
    amax = float(A.abs().max()) if A.numel() else 0.0
    bmax = float(B.abs().max()) if B.numel() else 0.0
    rep = tolerance.compare(got, ref, dtype, K, amax, bmax, use_floor=use_floor)
    assert rep["ok"], rep
    return rep


def sampled_check(A, B, dtype, C_gpu, n_points=100000, seed=0):
    M, K = A.shape
    N = B.shape[1]
    rng = np.random.default_rng(seed)
    rows = [0, M - 1, int(rng.integers(0, M))]
    cols = [0, N - 1, int(rng.integers(0, N))]
    pr = [np.full(N, r) for r in rows] + [np.arange(M) for _ in cols] + [rng.integers(0, M, n_points)]
    pc = [np.arange(N) for _ in rows] + [np.full(M, c) for c in cols] + [rng.integers(0, N, n_points)]
    pr = np.concatenate(pr)
    pc = np.concatenate(pc)
    A64 = A.to(torch.float64).numpy()
    B64 = B.to(torch.float64).numpy()
    exact_vals = gemm64.gemm_points_f64(A64, B64, pr, pc)
    ref = gemm64.bits_to_f64(gemm64.round_to_bits(exact_vals, dtype), dtype)
    got = C_gpu[torch.from_numpy(pr).cuda(), torch.from_numpy(pc).cuda()].to("cpu", torch.float64).numpy()
    rep = tolerance.compare(got, ref, dtype, K, float(A.abs().max()), float(B.abs().max()))
    assert rep["ok"], rep
    return rep


# ---------------------------------------------------------------- small workloads, whole
@pytest.mark.parametrize("name", ["f32_64x64x64", "f16_127x255x65"])
def test_small_workloads_whole(name):
    note(f"[parity] workload {name}")
    A, B = workload_operands(name)
    w = WORKLOADS[name]
    C = run_gpu(A, B)
    rep = check_full(A, B, w.dtype, C)
    note(f"  {rep}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 300, 17), (300, 1, 33), (7, 9, 1),
                                   (64, 64, 64), (65, 63, 31), (129, 257, 100),
                                   (300, 500, 200), (513, 257, 129)])
def test_mid_shapes_whole(dtype, shape):
    M, N, K = shape
    note(f"[parity] {dtype} {shape}")
    A, B = make_operands(M, N, K, dtype, "normal", 1000 + M + N + K)
    C = run_gpu(A, B)
    check_full(A, B, dtype, C)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (1000, 1000, 1000), (768, 1280, 520),
                                   (2048, 512, 4096)])
def test_larger_shapes_whole(dtype, shape):
    M, N, K = shape
    note(f"[parity] {dtype} {shape}")
    A, B = make_operands(M, N, K, dtype, "normal", 7 + M + N + K)
    C = run_gpu(A, B)
    check_full(A, B, dtype, C)


# ---------------------------------------------------------------- exactness and edges
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(5, 7, 5), (127, 255, 65), (256, 256, 512), (300, 200, 1000)])
def test_integer_inputs_bit_exact(dtype, shape):
    # integers in [-4, 4]: every product and partial sum is an exact integer
    # below 2^24, so any summation order gives the oracle's value exactly
    M, N, K = shape
    note(f"[parity] integers {dtype} {shape}")
    A, B = make_operands(M, N, K, dtype, "integers", 77)
    C = run_gpu(A, B)
    ref, _ = gemm64.reference(A, B, dtype)
    assert np.array_equal(C.to("cpu", torch.float64).numpy(), ref)


def test_worked_example_on_gpu():
    for dt in ("f32", "f16", "bf16"):
        A = torch.tensor([[1, 2, 3], [4, 5, 6]], dtype=DTYPES[dt])
        B = torch.tensor([[7, 8], [9, 10], [11, 12]], dtype=DTYPES[dt])
        C = run_gpu(A, B)
        assert C.cpu().double().tolist() == [[58, 64], [139, 154]]


def test_fp32_keeps_full_input_precision():
    # values with all 24 significand bits in use: a reduced-precision input
    # mode would be off by >1e-4 relative; the fp32 path must be within 1e-5
    # relative with no absolute floor
    # (the ragged shape runs the generic kernel, 64^3 and 256 x 260 x 1024 the
    # fp32 MFMA kernel)
    for shape in [(64, 64, 64), (130, 70, 257), (256, 260, 1024)]:
        A, B = make_operands(shape[0], shape[1], shape[2], "f32", "fp32_fine", 21)
        C = run_gpu(A, B)
        check_full(A, B, "f32", C, use_floor=False)


def test_k_zero_gives_zeros_and_empty_outputs_write_nothing():
    for dt in ("f32", "f16", "bf16"):
        A = torch.empty((5, 0), dtype=DTYPES[dt], device="cuda")
        B = torch.empty((0, 7), dtype=DTYPES[dt], device="cuda")
        out = torch.full((5, 7), float("nan"), dtype=DTYPES[dt], device="cuda")
        dg.gemm(A, B, out=out)
        torch.cuda.synchronize()
        assert (out == 0).all() and not torch.signbit(out).any()
    # M = 0 and N = 0: a guard-filled buffer stays untouched
    g = torch.full((64,), 7.0, dtype=torch.float16, device="cuda")
    dg.gemm(torch.empty((0, 4), dtype=torch.float16, device="cuda"),
            torch.ones((4, 8), dtype=torch.float16, device="cuda"), out=g[:0].view(0, 8))
    dg.gemm(torch.ones((4, 4), dtype=torch.float16, device="cuda"),
            torch.empty((4, 0), dtype=torch.float16, device="cuda"), out=g[:0].view(4, 0))
    torch.cuda.synchronize()
    assert (g == 7.0).all()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(127, 255, 65), (1, 1, 1), (65, 129, 8), (300, 260, 64),
                                   (264, 392, 136), (520, 776, 264)])
def test_masked_store_leaves_guards_untouched(dtype, shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, dtype, "normal", 5)
    guard = 4096
    buf = torch.empty(guard + M * N + guard, dtype=DTYPES[dtype], device="cuda")
    pattern = torch.full_like(buf, 1234.0)
    buf.copy_(pattern)
    out = buf[guard:guard + M * N].view(M, N)
    dg.gemm(A.cuda(), B.cuda(), out=out)
    torch.cuda.synchronize()
    assert torch.equal(buf[:guard], pattern[:guard])
    assert torch.equal(buf[guard + M * N:], pattern[guard + M * N:])
    check_full(A, B, dtype, out)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_unaligned_pointers(dtype):
    # views that start 1 element into a buffer: only the kernel choice changes
    M, N, K = 200, 136, 72
    A0, B0 = make_operands(M + 1, N + 1, K + 1, dtype, "normal", 8)
    a_buf = A0.reshape(-1)[: 1 + M * K].cuda()
    b_buf = B0.reshape(-1)[: 1 + K * N].cuda()
    a = a_buf[1:].view(M, K)
    b = b_buf[1:].view(K, N)
    c_buf = torch.empty(1 + M * N, dtype=DTYPES[dtype], device="cuda")
    c = c_buf[1:].view(M, N)
    dg.gemm(a, b, out=c)
    torch.cuda.synchronize()
    check_full(a.cpu(), b.cpu(), dtype, c)


def test_repeat_runs_are_bitwise_identical():
    A, B = make_operands(1000, 1000, 1000, "bf16", "normal", 3)
    a, b = A.cuda(), B.cuda()
    c1 = dg.gemm(a, b)
    c2 = dg.gemm(a, b)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("shape", [(520, 776, 264), (256, 256, 64), (8, 8, 8), (1, 8, 4096),
                                   (777, 8, 72), (300, 1000, 8)])
def test_every_configuration_that_accepts_the_arguments(dtype, shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, dtype, "normal", 4 + M)
    a, b = A.cuda(), B.cuda()
    for cid in range(dg.gemm_config_count()):
        info = dg.gemm_config_info(cid)
        if not (info["dtype_mask"] >> DT_CODE[dtype]) & 1:
            continue
        if not accepts(cid, a, b, M, N, K):
            continue
        note(f"[parity] config {cid} {info['name']} {dtype} {shape}")
        c = dg.gemm(a, b, config=cid)
        torch.cuda.synchronize()
        check_full(A, B, dtype, c)
        # the same configuration on integer inputs must be bit-exact
        Ai, Bi = make_operands(M, N, K, dtype, "integers", 5 + M)
        ci = dg.gemm(Ai.cuda(), Bi.cuda(), config=cid)
        torch.cuda.synchronize()
        ref, _ = gemm64.reference(Ai, Bi, dtype)
        assert np.array_equal(ci.to("cpu", torch.float64).numpy(), ref)


def test_api_errors_on_gpu():
    h = dg.gemm_create()
    try:
        a = torch.ones((4, 4), dtype=torch.float16, device="cuda")
        with pytest.raises(dg.GemmError) as e:
            dg.gemm_run(h, a.data_ptr(), a.data_ptr(), a.data_ptr(), 4, 4, 4, 1, None)
        assert e.value.name == "GEMM_ERR_ALIASING"
        with pytest.raises(ValueError):
            dg.gemm(a, torch.ones((5, 4), dtype=torch.float16, device="cuda"))
        with pytest.raises(ValueError):
            dg.gemm(a.t(), a)     # non-contiguous input: rejected, not copied
        with pytest.raises(TypeError):
            dg.gemm(a, a.float())
    finally:
        dg.gemm_destroy(h)


# ---------------------------------------------------------------- full-size workloads
def test_headline_workload_whole():
    """The square fp16 4096^3 product that bench.py times, in the
    configuration gemm_run picks, compared with the oracle on every one of
    its 16.8 M outputs (the correctness check of notebook "Triton tiled
    matmul", section "Correctness check", compares the whole output too)."""
    name = "f16_4096x4096x4096"
    w = WORKLOADS[name]
    note(f"[parity] full-size {name}, whole output")
    A, B = workload_operands(name)
    a, b = A.cuda(), B.cuda()
    C = torch.empty((w.M, w.N), dtype=a.dtype, device="cuda")
    cid = dg.gemm_select_config(a.data_ptr(), b.data_ptr(), C.data_ptr(), w.M, w.N, w.K,
                                DT_CODE[w.dtype])
    note(f"  config {cid} {dg.gemm_config_info(cid)['name']}")
    dg.gemm(a, b, out=C)
    torch.cuda.synchronize()
    rep = check_full(A, B, w.dtype, C)
    note(f"  {rep}")


def test_fp32_workload_sampled():
    """The square fp32 4096^3 product in the configuration gemm_run picks
    (the fp32 MFMA kernel): whole rows and columns and 100,000 random points,
    with fp32's 1e-5 relative tolerance."""
    name = "f32_4096x4096x4096"
    w = WORKLOADS[name]
    A, B = workload_operands(name)
    a, b = A.cuda(), B.cuda()
    C = torch.empty((w.M, w.N), dtype=a.dtype, device="cuda")
    cid = dg.gemm_select_config(a.data_ptr(), b.data_ptr(), C.data_ptr(), w.M, w.N, w.K, DT_CODE["f32"])
    note(f"[parity] full-size {name} config {cid} {dg.gemm_config_info(cid)['name']}")
    assert dg.gemm_config_info(cid)["name"] == "fp32_128x128x32"
    dg.gemm(a, b, out=C)
    torch.cuda.synchronize()
    rep = sampled_check(A, B, "f32", C, seed=w.seed)
    note(f"  {rep}")


FULL = ["bf16_8192x8192x8192", "bf16_prefill_qkv_8192x12288x4096",
        "bf16_prefill_out_8192x4096x4096", "bf16_prefill_up_8192x14336x4096",
        "bf16_prefill_down_8192x4096x14336"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workloads_sampled(name):
    """The 8192-row workloads: whole rows 0, M-1 and one random row, whole
    columns 0, N-1 and one random column, and 100,000 random points, each an
    fp64 dot product of the oracle."""
    w = WORKLOADS[name]
    note(f"[parity] full-size {name}")
    A, B = workload_operands(name)
    a, b = A.cuda(), B.cuda()
    C = torch.empty((w.M, w.N), dtype=a.dtype, device="cuda")
    cid = dg.gemm_select_config(a.data_ptr(), b.data_ptr(), C.data_ptr(), w.M, w.N, w.K,
                                DT_CODE[w.dtype])
    note(f"  config {cid} {dg.gemm_config_info(cid)['name']}")
    dg.gemm(a, b, out=C)
    torch.cuda.synchronize()
    assert not torch.isnan(C).any()
    rep = sampled_check(A, B, w.dtype, C, seed=w.seed)
    note(f"  {rep}")


@pytest.mark.parametrize("shape", [(3072, 3072, 3072), (3000, 3064, 1000), (6144, 6144, 1024)])
def test_partial_wave_shapes_in_the_192_row_tiles(shape):
    """Shapes whose 256 x 256 tiles leave a partial last wave run 192 x 256
    tiles (ragged in M and N for the second shape); sampled like the
    full-size workloads."""
    M, N, K = shape
    note(f"[parity] 192-row tiles {shape}")
    A, B = make_operands(M, N, K, "bf16", "normal", 40 + M)
    a, b = A.cuda(), B.cuda()
    C = torch.empty((M, N), dtype=a.dtype, device="cuda")
    cid = dg.gemm_select_config(a.data_ptr(), b.data_ptr(), C.data_ptr(), M, N, K, DT_CODE["bf16"])
    assert dg.gemm_config_info(cid)["name"].startswith("mfma16x16_192x256x32"), cid
    dg.gemm(a, b, out=C)
    torch.cuda.synchronize()
    rep = sampled_check(A, B, "bf16", C, seed=M)
    note(f"  {rep}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_short_k_kernel_walks_several_tiles_per_workgroup(dtype):
    """The persistent short-K kernel (config 48) on a ragged product with more
    128 x 128 tiles (24 x 23 = 552) than its resident workgroups (two per CU):
    workgroups walk several tiles, loading the next one during the current
    one's stores; K = 104 is zero-padded to the staged 128.  Whole output
    against the oracle, and bit-exact on integer inputs."""
    M, N, K = 3000, 2904, 104
    cid = next(i for i in range(dg.gemm_config_count()) if dg.gemm_config_info(i)["name"] == "shortk_128x128x128")
    A, B = make_operands(M, N, K, dtype, "normal", 48)
    note(f"[parity] short-K persistent {dtype} {(M, N, K)}")
    c = dg.gemm(A.cuda(), B.cuda(), config=cid)
    torch.cuda.synchronize()
    check_full(A, B, dtype, c)
    Ai, Bi = make_operands(M, N, K, dtype, "integers", 49)
    ci = dg.gemm(Ai.cuda(), Bi.cuda(), config=cid)
    torch.cuda.synchronize()
    ref, _ = gemm64.reference(Ai, Bi, dtype)
    assert np.array_equal(ci.to("cpu", torch.float64).numpy(), ref)


def test_clocked_run_matches_gemm_run_and_reads_a_plausible_clock():
    """gemm_run_clocked computes gemm_run's product bit for bit, and in the
    MFMA tile kernels its clock samples give a shader clock between 0.5 and
    2.5 GHz; a kernel without samples (the generic one) leaves clk as it
    was."""
    h = dg.gemm_create()
    try:
        stream = torch.cuda.current_stream().cuda_stream
        for dtype, (M, N, K) in [("f16", (4096, 4096, 4096)), ("bf16", (1000, 1000, 1000)),
                                 ("fp8_e4m3", (2048, 2048, 2048)), ("f32", (1024, 1024, 1024))]:
            A, B = make_operands(M, N, K, dtype, "normal", 77)
            a, b = A.cuda(), B.cuda()
            c1 = dg.gemm(a, b)
            c2 = torch.empty_like(c1)
            clk = torch.zeros(4, dtype=torch.int64, device="cuda")
            dg.gemm_run_clocked(h, a.data_ptr(), b.data_ptr(), c2.data_ptr(), M, N, K, dg.dtype_code(a.dtype),
                                clk.data_ptr(), stream)
            torch.cuda.synchronize()
            assert torch.equal(c1.view(torch.int8), c2.view(torch.int8)), dtype
            c0, cc1, r0, r1 = clk.tolist()
            assert cc1 > c0 > 0 and r1 > r0 > 0, (dtype, clk.tolist())
            mhz = 100.0 * (cc1 - c0) / (r1 - r0)
            note(f"[clock] {dtype} {(M, N, K)}: {mhz:.0f} MHz over {(r1 - r0) / 100:.1f} us")
            assert 500 < mhz < 2500, (dtype, mhz)
        # the generic kernel takes no samples
        A, B = make_operands(127, 255, 65, "f16", "normal", 78)
        a, b = A.cuda(), B.cuda()
        c = torch.empty((127, 255), dtype=torch.float16, device="cuda")
        clk = torch.zeros(4, dtype=torch.int64, device="cuda")
        dg.gemm_run_clocked(h, a.data_ptr(), b.data_ptr(), c.data_ptr(), 127, 255, 65, 1, clk.data_ptr(), stream)
        torch.cuda.synchronize()
        assert clk.tolist() == [0, 0, 0, 0]
        check_full(A, B, "f16", c)
    finally:
        dg.gemm_destroy(h)
