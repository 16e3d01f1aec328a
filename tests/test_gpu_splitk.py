"""GPU parity of split K (gemm_run_ws, gemm_run_ws_config) against the CPU oracle.

Each split walks its own range of K-steps and writes unrounded fp32 sums to
a slice of the caller's workspace; a second kernel adds the slices in split
order and rounds once.  The shapes below are ragged in M, N and K, so splits
end mid-tile, the last split is shorter than the others, and split counts
that do not divide the K-steps are lowered (every split keeps K-steps).
Same acceptance rule as the other parity tests; integer inputs bit-exact.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_run_amd as dg
from dense_gemm_run_amd import _lib
from dense_gemm_run_amd.inputs import make_operands
from oracle import gemm64
from test_gpu_parity import accepts, check_full, sampled_check

pytestmark = pytest.mark.gpu

DT_CODE = {"f16": 1, "bf16": 2}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def splits_k(name):
    """Whether a tile configuration has a split form: all with A through
    registers, and the 128 x 128 and 64 x 128 ones with A direct to LDS."""
    if name.endswith(("_apair", "_k128")):   # one pass only
        return False
    return not name.endswith("_adma") or "_128x128x" in name or "_64x128x" in name


def tile_configs():
    """The 16x16x32 tile configurations that split K."""
    return [c for c in range(dg.gemm_config_count())
            if dg.gemm_config_info(c)["name"].startswith("mfma16x16")
            and splits_k(dg.gemm_config_info(c)["name"])]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(300, 520, 1000), (128, 256, 4104), (64, 136, 2056), (257, 264, 520)])
def test_every_tile_configuration_at_every_split_count(dtype, shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, dtype, "normal", 1100 + M)
    Ai, Bi = make_operands(M, N, K, dtype, "integers", 1101 + M)
    a, b, ai, bi = A.cuda(), B.cuda(), Ai.cuda(), Bi.cuda()
    ref_i, _ = gemm64.reference(Ai, Bi, dtype)
    for cid in tile_configs():
        if not accepts(cid, a, b, M, N, K):
            continue
        for s in (2, 3, 7, 16):
            note(f"[splitk] config {cid} {dg.gemm_config_info(cid)['name']} splits {s} {dtype} {shape}")
            c = dg.gemm(a, b, config=cid, splits=s)
            torch.cuda.synchronize()
            check_full(A, B, dtype, c)
            ci = dg.gemm(ai, bi, config=cid, splits=s)
            torch.cuda.synchronize()
            assert np.array_equal(ci.to("cpu", torch.float64).numpy(), ref_i)


@pytest.mark.parametrize("shape", [(256, 4096, 4096), (64, 14336, 4096), (128, 1024, 8192)])
def test_selected_split_shapes_sampled(shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, "bf16", "prefill", 1200 + M)
    a, b = A.cuda(), B.cuda()
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    need = dg.gemm_workspace_size(M, N, K, DT_CODE["bf16"])
    cid, s = dg.gemm_select_config_ws(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, 2, need)
    note(f"[splitk] selected {dg.gemm_config_info(cid)['name']} x {s} for {shape}")
    assert s > 1 and need == s * M * N * 4
    dg.gemm(a, b, out=c, split_k=True)
    torch.cuda.synchronize()
    rep = sampled_check(A, B, "bf16", c, seed=M)
    note(f"  {rep}")


def test_configurations_without_a_split_form_refuse_splits():
    M, N, K = 256, 1024, 4096
    A, B = make_operands(M, N, K, "bf16", "normal", 1350)
    a, b = A.cuda(), B.cuda()
    for cid in range(dg.gemm_config_count()):
        name = dg.gemm_config_info(cid)["name"]
        if name.startswith("mfma16x16") and not splits_k(name):
            with pytest.raises(dg.GemmError) as e:
                dg.gemm(a, b, config=cid, splits=4)
            assert e.value.name == "GEMM_ERR_CONFIG_MISMATCH"


def test_split_results_are_bitwise_repeatable():
    M, N, K = 256, 1024, 4096
    A, B = make_operands(M, N, K, "bf16", "normal", 1300)
    a, b = A.cuda(), B.cuda()
    c1 = dg.gemm(a, b, config=12, splits=8)
    c2 = dg.gemm(a, b, config=12, splits=8)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_guards_around_c_and_the_workspace_are_untouched():
    M, N, K, s = 200, 264, 3000, 5
    A, B = make_operands(M, N, K, "f16", "normal", 1400)
    a, b = A.cuda(), B.cuda()
    guard = 4096
    cbuf = torch.full((guard + M * N + guard,), 77.0, dtype=torch.float16, device="cuda")
    cpat = cbuf.clone()
    c = cbuf[guard:guard + M * N].view(M, N)
    need = s * M * N * 4
    wbuf = torch.full((guard + need + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    wpat = wbuf.clone()
    h = dg.gemm_create()
    try:
        ws = wbuf[guard:guard + need]
        note(f"[splitk] guards {M}x{N}x{K} splits {s}")
        dg.gemm_run_ws_config(h, a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, 1, 12, s,
                              ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        dg.gemm_destroy(h)
    assert torch.equal(cbuf[:guard], cpat[:guard]) and torch.equal(cbuf[guard + M * N:], cpat[guard + M * N:])
    assert torch.equal(wbuf[:guard], wpat[:guard]) and torch.equal(wbuf[guard + need:], wpat[guard + need:])
    check_full(A, B, "f16", c)


def test_a_short_workspace_runs_the_single_pass_schedule():
    M, N, K = 256, 4096, 4096
    A, B = make_operands(M, N, K, "bf16", "normal", 1500)
    a, b = A.cuda(), B.cuda()
    need = dg.gemm_workspace_size(M, N, K, 2)
    assert need > 0
    work = torch.empty(need, dtype=torch.uint8, device="cuda")
    c_ws = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    c_short = torch.empty_like(c_ws)
    c_plain = torch.empty_like(c_ws)
    h = dg.gemm_create()
    st = torch.cuda.current_stream().cuda_stream
    try:
        dg.gemm_run_ws(h, a.data_ptr(), b.data_ptr(), c_ws.data_ptr(), M, N, K, 2, work.data_ptr(), need, st)
        dg.gemm_run_ws(h, a.data_ptr(), b.data_ptr(), c_short.data_ptr(), M, N, K, 2, work.data_ptr(),
                       need - 16, st)
        dg.gemm_run(h, a.data_ptr(), b.data_ptr(), c_plain.data_ptr(), M, N, K, 2, st)
        torch.cuda.synchronize()
    finally:
        dg.gemm_destroy(h)
    assert torch.equal(c_short.view(torch.int16), c_plain.view(torch.int16))
    sampled_check(A, B, "bf16", c_ws, seed=1)
    sampled_check(A, B, "bf16", c_short, seed=2)


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "fp8_e5m2"])
@pytest.mark.parametrize("shape", [(300, 528, 1040), (64, 272, 4112), (130, 256, 2064)])
def test_8bit_tile_configurations_at_every_split_count(dtype, shape):
    from test_gpu_fp8 import check as check8
    M, N, K = shape
    A, B = make_operands(M, N, K, dtype, "normal", 1600 + M)
    a, b = A.cuda(), B.cuda()
    for cid in range(dg.gemm_config_count()):
        info = dg.gemm_config_info(cid)
        if (not info["name"].startswith("fp8_") or not splits_k(info["name"])
                or not accepts(cid, a, b, M, N, K)):
            continue
        for s in (2, 3, 7, 16):
            note(f"[splitk] config {cid} {info['name']} splits {s} {dtype} {shape}")
            c = dg.gemm(a, b, config=cid, splits=s)
            torch.cuda.synchronize()
            check8(A, B, dtype, c)


@pytest.mark.parametrize("shape", [(64, 4096, 14336), (16, 14336, 4096), (100, 4096, 4096)])
def test_selected_8bit_split_shapes_sampled(shape):
    from oracle import fp8, tolerance
    M, N, K = shape
    A, B = make_operands(M, N, K, "fp8_e4m3", "normal", 1700 + M)
    a, b = A.cuda(), B.cuda()
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    need = dg.gemm_workspace_size(M, N, K, 3)
    cid, s = dg.gemm_select_config_ws(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, 3, need)
    note(f"[splitk] selected {dg.gemm_config_info(cid)['name']} x {s} for 8-bit {shape}")
    assert s > 1 and dg.gemm_config_info(cid)["name"].startswith("fp8_64x128")
    dg.gemm(a, b, out=c, split_k=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    pr = np.concatenate([np.full(N, 0), np.full(N, M - 1), np.arange(M), rng.integers(0, M, 20000)])
    pc = np.concatenate([np.arange(N), np.arange(N), np.full(M, N - 1), rng.integers(0, N, 20000)])
    A64 = fp8.decode(fp8._bits(A), "e4m3")
    B64 = fp8.decode(fp8._bits(B), "e4m3")
    ref = gemm64.bits_to_f64(gemm64.round_to_bits(gemm64.gemm_points_f64(A64, B64, pr, pc), "bf16"), "bf16")
    got = c[torch.from_numpy(pr).cuda(), torch.from_numpy(pc).cuda()].to("cpu", torch.float64).numpy()
    rep = tolerance.compare(got, ref, "bf16", K, float(np.abs(A64).max()), float(np.abs(B64).max()))
    assert rep["ok"], rep


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_long_k_single_pass_and_split(dtype):
    """K = 65536: 2048 K-steps of 32 in one workgroup (the K loop's counters
    and buffer offsets far from their first round), and the same product
    split 16 ways; a K that is not a multiple of 32 ends mid-step."""
    for M, N, K in [(136, 264, 65536), (128, 256, 40008)]:
        A, B = make_operands(M, N, K, dtype, "normal", 1800 + K % 97)
        a, b = A.cuda(), B.cuda()
        for cid, s in [(12, 1), (6, 1), (12, 16), (28, 5)]:
            note(f"[splitk] long K {dtype} {(M, N, K)} config {cid} splits {s}")
            c = dg.gemm(a, b, config=cid, splits=s)
            torch.cuda.synchronize()
            check_full(A, B, dtype, c)
