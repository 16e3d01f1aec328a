"""GPU parity of the few-row kernel (gemm_skinny.hip) against the CPU oracle.

Its wavefronts split K and each runs a pipeline whose waits depend on how
many K-steps it gets: only a partial round, exactly one round, several
rounds plus a partial one.  The K values below give every configuration
1 .. 16 K-steps per wavefront, with ragged last steps, and the shapes cover
M below, at and above the configuration's rows, N not a multiple of the
strip, batches, and the selected configuration on the few-row workloads.
Same acceptance rule as the other parity tests; integer inputs bit-exact.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_run_amd as dg
from dense_gemm_run_amd.inputs import make_batched_operands, make_operands
from oracle import gemm64, tolerance
from test_gpu_parity import accepts

pytestmark = pytest.mark.gpu

DT_CODE = {"f16": 1, "bf16": 2}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def skinny_configs(eight=False):
    """The few-row configurations for 16-bit (or, with eight, 8-bit) inputs."""
    return [c for c in range(dg.gemm_config_count())
            if dg.gemm_config_info(c)["name"].startswith("skinny")
            and (dg.gemm_config_info(c)["dtype_mask"] == 0x18) == eight]


def check(A, B, dtype, c):
    ref, _ = (gemm64.reference_batched if A.ndim == 3 or B.ndim == 3 else gemm64.reference)(A, B, dtype)
    got = c.to("cpu", torch.float64).numpy()
    K = A.shape[-1]
    rep = tolerance.compare(got, ref, dtype, K, float(A.abs().max()) if A.numel() else 0.0,
                            float(B.abs().max()) if B.numel() else 0.0)
    assert rep["ok"], rep


@pytest.mark.parametrize("cid", range(15, 26))
def test_every_k_step_count(cid):
    if cid >= dg.gemm_config_count() or not dg.gemm_config_info(cid)["name"].startswith("skinny"):
        pytest.skip("not a few-row configuration")
    info = dg.gemm_config_info(cid)
    eight = info["dtype_mask"] == 0x18
    dtype = "fp8_e4m3" if eight else "bf16"
    per16 = 16 if eight else 8                 # elements per 16 bytes
    waves = info["threads"] // 64
    per_step = info["bk"] * waves            # K covered by one K-step of every wavefront
    for steps in [1, 2, 6, 7, 8, 13, 14, 15, 16]:
        K = steps * per_step - (3 * per16 if steps % 2 else 0)   # odd counts end with a ragged step
        M, N = info["bm"] - 3, 3 * info["bn"] + 2 * per16
        A, B = make_operands(M, N, K, dtype, "normal", 500 + steps)
        a, b = A.cuda(), B.cuda()
        assert accepts(cid, a, b, M, N, K)
        note(f"[skinny] config {cid} {info['name']} K-steps/wavefront {steps} shape {(M, N, K)}")
        c = dg.gemm(a, b, config=cid)
        torch.cuda.synchronize()
        if eight:
            from test_gpu_fp8 import check as check8
            check8(A, B, dtype, c)
        else:
            check(A, B, dtype, c)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1024, 4096), (16, 776, 520), (17, 256, 1032), (64, 512, 2048),
                                   (100, 264, 1000), (128, 1024, 4104), (300, 136, 512)])
def test_every_skinny_configuration(dtype, shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, dtype, "normal", 600 + M)
    Ai, Bi = make_operands(M, N, K, dtype, "integers", 601 + M)
    a, b, ai, bi = A.cuda(), B.cuda(), Ai.cuda(), Bi.cuda()
    ref_i, _ = gemm64.reference(Ai, Bi, dtype)
    for cid in skinny_configs():
        if not accepts(cid, a, b, M, N, K):
            continue
        note(f"[skinny] config {cid} {dg.gemm_config_info(cid)['name']} {dtype} {shape}")
        c = dg.gemm(a, b, config=cid)
        torch.cuda.synchronize()
        check(A, B, dtype, c)
        ci = dg.gemm(ai, bi, config=cid)
        torch.cuda.synchronize()
        assert np.array_equal(ci.to("cpu", torch.float64).numpy(), ref_i)


def test_skinny_batched_and_shared_b():
    batch, M, N, K = 5, 24, 528, 1544
    A, B = make_batched_operands(batch, M, N, K, "bf16", "normal", 610)
    a, b = A.cuda(), B.cuda()
    for cid in skinny_configs():
        note(f"[skinny] batched config {cid}")
        c = dg.gemm_batched(a, b, config=cid)
        torch.cuda.synchronize()
        check(A, B, "bf16", c)
    Bs = B[0].contiguous()
    c = dg.gemm_batched(a, Bs.cuda())
    torch.cuda.synchronize()
    check(A, Bs, "bf16", c)


def test_skinny_guards_untouched():
    M, N, K = 21, 200, 3000
    A, B = make_operands(M, N, K, "f16", "normal", 620)
    guard = 2048
    buf = torch.full((guard + M * N + guard,), 77.0, dtype=torch.float16, device="cuda")
    pattern = buf.clone()
    out = buf[guard:guard + M * N].view(M, N)
    for cid in skinny_configs():
        note(f"[skinny] guards config {cid}")
        dg.gemm(A.cuda(), B.cuda(), out=out, config=cid)
        torch.cuda.synchronize()
        assert torch.equal(buf[:guard], pattern[:guard]) and torch.equal(buf[guard + M * N:], pattern[guard + M * N:])
        check(A, B, "f16", out)


@pytest.mark.parametrize("shape", [(16, 14336, 512), (32, 14336, 256)])
def test_few_row_shapes_in_the_selected_configuration(shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, "bf16", "prefill", 630)
    a, b = A.cuda(), B.cuda()
    c = dg.gemm(a, b)
    torch.cuda.synchronize()
    cid = dg.gemm_select_config(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, 2)
    note(f"[skinny] selected {dg.gemm_config_info(cid)['name']} for {shape}")
    assert dg.gemm_config_info(cid)["name"].startswith("skinny")
    check(A, B, "bf16", c)


def test_8bit_few_rows_batched_guarded_and_full_size():
    from test_gpu_fp8 import check as check8
    for dtype in ("fp8_e4m3", "fp8_e5m2"):
        A, B = make_batched_operands(3, 24, 544, 1552, dtype, "normal", 640)
        a, b = A.cuda(), B.cuda()
        for cid in skinny_configs(eight=True):
            note(f"[skinny] 8-bit batched {dtype} config {cid}")
            c = dg.gemm_batched(a, b, config=cid)
            torch.cuda.synchronize()
            check8(A, B, dtype, c)
    M, N, K = 21, 208, 3008
    A, B = make_operands(M, N, K, "fp8_e4m3", "normal", 641)
    guard = 2048
    buf = torch.full((guard + M * N + guard,), 77.0, dtype=torch.bfloat16, device="cuda")
    pattern = buf.clone()
    out = buf[guard:guard + M * N].view(M, N)
    for cid in skinny_configs(eight=True):
        note(f"[skinny] 8-bit guards config {cid}")
        dg.gemm(A.cuda(), B.cuda(), out=out, config=cid)
        torch.cuda.synchronize()
        assert torch.equal(buf[:guard], pattern[:guard]) and torch.equal(buf[guard + M * N:], pattern[guard + M * N:])
        check8(A, B, "fp8_e4m3", out)
    for M, N, K in [(16, 4096, 4096), (64, 4096, 4096), (32, 4096, 4096), (16, 4096, 14336)]:
        A, B = make_operands(M, N, K, "fp8_e4m3", "normal", 642)
        a, b = A.cuda(), B.cuda()
        for cid in skinny_configs(eight=True):
            note(f"[skinny] 8-bit config {cid} for {(M, N, K)}")
            c = dg.gemm(a, b, config=cid)
            torch.cuda.synchronize()
            check8(A, B, "fp8_e4m3", c)
