"""GPU parity of the one-launch few-row kernel (gemm_fewrow.hip) against the
CPU oracle.

Each wavefront owns a contiguous range of S K-steps (a multiple of the 4
ring stages, rounded up so that steps past K read zeros) and walks it from a
strip-dependent starting step.  The K values below give every configuration
one, two, three and several rounds of its ring, a ragged last K-step and
steps wholly past K; the shapes cover M below, at and above the 16 rows of a
workgroup, N not a multiple of the strip, enough strips for every starting
step, batches with a shared B, K = 0, and the guards around C.  Same
acceptance rule as the other parity tests; integer inputs bit-exact.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_run_amd as dg
from dense_gemm_run_amd.inputs import make_batched_operands, make_operands
from oracle import fp8, gemm64, tolerance
from test_gpu_parity import accepts

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def fewrow_configs(eight=False):
    """The one-launch few-row configurations for 16-bit (or, with eight, 8-bit) inputs."""
    return [c for c in range(dg.gemm_config_count())
            if dg.gemm_config_info(c)["name"].startswith("fewrow")
            and (dg.gemm_config_info(c)["dtype_mask"] == 0x18) == eight]


def check(A, B, dtype, c):
    if dtype.startswith("fp8"):
        from test_gpu_fp8 import check as check8
        check8(A, B, dtype, c)
        return
    ref, _ = (gemm64.reference_batched if A.ndim == 3 or B.ndim == 3 else gemm64.reference)(A, B, dtype)
    got = c.to("cpu", torch.float64).numpy()
    K = A.shape[-1]
    rep = tolerance.compare(got, ref, dtype, K, float(A.abs().max()) if A.numel() else 0.0,
                            float(B.abs().max()) if B.numel() else 0.0)
    assert rep["ok"], rep


def test_there_are_few_row_configurations():
    assert len(fewrow_configs()) >= 1 and len(fewrow_configs(eight=True)) >= 1


@pytest.mark.parametrize("eight", [False, True])
def test_every_round_count(eight):
    """1, 2, 3 and 5 rounds of the ring per wavefront, ragged last steps,
    steps past K, one and two row blocks, N off the strip width."""
    for cid in fewrow_configs(eight):
        info = dg.gemm_config_info(cid)
        dtype = "fp8_e4m3" if eight else "bf16"
        per16 = 16 if eight else 8                  # elements per 16 bytes
        waves = info["threads"] // 64
        per_round = 4 * waves * info["bk"]          # K one round of every wavefront covers
        for rounds, M in [(1, 16), (2, 7), (3, 19), (5, 1)]:
            for K in (rounds * per_round, rounds * per_round - 3 * per16 - per_round // 2):
                if K <= (rounds - 1) * per_round:
                    continue
                N = 3 * info["bn"] + 2 * per16
                A, B = make_operands(M, N, K, dtype, "normal", 700 + rounds * 10 + M)
                a, b = A.cuda(), B.cuda()
                assert accepts(cid, a, b, M, N, K)
                note(f"[fewrow] config {cid} {info['name']} rounds {rounds} shape {(M, N, K)}")
                c = dg.gemm(a, b, config=cid)
                torch.cuda.synchronize()
                check(A, B, dtype, c)
                Ai, Bi = make_operands(M, N, K, dtype, "integers", 701 + rounds * 10 + M)
                ci = dg.gemm(Ai.cuda(), Bi.cuda(), config=cid)
                torch.cuda.synchronize()
                if eight:
                    ref_i, _ = fp8.reference_fp8(Ai, Bi, "e4m3")
                else:
                    ref_i, _ = gemm64.reference(Ai, Bi, dtype)
                assert np.array_equal(ci.to("cpu", torch.float64).numpy(), ref_i), (cid, M, N, K)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8_e4m3", "fp8_e5m2"])
@pytest.mark.parametrize("shape", [(1, 64, 16), (16, 1000, 520), (13, 4096, 1032), (33, 136, 2048)])
def test_every_few_row_configuration(dtype, shape):
    M, N, K = shape
    eight = dtype.startswith("fp8")
    A, B = make_operands(M, N, K, dtype, "normal", 720 + M)
    a, b = A.cuda(), B.cuda()
    for cid in fewrow_configs(eight):
        if not accepts(cid, a, b, M, N, K):
            continue
        note(f"[fewrow] config {cid} {dg.gemm_config_info(cid)['name']} {dtype} {shape}")
        c = dg.gemm(a, b, config=cid)
        torch.cuda.synchronize()
        check(A, B, dtype, c)


def test_k_zero_gives_zeros():
    for eight in (False, True):
        dtype = "fp8_e4m3" if eight else "bf16"
        A, B = make_operands(5, 64, 0, dtype, "normal", 730)
        for cid in fewrow_configs(eight):
            note(f"[fewrow] K = 0 config {cid}")
            c = dg.gemm(A.cuda(), B.cuda(), config=cid)
            torch.cuda.synchronize()
            assert torch.count_nonzero(c.float()).item() == 0


def test_batched_and_shared_b():
    for eight in (False, True):
        dtype = "fp8_e5m2" if eight else "f16"
        batch, M, N, K = 5, 12, 560, 1552
        A, B = make_batched_operands(batch, M, N, K, dtype, "normal", 740)
        a, b = A.cuda(), B.cuda()
        for cid in fewrow_configs(eight):
            note(f"[fewrow] batched {dtype} config {cid}")
            c = dg.gemm_batched(a, b, config=cid)
            torch.cuda.synchronize()
            check(A, B, dtype, c)
            Bs = B[0].contiguous()
            c = dg.gemm_batched(a, Bs.cuda(), config=cid)
            torch.cuda.synchronize()
            check(A, Bs, dtype, c)


def test_guards_untouched():
    for eight in (False, True):
        dtype = "fp8_e4m3" if eight else "f16"
        out_dtype = torch.bfloat16 if eight else torch.float16
        M, N, K = 21, 208, 3008
        A, B = make_operands(M, N, K, dtype, "normal", 750)
        guard = 2048
        buf = torch.full((guard + M * N + guard,), 77.0, dtype=out_dtype, device="cuda")
        pattern = buf.clone()
        out = buf[guard:guard + M * N].view(M, N)
        for cid in fewrow_configs(eight):
            note(f"[fewrow] guards {dtype} config {cid}")
            dg.gemm(A.cuda(), B.cuda(), out=out, config=cid)
            torch.cuda.synchronize()
            assert torch.equal(buf[:guard], pattern[:guard])
            assert torch.equal(buf[guard + M * N:], pattern[guard + M * N:])
            check(A, B, dtype, out)


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_full_size_sixteen_tokens_whole(dtype):
    """16 x 4096 x 4096 (256 or 128 strips: every starting step of the walk)
    in every configuration, compared whole."""
    M, N, K = 16, 4096, 4096
    A, B = make_operands(M, N, K, dtype, "prefill", 760)
    a, b = A.cuda(), B.cuda()
    for cid in fewrow_configs(dtype.startswith("fp8")):
        note(f"[fewrow] full size {dtype} config {cid}")
        c = dg.gemm(a, b, config=cid)
        torch.cuda.synchronize()
        check(A, B, dtype, c)


SELECTED16 = [(16, 4096, 4096), (1, 4096, 4096), (24, 4096, 4096), (16, 4096, 14336), (16, 8192, 4096),
              (16, 4096, 2048), (32, 8192, 4096), (48, 4096, 4096), (64, 2048, 4096), (96, 4096, 4096),
              (128, 4096, 4096), (100, 4096, 1000), (1, 6144, 4096), (40, 6144, 4096), (24, 2048, 8192),
              (40, 2048, 8192), (1, 11008, 4096), (3, 3072, 3072)]
SELECTED8 = [(16, 4096, 4096), (1, 4096, 4096), (24, 4096, 4096), (16, 4096, 14336), (16, 8192, 4096),
             (16, 4096, 2048), (32, 8192, 4096), (48, 4096, 4096), (64, 2048, 4096), (96, 2048, 4096),
             (1, 3072, 8192), (24, 1024, 4096), (40, 2048, 2048)]


@pytest.mark.parametrize("dtype,shape", [("bf16", s) for s in SELECTED16] + [("fp8_e4m3", s) for s in SELECTED8])
def test_few_row_shapes_in_the_selected_configuration(dtype, shape):
    """gemm_run's choice for few rows where one of the kernel's configurations
    fits one wave of workgroups (up to 8 rows, 16-bit, also 11008 columns in
    344 strips) is this kernel; the product is compared with the oracle
    whole."""
    M, N, K = shape
    code = 3 if dtype.startswith("fp8") else 2
    A, B = make_operands(M, N, K, dtype, "prefill" if code == 2 else "normal", 770 + M)
    a, b = A.cuda(), B.cuda()
    c = dg.gemm(a, b)
    torch.cuda.synchronize()
    cid = dg.gemm_select_config(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, code)
    note(f"[fewrow] selected {dg.gemm_config_info(cid)['name']} for {dtype} {shape}")
    assert dg.gemm_config_info(cid)["name"].startswith("fewrow")
    check(A, B, dtype, c)
