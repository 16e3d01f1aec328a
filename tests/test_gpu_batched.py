"""GPU parity of the batched product (gemm_run_batched) against the CPU oracle.

Same acceptance rule as tests/test_gpu_parity.py (``oracle.tolerance``),
applied to every matrix of the batch; integer inputs must match bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_run_amd as dg
from dense_gemm_run_amd.inputs import WORKLOADS, make_batched_operands, workload_operands
from oracle import gemm64, tolerance
from test_gpu_parity import accepts

pytestmark = pytest.mark.gpu

DT_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_batch(A, B, dtype, C_gpu):
    K = A.shape[-1]
    ref, _ = gemm64.reference_batched(A, B, dtype)
    got = C_gpu.detach().to("cpu", torch.float64).numpy()
    assert got.shape == ref.shape
    amax = float(A.abs().max()) if A.numel() else 0.0
    bmax = float(B.abs().max()) if B.numel() else 0.0
    for i in range(ref.shape[0]):
        rep = tolerance.compare(got[i], ref[i], dtype, K, amax, bmax)
        assert rep["ok"], (i, rep)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 520, 776, 264), (4, 256, 256, 64), (5, 8, 8, 8),
                                   (2, 300, 1000, 40), (9, 1, 8, 128)])
def test_batched_every_configuration(dtype, shape):
    batch, M, N, K = shape
    A, B = make_batched_operands(batch, M, N, K, dtype, "normal", 20 + M)
    Ai, Bi = make_batched_operands(batch, M, N, K, dtype, "integers", 21 + M)
    a, b, ai, bi = A.cuda(), B.cuda(), Ai.cuda(), Bi.cuda()
    ref_i, _ = gemm64.reference_batched(Ai, Bi, dtype)
    for cid in range(dg.gemm_config_count()):
        info = dg.gemm_config_info(cid)
        if not (info["dtype_mask"] >> DT_CODE[dtype]) & 1:
            continue
        if not accepts(cid, a, b, M, N, K, batch):
            continue
        note(f"[batched] config {cid} {info['name']} {dtype} {shape}")
        c = dg.gemm_batched(a, b, config=cid)
        torch.cuda.synchronize()
        check_batch(A, B, dtype, c)
        ci = dg.gemm_batched(ai, bi, config=cid)
        torch.cuda.synchronize()
        assert np.array_equal(ci.to("cpu", torch.float64).numpy(), ref_i)


def test_batched_short_k_walks_several_tiles_per_workgroup():
    """The persistent short-K kernel (config 48) on a batch of 60 ragged
    matrices, 540 tiles of 128 x 128, more than its resident workgroups (two
    per CU), so workgroups walk tiles of different matrices: whole output
    against the oracle, and bit-exact on integer inputs."""
    batch, M, N, K = 60, 300, 264, 72
    cid = next(i for i in range(dg.gemm_config_count()) if dg.gemm_config_info(i)["name"] == "shortk_128x128x128")
    A, B = make_batched_operands(batch, M, N, K, "bf16", "normal", 60)
    Ai, Bi = make_batched_operands(batch, M, N, K, "bf16", "integers", 61)
    note(f"[batched] short-K persistent {(batch, M, N, K)}")
    c = dg.gemm_batched(A.cuda(), B.cuda(), config=cid)
    torch.cuda.synchronize()
    check_batch(A, B, "bf16", c)
    ci = dg.gemm_batched(Ai.cuda(), Bi.cuda(), config=cid)
    torch.cuda.synchronize()
    ref_i, _ = gemm64.reference_batched(Ai, Bi, "bf16")
    assert np.array_equal(ci.to("cpu", torch.float64).numpy(), ref_i)


@pytest.mark.parametrize("shared", ["a", "b"])
def test_batched_shared_operand(shared):
    batch, M, N, K = 6, 384, 512, 96
    A, B = make_batched_operands(batch, M, N, K, "bf16", "normal", 30, share_b=(shared == "b"))
    if shared == "a":
        A = A[0].contiguous()            # one [M, K] matrix for every product
    note(f"[batched] shared {shared}: A {tuple(A.shape)} B {tuple(B.shape)}")
    c = dg.gemm_batched(A.cuda(), B.cuda())
    torch.cuda.synchronize()
    check_batch(A, B, "bf16", c)


def test_batch_of_one_matches_the_single_call_bitwise():
    A, B = make_batched_operands(1, 777, 1032, 200, "f16", "normal", 31)
    cb = dg.gemm_batched(A.cuda(), B.cuda())
    cs = dg.gemm(A[0].cuda(), B[0].cuda())
    torch.cuda.synchronize()
    assert torch.equal(cb[0], cs)


def test_batched_errors_and_empty_batch():
    h = dg.gemm_create()
    try:
        a = torch.ones((2, 4, 4), dtype=torch.float16, device="cuda")
        c = torch.empty((2, 4, 4), dtype=torch.float16, device="cuda")
        with pytest.raises(dg.GemmError) as e:    # C matrices overlapping each other
            dg.gemm_run_batched(h, a.data_ptr(), a.data_ptr(), c.data_ptr(), 2, 4, 4, 4,
                                16, 16, 8, 1, None)
        assert e.value.name == "GEMM_ERR_ALIASING"
        dg.gemm_run_batched(h, a.data_ptr(), a.data_ptr(), c.data_ptr(), 0, 4, 4, 4,
                            16, 16, 16, 1, None)   # empty batch: nothing to do
        with pytest.raises(ValueError):
            dg.gemm_batched(a, torch.ones((3, 4, 4), dtype=torch.float16, device="cuda"))
        with pytest.raises(ValueError):
            dg.gemm_batched(a.transpose(1, 2), a)   # non-row-major matrices: rejected
        torch.cuda.synchronize()
    finally:
        dg.gemm_destroy(h)


@pytest.mark.parametrize("name", ["bf16_batched_16x2048x2048x2048", "bf16_batched_64x2048x2048x128"])
def test_batched_workloads_sampled(name):
    """The batched workloads at full size, in bench.py's configuration: three
    matrices of the batch checked on whole rows, columns and random points."""
    w = WORKLOADS[name]
    note(f"[batched] full-size {name}")
    A, B = workload_operands(name)
    a, b = A.cuda(), B.cuda()
    C = torch.empty((w.batch, w.M, w.N), dtype=a.dtype, device="cuda")
    cid = dg.gemm_select_config_batched(a.data_ptr(), b.data_ptr(), C.data_ptr(), w.batch, w.M,
                                        w.N, w.K, w.M * w.K, w.K * w.N, w.M * w.N,
                                        DT_CODE[w.dtype])
    note(f"  config {cid} {dg.gemm_config_info(cid)['name']}")
    dg.gemm_batched(a, b, out=C)
    torch.cuda.synchronize()
    assert not torch.isnan(C).any()
    rng = np.random.default_rng(w.seed)
    for i in [0, w.batch - 1, int(rng.integers(0, w.batch))]:
        Ai, Bi = A[i], B[i]
        rows = [0, w.M - 1, int(rng.integers(0, w.M))]
        cols = [0, w.N - 1, int(rng.integers(0, w.N))]
        pr = np.concatenate([np.full(w.N, r) for r in rows] + [np.arange(w.M) for _ in cols]
                            + [rng.integers(0, w.M, 5000)])
        pc = np.concatenate([np.arange(w.N) for _ in rows] + [np.full(w.M, c) for c in cols]
                            + [rng.integers(0, w.N, 5000)])
        exact_vals = gemm64.gemm_points_f64(Ai.to(torch.float64).numpy(),
                                            Bi.to(torch.float64).numpy(), pr, pc)
        ref = gemm64.bits_to_f64(gemm64.round_to_bits(exact_vals, w.dtype), w.dtype)
        got = C[i][torch.from_numpy(pr).cuda(), torch.from_numpy(pc).cuda()].to(
            "cpu", torch.float64).numpy()
        rep = tolerance.compare(got, ref, w.dtype, w.K, float(A.abs().max()), float(B.abs().max()))
        assert rep["ok"], (i, rep)
        note(f"  matrix {i}: {rep}")
