"""GPU parity of the matrix-vector kernel (C = A·B with N <= 4: y = W·x)
against the CPU oracle, whole outputs, with the tolerance of
``oracle.tolerance``; integer inputs bit for bit."""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_run_amd as dg
from dense_gemm_run_amd.inputs import WORKLOADS, make_batched_operands, make_operands, workload_operands
from oracle import gemm64, tolerance

pytestmark = pytest.mark.gpu

DT_CODE = {"f32": 0, "f16": 1, "bf16": 2}
GEMV_CONFIGS = [i for i in range(dg.gemm_config_count())
                if dg.gemm_config_info(i)["name"].startswith("gemv")]


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(A, B, dtype, C):
    ref, _ = gemm64.reference(A, B, dtype)
    got = C.to("cpu", torch.float64).numpy()
    rep = tolerance.compare(got, ref, dtype, A.shape[1], float(A.abs().max()),
                            float(B.abs().max()))
    assert rep["ok"], rep
    return rep


def test_there_are_gemv_configurations():
    assert GEMV_CONFIGS


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 8), (37, 1, 520), (1000, 2, 4096), (777, 3, 1032),
                                   (64, 4, 264), (5000, 1, 8), (8191, 1, 4104), (17, 4, 1544)])
def test_gemv_configurations(dtype, shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, dtype, "decode", 40 + M + N)
    Ai, Bi = make_operands(M, N, K, dtype, "integers", 41 + M)
    a, b = A.cuda(), B.cuda()
    sel = dg.gemm_select_config(a.data_ptr(), b.data_ptr(), a.data_ptr() + (1 << 40), M, N, K,
                                DT_CODE[dtype])
    assert sel in GEMV_CONFIGS, sel
    ref_i, _ = gemm64.reference(Ai, Bi, dtype)
    for cid in GEMV_CONFIGS + [None]:
        note(f"[gemv] config {cid} {dtype} {shape}")
        c = dg.gemm(a, b, config=cid)
        torch.cuda.synchronize()
        check(A, B, dtype, c)
        ci = dg.gemm(Ai.cuda(), Bi.cuda(), config=cid)
        torch.cuda.synchronize()
        assert np.array_equal(ci.to("cpu", torch.float64).numpy(), ref_i)


def test_gemv_batched_and_unaligned():
    A, B = make_batched_operands(5, 300, 2, 1040, "bf16", "decode", 44)
    c = dg.gemm_batched(A.cuda(), B.cuda())
    torch.cuda.synchronize()
    ref, _ = gemm64.reference_batched(A, B, "bf16")
    got = c.to("cpu", torch.float64).numpy()
    for i in range(5):
        assert tolerance.compare(got[i], ref[i], "bf16", 1040, float(A.abs().max()),
                                 float(B.abs().max()))["ok"]
    # K not a multiple of 8, or an unaligned A: not the vector kernel, same answer
    A2, B2 = make_operands(300, 1, 1037, "f16", "decode", 45)
    a2, b2 = A2.cuda(), B2.cuda()
    assert dg.gemm_select_config(a2.data_ptr(), b2.data_ptr(), a2.data_ptr() + (1 << 40), 300, 1,
                                 1037, 1) not in GEMV_CONFIGS
    check(A2, B2, "f16", dg.gemm(a2, b2))
    with pytest.raises(dg.GemmError) as e:
        dg.gemm(a2, b2, config=GEMV_CONFIGS[0])
    assert e.value.name == "GEMM_ERR_CONFIG_MISMATCH"


@pytest.mark.parametrize("name", ["bf16_gemv_14336x1x4096", "bf16_gemv_4096x1x14336",
                                  "bf16_gemv_12288x4x4096"])
def test_gemv_workloads_whole(name):
    """The decode workloads at full size in bench.py's configuration, every
    output checked."""
    w = WORKLOADS[name]
    note(f"[gemv] full-size {name}")
    A, B = workload_operands(name)
    a, b = A.cuda(), B.cuda()
    C = torch.empty((w.M, w.N), dtype=a.dtype, device="cuda")
    cid = dg.gemm_select_config(a.data_ptr(), b.data_ptr(), C.data_ptr(), w.M, w.N, w.K,
                                DT_CODE[w.dtype])
    note(f"  config {cid} {dg.gemm_config_info(cid)['name']}")
    assert cid in GEMV_CONFIGS
    dg.gemm(a, b, out=C)
    torch.cuda.synchronize()
    note(f"  {check(A, B, w.dtype, C)}")


@pytest.mark.parametrize("shape", [(3, 300, 4, 4104), (3, 3000, 3, 4096), (2, 777, 1, 8200)])
def test_gemv_batched_at_long_k_every_configuration(shape):
    """Batches whose K reaches the K-split schedules (wavefronts splitting K,
    partial sums added in LDS): the selected configuration and every other
    vector configuration, each matrix of the batch against the oracle; K not
    a multiple of the 512-element chunk, M not a multiple of the rows per
    workgroup."""
    batch, M, N, K = shape
    A, B = make_batched_operands(batch, M, N, K, "bf16", "decode", 60 + M)
    a, b = A.cuda(), B.cuda()
    sel = dg.gemm_select_config_batched(a.data_ptr(), b.data_ptr(), a.data_ptr() + (1 << 40), batch, M,
                                        N, K, M * K, K * N, M * N, DT_CODE["bf16"])
    assert sel in GEMV_CONFIGS and dg.gemm_config_info(sel)["name"].startswith("gemv_kslice"), sel
    ref, _ = gemm64.reference_batched(A, B, "bf16")
    for cid in GEMV_CONFIGS + [None]:
        note(f"[gemv] batched config {cid} {shape}")
        c = dg.gemm_batched(a, b, config=cid)
        torch.cuda.synchronize()
        got = c.to("cpu", torch.float64).numpy()
        for i in range(batch):
            rep = tolerance.compare(got[i], ref[i], "bf16", K, float(A.abs().max()), float(B.abs().max()))
            assert rep["ok"], (cid, i, rep)
