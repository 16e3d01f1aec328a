"""gemm_run_noalloc (split K over the library's own scratch, for callers that
cannot allocate) against gemm_run_ws with a caller workspace, through the C
ABI: the same kernels and split count, so the results must be equal bit for
bit, and both must meet the oracle's acceptance rule.

Two calls in a row share the device's scratch; the second has a smaller
input, so the array still holds the first call's larger partial sums beyond
what the second one writes and reads.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_run_amd as dg
from dense_gemm_run_amd import _lib
from dense_gemm_run_amd.inputs import make_operands
from oracle import fp8, gemm64, tolerance

pytestmark = pytest.mark.gpu

CODE = {"f16": 1, "bf16": 2, "fp8_e4m3": 3}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_both(h, A, B, dtype):
    """C through gemm_run_ws (workspace from torch) and through
    gemm_run_noalloc; returns both and the split count."""
    M, K = A.shape
    N = B.shape[1]
    code = CODE[dtype]
    a, b = A.cuda(), B.cuda()
    odt = dg.out_dtype(a.dtype)
    need = dg.gemm_workspace_size(M, N, K, code)
    c_ws = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    c_na = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    _, splits = dg.gemm_select_config_ws(a.data_ptr(), b.data_ptr(), c_ws.data_ptr(), M, N, K, code, need)
    work = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    dg.gemm_run_ws(h, a.data_ptr(), b.data_ptr(), c_ws.data_ptr(), M, N, K, code, work.data_ptr(), need, stream)
    st = _lib.lib().gemm_run_noalloc(h, a.data_ptr(), b.data_ptr(), c_na.data_ptr(), M, N, K, code, stream)
    assert st == 0, dg.status_string(st)
    torch.cuda.synchronize()
    return c_ws, c_na, splits, need


def check_oracle(A, B, dtype, c):
    if dtype.startswith("fp8"):
        A64, B64 = fp8.decode(fp8._bits(A), "e4m3"), fp8.decode(fp8._bits(B), "e4m3")
        out = "bf16"
    else:
        A64, B64 = A.to(torch.float64).numpy(), B.to(torch.float64).numpy()
        out = dtype
    ref = gemm64.bits_to_f64(gemm64.round_to_bits(gemm64.gemm_f64(A64, B64), out), out)
    rep = tolerance.compare(c.to("cpu", torch.float64).numpy(), ref, out, A.shape[1],
                            float(np.abs(A64).max()), float(np.abs(B64).max()))
    assert rep["ok"], rep


@pytest.mark.parametrize("dtype", ["bf16", "f16", "fp8_e4m3"])
def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row(dtype):
    h = dg.gemm_create()
    try:
        # the larger product first, then a smaller one on the same scratch
        for M, N, K in [(128, 4096, 4096), (24, 3072, 8192)]:
            A, B = make_operands(M, N, K, dtype, "normal", 900 + M)
            c_ws, c_na, splits, need = run_both(h, A, B, dtype)
            note(f"[noalloc] {dtype} {(M, N, K)} splits {splits} scratch bytes {need}")
            assert splits > 1 and 0 < need <= _lib.NOALLOC_SCRATCH_BYTES
            assert torch.equal(c_ws.view(torch.int16), c_na.view(torch.int16))
            check_oracle(A, B, dtype, c_na)
    finally:
        dg.gemm_destroy(h)


def test_noalloc_without_a_split_runs_as_gemm_run():
    h = dg.gemm_create()
    try:
        M, N, K = 1024, 1024, 512     # many tiles, short K: no split
        A, B = make_operands(M, N, K, "bf16", "normal", 950)
        c_ws, c_na, splits, need = run_both(h, A, B, "bf16")
        assert splits == 1 and need == 0
        c = dg.gemm(A.cuda(), B.cuda())
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), c_na.view(torch.int16))
        check_oracle(A, B, "bf16", c_na)
    finally:
        dg.gemm_destroy(h)


def test_noalloc_argument_errors():
    h = dg.gemm_create()
    try:
        a = torch.ones((16, 64), dtype=torch.bfloat16, device="cuda")
        b = torch.ones((64, 32), dtype=torch.bfloat16, device="cuda")
        c = torch.empty((16, 32), dtype=torch.bfloat16, device="cuda")
        L = _lib.lib()
        assert L.gemm_run_noalloc(None, a.data_ptr(), b.data_ptr(), c.data_ptr(), 16, 32, 64, 2, None) == 1
        assert L.gemm_run_noalloc(h, a.data_ptr(), b.data_ptr(), c.data_ptr(), 16, 32, 64, 9, None) == 2
        assert L.gemm_run_noalloc(h, a.data_ptr(), b.data_ptr(), a.data_ptr(), 16, 32, 64, 2, None) == 5
        assert L.gemm_run_noalloc(h, a.data_ptr(), b.data_ptr(), c.data_ptr(), 0, 32, 64, 2, None) == 0
    finally:
        dg.gemm_destroy(h)
