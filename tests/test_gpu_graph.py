"""gemm_run inside a HIP graph (captured through torch's graph API on the
caller's stream).  The launch path makes no allocation and no memset, so a
captured product is one kernel node (two for a product split over K, whose
workspace comes from the graph's memory pool); every replay must give, bit for bit, what
an eager call gives on the inputs as they are at that moment.  Between the
replays the test does eager work of its own (rewriting A in place, an eager
product, synchronisation), as a program around a graph would.
"""
import sys

import pytest
import torch

import dense_gemm_run_amd as dg
from dense_gemm_run_amd.inputs import make_batched_operands, make_operands

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# one shape per kernel family the selection reaches, through gemm_run, or
# through gemm_run_ws where the last field asks for split K (the workspace
# then comes from the graph's memory pool), and the strip kernels forced by
# name
CASES = [(1000, 1000, 1000, "f16", None, False),        # 16x16x32 kernel at 64 x 128
         (2048, 2048, 1024, "bf16", None, False),       # 16x16x32 kernel at 256 x 256
         (16, 4096, 4096, "bf16", None, True),          # split K on 64 x 128 tiles
         (16, 4096, 4096, "bf16", None, False),         # few-row strip kernel (gemm_run's choice)
         (4096, 4, 4096, "bf16", None, False),          # matrix-vector kernel (K split over wavefronts)
         (127, 255, 65, "f16", None, False),            # generic kernel
         (1024, 1024, 2048, "fp8_e4m3", None, False),   # 8-bit kernel at 64 x 128
         (32, 4096, 4096, "fp8_e5m2", None, True),      # 8-bit split K on 64 x 128 tiles
         (32, 4096, 4096, "fp8_e5m2", None, False),     # 8-bit strip kernel (gemm_run's choice)
         (1024, 1024, 1024, "f32", None, False),        # fp32 MFMA kernel
         (4096, 4096, 128, "bf16", None, False),        # persistent short-K kernel
         (256, 4096, 4096, "bf16", None, True)]         # split K: partial sums in a workspace, then the sum


def config_id(name):
    return None if name is None else next(i for i in range(dg.gemm_config_count())
                                          if dg.gemm_config_info(i)["name"] == name)


@pytest.mark.parametrize("case", CASES)
def test_every_replay_matches_the_eager_call(case):
    M, N, K, dtype, cname, split_k = case
    cid = config_id(cname)
    note(f"[graph] {case}")
    A, B = make_operands(M, N, K, dtype, "normal", 800 + M)
    A2, _ = make_operands(M, N, K, dtype, "normal", 900 + M)
    a, b = A.cuda(), B.cuda()
    c = torch.empty((M, N), dtype=dg.out_dtype(a.dtype), device="cuda")
    dg.gemm(a, b, out=c, config=cid, split_k=split_k)      # creates the handle outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dg.gemm(a, b, out=c, config=cid, split_k=split_k)
    sources = [A, A2, A, A2]
    for r, src in enumerate(sources):
        a.copy_(src.cuda())               # eager work between replays
        torch.cuda.synchronize()
        c.zero_()
        g.replay()
        torch.cuda.synchronize()
        eager = dg.gemm(a, b, config=cid, split_k=split_k)
        torch.cuda.synchronize()
        same = torch.equal(c.view(torch.int16), eager.view(torch.int16))
        note(f"  replay {r}: identical to the eager call: {same}")
        assert same, (case, r)


def test_batched_replays_match_the_eager_call():
    batch, M, N, K = 4, 512, 768, 1024
    A, B = make_batched_operands(batch, M, N, K, "bf16", "normal", 950)
    a, b = A.cuda(), B.cuda()
    c = torch.empty((batch, M, N), dtype=torch.bfloat16, device="cuda")
    dg.gemm_batched(a, b, out=c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dg.gemm_batched(a, b, out=c)
    for r in range(3):
        a.mul_(-1.0)
        torch.cuda.synchronize()
        c.zero_()
        g.replay()
        torch.cuda.synchronize()
        eager = dg.gemm_batched(a, b)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), eager.view(torch.int16)), r
