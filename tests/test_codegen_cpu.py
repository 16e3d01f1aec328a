"""Structure of the generated code of the 16x16x32 MFMA kernel.

Its B tiles reach LDS through direct buffer->LDS loads that the kernel waits
for by count: before each barrier a wavefront waits until at most a fixed
number of its own loads are outstanding, which is right only if every K-step
issues its A loads before its barrier and its B loads after it, in that
order.  The MFMAs are inline assembly, so the compiler may move other
instructions around them; these tests compile the kernel to gfx950 assembly
(no GPU needed) and check that the issue order is the one the counts assume,
and that the accumulators stay in place.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "dense_gemm_run_amd", "csrc", "gemm_mfma16x16.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "k.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = out.read_text().split("\n")
    found = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S*gemm_mfma16x16_kernel\S*?Li(\d+)ELi(\d+)E\S*):", l)
        if m:
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            found[m.group(1)] = (int(m.group(2)), int(m.group(3)), lines[i:end])
    assert len(found) == 4, sorted(found)   # {f16, bf16} x {256x256, 256x128}
    return found


def events(body):
    """Vector-memory loads, waits and barriers in issue order."""
    ev = []
    for x in body:
        x = x.strip()
        if not x or x.startswith(";"):
            continue
        op = x.split()[0]
        if op.startswith("buffer_load"):
            ev.append("L" if " lds" in x or x.endswith("lds") else "g")
        elif op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", x)
            if m:
                ev.append(("vm", int(m.group(1))))
        elif op == "s_barrier":
            ev.append("B")
    return ev


def test_every_k_step_issues_its_loads_in_order_before_the_counted_wait(kernels):
    for name, (bm, bn, body) in kernels.items():
        a_loads = bm * 64 // 1024 // 4
        b_loads = 32 * bn * 2 // 1024 // 4
        count = a_loads + b_loads + a_loads
        ev = events(body)
        bars = [i for i, e in enumerate(ev) if e == "B"]
        # prologue + 4 peeled K-steps + the 4 of the loop body, then the epilogue's
        assert len(bars) == 10, (name, len(bars))
        # prologue: A(0) A(1) B(0) A(2) B(1) A(3) B(2), then a wait for B(0)
        pro = [e for e in ev[:bars[0]] if e in ("g", "L")]
        assert pro == (["g"] * a_loads * 2 + ["L"] * b_loads + (["g"] * a_loads + ["L"] * b_loads) * 2), name
        pro_waits = [e[1] for e in ev[:bars[0]] if isinstance(e, tuple)]
        assert pro_waits and pro_waits[-1] == 2 * (a_loads + b_loads), (name, pro_waits)
        # a K-step issues its A loads before its barrier and its B loads
        # after it, so between two barriers: B loads of the previous step,
        # then A loads of this one
        for k in range(8):
            seg = ev[bars[k] + 1:bars[k + 1]]
            loads = [e for e in seg if e in ("g", "L")]
            expect = (["L"] * b_loads if k else []) + ["g"] * a_loads
            assert loads == expect, (name, k, loads)
            # the last vmcnt wait before the barrier is the counted one, and
            # nothing inside the step waits for more
            waits = [e[1] for e in seg if isinstance(e, tuple)]
            assert waits and waits[-1] == count, (name, k, waits)
            assert min(waits) == count, (name, k, waits)


def test_accumulators_stay_in_place(kernels):
    for name, (bm, bn, body) in kernels.items():
        text = [x.strip() for x in body]
        mfma = [x for x in text if x.startswith("v_mfma_f32_16x16x32")]
        fm, fn = bm // 32, bn // 32
        # 4 peeled K-steps + a 4-step loop body
        assert len(mfma) == 8 * fm * fn, (name, len(mfma))
        for x in mfma:
            ops = [o.strip() for o in x.split(None, 1)[1].split(",")]
            assert ops[3] in (ops[0], "0"), x   # accumulate in place or start from 0
        first = next(i for i, x in enumerate(text) if x.startswith("v_mfma"))
        last = max(i for i, x in enumerate(text) if x.startswith("v_mfma"))
        between = text[first:last]
        assert not [x for x in between if x.startswith(("v_accvgpr_write", "v_accvgpr_mov", "v_accvgpr_read"))], name
        # no accumulator is written before the first MFMA (it starts from 0)
        assert not [x for x in text[:first] if x.startswith("v_accvgpr_write")], name
