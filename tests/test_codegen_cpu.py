"""Structure of the generated code of the pipelined MFMA kernels (16x16x32
for fp16/bf16, 32x32x64 for the 8-bit formats).

Their B tiles reach LDS through direct buffer->LDS loads that the kernel waits
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
CSRC = os.path.join(ROOT, "dense_gemm_run_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# source file, kernel-name pattern (-> bm, bn, bk), instances, element bytes,
# MFMA mnemonic, K depth of one MFMA, outputs of one MFMA
FAMILIES = {
    "mfma16x16": ("gemm_mfma16x16.hip", r"gemm_mfma16x16_kernel\S*?Li(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)E",
                  # {f16, bf16} x ({256x256, 256x128} x {32, 64} + 128x128x32 + 192x256x32
                  # + 64x128x32) x {one pass, split K}, + {256x256x32, 128x128x32,
                  # 192x256x32, 64x128x32} with A direct to LDS, + {128x128x32, 64x128x32}
                  # split with A direct to LDS
                  40, 2, "v_mfma_f32_16x16x32", 32, 16 * 16),
    "fp8": ("gemm_fp8.hip", r"gemm_fp8_kernelILi\d+ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)E",
            # {e4m3, e5m2} x ({256x256, 128x128} x {64, 128} x {one pass, split K}
            #                 + {256x256, 192x256, 128x128, 64x128} x 64 with A direct to LDS
            #                 + {128x128, 64x128} x 64 split with A direct to LDS)
            28, 1, "v_mfma_f32_32x32x64_f8f6f4", 64, 32 * 32),
}


def compile_family(fam, tmp):
    src, pat, count, ebytes, mnem, kdepth, outs = FAMILIES[fam]
    out = tmp / (fam + ".s")
    from dense_gemm_run_amd import build as lib_build
    flags = [f for f in lib_build.COMMON if f not in ("-fPIC",)]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = out.read_text().split("\n")
    found = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S*" + pat + r"\S*):", l)
        if m:
            bm, bn, bk = [int(x) for x in m.groups()[1:4]]
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            found[m.group(1)] = Kernel(fam, bm, bn, bk, ebytes, mnem, kdepth, outs, lines[i:end])
            found[m.group(1)].split = m.group(5) == '1'
            found[m.group(1)].adma = m.group(6) == '1'
    # per-kernel scratch use from the kernel descriptors
    for i, l in enumerate(lines):
        m = re.match(r"^\s*\.amdhsa_kernel (\S+)", l)
        if m and m.group(1) in found:
            for l2 in lines[i:i + 80]:
                m2 = re.match(r"^\s*\.amdhsa_private_segment_fixed_size (\d+)", l2)
                if m2:
                    found[m.group(1)].scratch = int(m2.group(1))
                    break
    assert len(found) == count, sorted(found)
    return found


class Kernel:
    def __init__(self, fam, bm, bn, bk, ebytes, mnem, kdepth, outs, body):
        self.fam, self.bm, self.bn, self.bk, self.body = fam, bm, bn, bk, body
        self.mnem, self.kdepth, self.outs = mnem, kdepth, outs
        # loads per wavefront per K-step and the pipeline depths
        self.a_loads = bm * bk * ebytes // 1024 // 4
        self.b_loads = bk * bn * ebytes // 1024 // 4
        self.lead = 256 // (bk * ebytes)                  # A register slots
        self.sb = 4 if bk * ebytes == 64 else 2           # B stages
        self.scratch = None
        self.split = False  # split-K instance: fp32 partials, no LDS epilogue
        self.adma = False   # A direct to LDS too, in B's ring


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("asm")
    found = {}
    for fam in FAMILIES:
        found.update(compile_family(fam, tmp))
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
    for name, kn in kernels.items():
        a_loads, b_loads, lead, sb, body = kn.a_loads, kn.b_loads, kn.lead, kn.sb, kn.body
        loads = a_loads + b_loads
        # the B loads of K-step it+1 were followed by groups it+2-SB .. it-1
        # and the A loads of group it (none when A goes direct to LDS after
        # the barrier, with B)
        count = (sb - 2) * loads + (0 if kn.adma else a_loads)
        ev = events(body)
        bars = [i for i, e in enumerate(ev) if e == "B"]
        # prologue, the peeled K-steps, the K-steps of the loop body, epilogue
        # (a split-K instance stores its partial sums without LDS: no
        # epilogue barrier)
        assert len(bars) == (1 if kn.split else 2) + 2 * lead, (name, len(bars))
        # prologue: groups -lead .. -1, each [A loads, B loads (if any)], then
        # a wait for the B loads of K-step 0
        pro = [e for e in ev[:bars[0]] if e in ("g", "L")]
        expect = []
        for g in range(-lead, 0):
            expect += ["L" if kn.adma else "g"] * a_loads + (["L"] * b_loads if g + sb >= 0 else [])
        assert pro == expect, (name, pro)
        pro_waits = [e[1] for e in ev[:bars[0]] if isinstance(e, tuple)]
        # before the prologue barrier at most the loads issued after the B
        # loads of K-step 0 may be in flight (the compiler may replace the
        # counted wait by stricter ones of its own)
        assert pro_waits and pro_waits[-1] <= (sb - 1) * loads, (name, pro_waits)
        # a K-step issues its A loads before its barrier and its B loads
        # after it, so between two barriers: B loads of the previous step,
        # then A loads of this one (A direct to LDS: A then B of the previous
        # step, all after its barrier)
        for k in range(2 * lead):
            seg = ev[bars[k] + 1:bars[k + 1]]
            got = [e for e in seg if e in ("g", "L")]
            if kn.adma:
                want = ["L"] * (a_loads + b_loads) if k else []
            else:
                want = (["L"] * b_loads if k else []) + ["g"] * a_loads
            assert got == want, (name, k, got)
            # the last vmcnt wait before the barrier is the counted one (the
            # compiler adds stricter waits of its own for register data)
            waits = [e[1] for e in seg if isinstance(e, tuple)]
            assert waits and waits[-1] == count, (name, k, waits)


def test_accumulators_stay_in_place(kernels):
    for name, kn in kernels.items():
        text = [x.strip() for x in kn.body]
        mfma = [x for x in text if x.startswith(kn.mnem)]
        per_slice = kn.bm * kn.bn // 4 // kn.outs     # MFMAs per wavefront per K-slice
        # peeled K-steps + the loop body's, bk/kdepth K-slices each
        assert len(mfma) == 2 * kn.lead * (kn.bk // kn.kdepth) * per_slice, (name, len(mfma))
        # only the first K-slice starts from 0
        ops_of = lambda x: [o.strip().split()[0] for o in x.split(None, 1)[1].split(",")]
        assert sum(1 for x in mfma if ops_of(x)[3] == "0") == per_slice, name
        for x in mfma:
            ops = ops_of(x)
            assert ops[3] in (ops[0], "0"), x   # accumulate in place or start from 0
        first = next(i for i, x in enumerate(text) if x.startswith("v_mfma"))
        last = max(i for i, x in enumerate(text) if x.startswith("v_mfma"))
        between = text[first:last]
        assert not [x for x in between if x.startswith(("v_accvgpr_write", "v_accvgpr_mov", "v_accvgpr_read"))], name
        # no accumulator is written before the first MFMA (it starts from 0)
        assert not [x for x in text[:first] if x.startswith("v_accvgpr_write")], name


def test_no_kernel_uses_scratch(kernels):
    # every loop over slots, stages and tiles is unrolled, so the register
    # arrays stay in registers: a rolled loop would index them at run time
    # and move them to scratch memory
    for name, kn in kernels.items():
        assert kn.scratch == 0, (name, kn.scratch)


def test_strip_kernel_uses_no_scratch_and_unscaled_8bit_mfma(tmp_path):
    """The few-row kernel (all element types) keeps its register arrays in
    registers, and its 8-bit MFMAs are the unscaled instruction (the
    builtin is the scaled one with zero scales)."""
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    from dense_gemm_run_amd import build as lib_build
    flags = [f for f in lib_build.COMMON if f not in ("-fPIC",)]
    out = tmp_path / "skinny.s"
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "gemm_skinny.hip"),
                        "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    sizes = [int(x) for x in re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", text)]
    assert len(sizes) >= 8 and all(x == 0 for x in sizes), sizes
    assert "v_mfma_f32_16x16x128_f8f6f4" in text
    assert "v_mfma_scale" not in text


def test_matrix_vector_kernel_structure(tmp_path):
    """The matrix-vector kernel (every element type, column count, rows per
    wavefront and schedule): each K step issues all of its U*(R+N) 16-byte
    loads (U chunks of R rows of A and N pieces of B) before its first wait
    for them, its products are exactly U*R*4*N two-element dot products on
    whole 32-bit words of A (no single-word loads of a piece), the
    cross-lane reduction selects with masks rather than with a lane-dependent
    array index (no chain of compares), and nothing spills."""
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    from dense_gemm_run_amd import build as lib_build
    flags = [f for f in lib_build.COMMON if f not in ("-fPIC",)]
    out = tmp_path / "gemv.s"
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "gemm_gemv.hip"),
                        "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = out.read_text().split("\n")
    pat = r"^(_Z\S*gemv_kernelI(DF16_|DF16b)Li(\d)ELi(\d+)ELi(\d+)ELb(\d)E\S*):"
    seen = []
    for i, l in enumerate(lines):
        m = re.match(pat, l)
        if not m:
            continue
        nv, rows, u = int(m.group(3)), int(m.group(4)), int(m.group(5))
        end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
        body = [x.strip() for x in lines[i:end]]
        name = m.group(1)
        seen.append((m.group(2), nv, rows, u, m.group(6)))
        insts = [x for x in body if x and not x.startswith((";", ".")) and not x.endswith(":")]
        ops = [x.split()[0] for x in insts]
        first_load = ops.index("buffer_load_dwordx4")
        first_wait = next(k for k in range(first_load, len(ops))
                          if ops[k] == "s_waitcnt" and "vmcnt" in insts[k])
        loads_before = ops[:first_wait].count("buffer_load_dwordx4")
        assert loads_before >= u * (rows + nv), (name, loads_before, u * (rows + nv))
        assert "buffer_load_dword" not in ops, name
        dots = sum(op.startswith("v_dot2") for op in ops)
        assert dots == u * rows * 4 * nv, (name, dots)
        assert sum(op.startswith("v_cmp_eq_u32") for op in ops) < 16, name
    assert len(seen) == 2 * 4 * 4, seen
    sizes = [int(x) for x in re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", "\n".join(lines))]
    assert len(sizes) == 32 and all(x == 0 for x in sizes), sizes


# ---------------------------------------------------------------- wait states around the MFMAs
# The MFMAs are inline assembly, so the compiler's hazard recognizer does not
# see them; the schedule relies on these rules of the CDNA3/CDNA4 ISA for
# XDL (matrix) instructions, checked here on the generated code:
#  * an MFMA with P passes needs P + 3 independent wait states between its
#    last write of an accumulator and a VALU or memory instruction reading
#    that accumulator; the MFMAs here have at most 16 passes, so 19;
#  * a VALU write of a VGPR needs a few wait states before an MFMA reads it
#    as source A or B (the fragments come from LDS reads, whose data the
#    compiler's own s_waitcnt covers; VALU writes of an operand register
#    must be further away than that small count);
#  * an MFMA accumulating into the registers of an earlier MFMA of the same
#    opcode (source C = destination, exactly overlapped) is ordered by the
#    hardware; every other MFMA-to-MFMA register dependence is absent.
ACC_READ_WAIT = 19
VALU_TO_MFMA_WAIT = 5


def _instructions(body):
    return [l.strip() for l in body
            if l.strip() and not l.strip().startswith((";", ".")) and not l.strip().split()[0].endswith(":")]


def _regs(tok, kind):
    m = re.match(kind + r"\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(kind + r"(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(line):
    parts = line.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def _wait_states(line):
    ops = _operands(line)
    return int(ops[0]) + 1 if line.split()[0] == "s_nop" else 1


def test_accumulators_are_read_only_after_the_mfma_latency(kernels):
    """Every non-MFMA read of an accumulator comes at least 19 wait states
    after the last MFMA that wrote it (the epilogue's s_nop waits plus the
    instructions before the read; the loop falls through into it)."""
    for name, kn in kernels.items():
        ins = _instructions(kn.body)
        last_write, ws, worst = {}, 0, None
        for l in ins:
            op = l.split()[0]
            ops = _operands(l)
            if op.startswith("v_mfma"):
                for r in _regs(ops[0], "a"):
                    last_write[r] = ws
            elif op != "s_nop":
                for o in ops[1:]:
                    for r in _regs(o, "a"):
                        if r in last_write:
                            d = ws - last_write.pop(r) - 1
                            worst = d if worst is None else min(worst, d)
            ws += _wait_states(l)
        assert worst is not None and worst >= ACC_READ_WAIT, (name, worst)


def test_mfma_operands_are_not_fresh_valu_results(kernels):
    """Between the first and the last MFMA, no VALU instruction writes a
    VGPR that an MFMA reads as source A or B within 5 wait states."""
    for name, kn in kernels.items():
        ins = _instructions(kn.body)
        first = next(i for i, l in enumerate(ins) if l.startswith("v_mfma"))
        last = max(i for i, l in enumerate(ins) if l.startswith("v_mfma"))
        written, ws = {}, 0
        for l in ins[first:last + 1]:
            op = l.split()[0]
            ops = _operands(l)
            if op.startswith("v_mfma"):
                for o in ops[1:3]:
                    for r in _regs(o, "v"):
                        if r in written:
                            assert ws - written[r] - 1 >= VALU_TO_MFMA_WAIT, (name, l)
            elif op.startswith("v_") and ops:
                for r in _regs(ops[0], "v"):
                    written[r] = ws
            elif op.startswith(("ds_read", "buffer_load", "global_load")) and ops and " lds" not in l:
                for r in _regs(ops[0], "v"):
                    written.pop(r, None)
            ws += _wait_states(l)


def test_fp32_kernel_structure(tmp_path):
    """The fp32 MFMA kernels (128 x 128, 64 x 128 and 64 x 64 tiles): no
    scratch, the 16x16x4 fp32 MFMA only, two blocks of FM x FN tiles x 8
    K-steps per round of the loop (256, 128 and 64 MFMAs), and one barrier
    per block besides the prologue's."""
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    from dense_gemm_run_amd import build as lib_build
    flags = [f for f in lib_build.COMMON if f not in ("-fPIC",)]
    out = tmp_path / "fp32.s"
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "gemm_fp32.hip"),
                        "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    sizes = [int(x) for x in re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", text)]
    assert sizes == [0, 0, 0], sizes
    bodies = {}
    for m in re.finditer(r"^(_Z\S*gemm_fp32_kernelILi(\d+)ELi(\d+)E\S*):[^\n]*$(.*?)^\.Lfunc_end", text, re.M | re.S):
        bodies[(int(m.group(2)), int(m.group(3)))] = m.group(4)
    assert sorted(bodies) == [(64, 64), (64, 128), (128, 128)], sorted(bodies)
    for (bm, bn), body in bodies.items():
        ins = [l.strip() for l in body.split("\n") if l.strip() and not l.strip().startswith((";", "."))]
        mfma = [l for l in ins if l.startswith("v_mfma")]
        assert len(mfma) == 2 * 8 * (bm // 32) * (bn // 32), (bm, bn, len(mfma))
        assert all(l.startswith("v_mfma_f32_16x16x4_f32") for l in mfma), (bm, bn)
        # prologue barrier + one per block of the loop round
        assert sum(1 for l in ins if l.split()[0] == "s_barrier") == 3, (bm, bn)


def test_short_k_kernel_structure(tmp_path):
    """The persistent short-K kernel (fp16 and bf16): no scratch, 64 MFMAs of
    16x16x32 per tile (4 K-steps x 4 x 4 tiles), two barriers per tile (data
    landed; operands read out of LDS), and only loads with the LDS destination
    for A and B (their registers are never staged)."""
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    from dense_gemm_run_amd import build as lib_build
    flags = [f for f in lib_build.COMMON if f not in ("-fPIC",)]
    out = tmp_path / "shortk.s"
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "gemm_shortk.hip"),
                        "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    sizes = [int(x) for x in re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", text)]
    assert sizes == [0, 0], sizes
    bodies = re.findall(r"^_Z\S*gemm_shortk_kernel\S*:[^\n]*$(.*?)^\.Lfunc_end", text, re.M | re.S)
    assert len(bodies) == 2
    for body in bodies:
        ins = [l.strip() for l in body.split("\n") if l.strip() and not l.strip().startswith((";", "."))]
        mfma = [l for l in ins if l.startswith("v_mfma")]
        assert len(mfma) == 64 and all(l.startswith("v_mfma_f32_16x16x32_") for l in mfma), len(mfma)
        assert sum(1 for l in ins if l.split()[0] == "s_barrier") == 2
        loads = [l for l in ins if l.split()[0].startswith("buffer_load")]
        assert loads and all(l.rstrip().endswith("lds") for l in loads), loads[:3]


def test_few_row_kernel_structure(tmp_path):
    """The one-launch few-row kernel (every instance): no scratch, only loads
    with the LDS destination (A and B of a K-step go straight to its ring
    stage), two barriers (both in the final sum of the wavefronts' partial
    sums: no wavefront waits for another during the K walk), the unscaled
    8-bit MFMA, and vector-memory waits only at the counts its ring assumes:
    (stages - 1 - t) K-steps of loads, t = 0 .. 3."""
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    from dense_gemm_run_amd import build as lib_build
    flags = [f for f in lib_build.COMMON if f not in ("-fPIC",)]
    out = tmp_path / "fewrow.s"
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "gemm_fewrow.hip"),
                        "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    sizes = [int(x) for x in re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", text)]
    assert len(sizes) == 24 and all(x == 0 for x in sizes), sizes
    assert "v_mfma_scale" not in text
    pat = r"^(_Z\S*gemm_fewrow_kernel\S*?(DF16_|DF16b|E4M3|E5M2)E?Li(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi4E\S*):[^\n]*$(.*?)^\.Lfunc_end"
    bodies = re.findall(pat, text, re.M | re.S)
    assert len(bodies) == 24
    for name, ty, bms, bn, bk, w, body in bodies:
        es = 1 if ty in ("E4M3", "E5M2") else 2
        bms, bn, bk = int(bms), int(bn), int(bk)
        assert bms in (8, 16, 32, 64), name
        per_step = (bk * bn * es) // 1024 + (bms * bk * es) // 1024     # B then A loads of a K-step
        ins = [l.strip() for l in body.split("\n") if l.strip() and not l.strip().startswith((";", "."))]
        loads = [l for l in ins if l.split()[0].startswith("buffer_load")]
        assert loads and all(l.rstrip().endswith("lds") for l in loads), (name, loads[:3])
        assert sum(1 for l in ins if l.split()[0] == "s_barrier") == 2, name
        mfma = [l.split()[0] for l in ins if l.startswith("v_mfma")]
        want = "v_mfma_f32_16x16x128_f8f6f4" if es == 1 else "v_mfma_f32_16x16x32_" + ("f16" if ty == "DF16_" else "bf16")
        assert mfma and all(m == want for m in mfma), (name, set(mfma))
        waits = {int(x) for x in re.findall(r"s_waitcnt[^\n]*vmcnt\((\d+)\)", body)}
        assert waits <= {t * per_step for t in range(4)}, (name, sorted(waits), per_step)
        assert 3 * per_step in waits, (name, sorted(waits))


# ---- the kernels with A staged two K-steps at a time (16-bit: 16x16x32
# MFMAs, 32-deep K-steps; 8-bit: 32x32x64 MFMAs, 64-deep K-steps)

PAIR_FAMILIES = {
    # source, kernel-name pattern (-> bm, bn), MFMA mnemonic, MFMA tile edge,
    # bytes of an A row per K-step (= bytes of a B row per K-step / (bn / 64))
    "mfma16x16": ("gemm_mfma16x16.hip", r"gemm_mfma16x16_pair_kernel\S*?Li(\d+)ELi(\d+)E", "v_mfma_f32_16x16x32", 16, 2),
    "fp8": ("gemm_fp8.hip", r"gemm_fp8_pair_kernelILi\d+ELi(\d+)ELi(\d+)E", "v_mfma_f32_32x32x64_f8f6f4", 32, 1),
}


@pytest.fixture(scope="module")
def pair_kernels(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    from dense_gemm_run_amd import build as lib_build
    flags = [f for f in lib_build.COMMON if f not in ("-fPIC",)]
    tmp = tmp_path_factory.mktemp("asm_pair")
    found, scratch = {}, {}
    for fam, (src, pat, mnem, edge, ebytes) in PAIR_FAMILIES.items():
        out = tmp / (fam + ".s")
        r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        lines = out.read_text().split("\n")
        here = {}
        for i, l in enumerate(lines):
            m = re.match(r"^(_Z\S*" + pat + r"\S*):", l)
            if m:
                end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
                here[m.group(1)] = (int(m.group(2)), int(m.group(3)), lines[i:end], mnem, edge, ebytes)
        for i, l in enumerate(lines):
            m = re.match(r"^\s*\.amdhsa_kernel (\S+)", l)
            if m and m.group(1) in here:
                for l2 in lines[i:i + 80]:
                    m2 = re.match(r"^\s*\.amdhsa_private_segment_fixed_size (\d+)", l2)
                    if m2:
                        scratch[m.group(1)] = int(m2.group(1))
                        break
        # 16-bit: {f16, bf16} x {256 x 256, 192 x 256, 128 x 128}; 8-bit: {E4M3, E5M2} x
        # {256 x 256, 192 x 256}
        assert len(here) == (6 if fam == "mfma16x16" else 4), (fam, sorted(here))
        found.update(here)
    return found, scratch


def test_pair_kernel_loads_and_counted_waits(pair_kernels):
    """Per wavefront: AH = bm/64 A loads per half K-step pair (a pair is bm
    rows of 128 bytes) and 4 B loads per K-step; odd K-steps issue B before
    their barrier and half an A pair after it, even K-steps the other half
    of the pair before and B after; the wait before barrier it leaves 2*4
    loads in flight (odd it) or 4 + 2*AH (even it), and the prologue 2*4 + AH."""
    found, _ = pair_kernels
    for name, (bm, bn, body, _, _, _) in found.items():
        ah, bl = bm // 64, bn // 64
        ev = events(body)
        bars = [i for i, e in enumerate(ev) if e == "B"]
        # prologue, 4 peeled K-steps, 4 in the loop body, epilogue
        assert len(bars) == 10, (name, len(bars))
        pro = [e for e in ev[:bars[0]] if e in ("g", "L")]
        assert pro == ["L"] * (2 * ah + 3 * bl + ah), (name, pro)
        pro_waits = [e[1] for e in ev[:bars[0]] if isinstance(e, tuple)]
        assert pro_waits and pro_waits[-1] == 2 * bl + ah, (name, pro_waits)
        for k in range(8):                     # K-step k's barrier is bars[k + 1]
            seg = ev[bars[k] + 1:bars[k + 1]]
            got = [e for e in seg if e in ("g", "L")]
            q = k % 4
            first_half = bl if q & 1 else ah
            prev_second = 0 if k == 0 else (ah if (k - 1) & 1 else bl)
            assert got == ["L"] * (prev_second + first_half), (name, k, got)
            waits = [e[1] for e in seg if isinstance(e, tuple)]
            assert waits and waits[-1] == (2 * bl if q & 1 else bl + 2 * ah), (name, k, waits)


def test_pair_kernel_accumulators_stay_in_place_without_scratch(pair_kernels):
    found, scratch = pair_kernels
    for name, (bm, bn, body, mnem, edge, _) in found.items():
        assert scratch[name] == 0, (name, scratch[name])
        text = [x.strip() for x in body]
        mfma = [x for x in text if x.startswith(mnem)]
        per_step = (bm // 2 // edge) * (bn // 2 // edge)
        assert len(mfma) == 8 * per_step, (name, len(mfma))
        ops_of = lambda x: [o.strip().split()[0] for o in x.split(None, 1)[1].split(",")]
        assert sum(1 for x in mfma if ops_of(x)[3] == "0") == per_step, name
        for x in mfma:
            ops = ops_of(x)
            assert ops[3] in (ops[0], "0"), x
        first = next(i for i, x in enumerate(text) if x.startswith("v_mfma"))
        last = max(i for i, x in enumerate(text) if x.startswith("v_mfma"))
        assert not [x for x in text[first:last]
                    if x.startswith(("v_accvgpr_write", "v_accvgpr_mov", "v_accvgpr_read"))], name


# ---- the 8-bit kernel with 128-deep K-steps on 16x16x128 MFMAs (two A slots
# and two B stages; barrier M after rows 0 .. MB-1 of tiles, barrier E before
# the last row)

K128_PAT = r"gemm_fp8_k128_kernelILi\d+ELi(\d+)ELi(\d+)E"


@pytest.fixture(scope="module")
def k128_kernels(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    from dense_gemm_run_amd import build as lib_build
    flags = [f for f in lib_build.COMMON if f not in ("-fPIC",)]
    out = tmp_path_factory.mktemp("asm_k128") / "fp8.s"
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "gemm_fp8.hip"), "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = out.read_text().split("\n")
    found, scratch = {}, {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S*" + K128_PAT + r"\S*):", l)
        if m:
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            found[m.group(1)] = (int(m.group(2)), int(m.group(3)), lines[i:end])
    for i, l in enumerate(lines):
        m = re.match(r"^\s*\.amdhsa_kernel (\S+)", l)
        if m and m.group(1) in found:
            for l2 in lines[i:i + 80]:
                m2 = re.match(r"^\s*\.amdhsa_private_segment_fixed_size (\d+)", l2)
                if m2:
                    scratch[m.group(1)] = int(m2.group(1))
                    break
    assert len(found) == 4, sorted(found)   # {E4M3, E5M2} x {256 x 256, 192 x 256}
    return found, scratch


def _k128_schedule(bm, bn):
    """Loads and waits of one K-step: per wavefront A_LOADS = bm/32 A loads
    (bm rows of 128 bytes) before barrier M, B_LOADS = bn/32 B loads (128
    rows of bn bytes) spread evenly over the NY MFMAs after it, NBE of them
    before barrier E; M waits for all but the A loads and all but the 2*MB
    A-fragment reads of rows 0 .. MB-1; E for all but NBE loads and all but
    the NRE transpose reads issued after the last A-fragment read."""
    fm, fn = bm // 32, bn // 32
    mb = fm // 2 - 1
    ny, nye = (fm - mb) * fn, (fm - 1 - mb) * fn
    op_lo = lambda pos, n, span: (pos * n + span - 1) // span
    a_loads, b_loads = bm // 32, bn // 32
    nbe = op_lo(nye, b_loads, ny)
    ya = (fm - 3 - mb) * fn + fn // 2
    nre = op_lo(nye, 4 * fn, ny) - op_lo(ya + 1, 4 * fn, ny)
    return a_loads, b_loads, nbe, 2 * mb, nre


def test_k128_kernel_loads_and_counted_waits(k128_kernels):
    found, _ = k128_kernels
    for name, (bm, bn, body) in found.items():
        a_loads, b_loads, nbe, lgkm_m, lgkm_e = _k128_schedule(bm, bn)
        ev = events(body)
        bars = [i for i, e in enumerate(ev) if e == "B"]
        # prologue, 2 barriers in each of 2 peeled and 2 looped K-steps, epilogue
        assert len(bars) == 10, (name, len(bars))
        pro = [e for e in ev[:bars[0]] if e in ("g", "L")]
        assert pro == ["L"] * (a_loads + 2 * b_loads), (name, pro)
        assert [e[1] for e in ev[:bars[0]] if isinstance(e, tuple)][-1] == b_loads, name
        for k in range(4):
            m_seg = ev[bars[2 * k] + 1:bars[2 * k + 1]]
            e_seg = ev[bars[2 * k + 1] + 1:bars[2 * k + 2]]
            carried = 0 if k == 0 else b_loads - nbe   # B loads after the previous barrier E
            assert [e for e in m_seg if e in ("g", "L")] == ["L"] * (carried + a_loads), (name, k)
            assert [e[1] for e in m_seg if isinstance(e, tuple)][-1] == a_loads, (name, k)
            assert [e for e in e_seg if e in ("g", "L")] == ["L"] * nbe, (name, k)
            assert [e[1] for e in e_seg if isinstance(e, tuple)][-1] == nbe, (name, k)
        text = [x.strip() for x in body]
        bar_lines = [i for i, x in enumerate(text) if x.startswith("s_barrier")]
        lgkm = []
        for i in bar_lines[1:-1]:
            w = next(text[j] for j in range(i - 1, 0, -1) if text[j].startswith("s_waitcnt"))
            m = re.search(r"lgkmcnt\((\d+)\)", w)
            lgkm.append(int(m.group(1)) if m else 15)
        assert lgkm == [lgkm_m, min(lgkm_e, 15)] * 4, (name, lgkm)


def test_k128_kernel_accumulators_stay_in_place_without_scratch(k128_kernels):
    found, scratch = k128_kernels
    for name, (bm, bn, body) in found.items():
        assert scratch[name] == 0, (name, scratch[name])
        text = [x.strip() for x in body]
        mfma = [x for x in text if x.startswith("v_mfma")]
        per_step = (bm // 32) * (bn // 32)
        assert mfma and all(x.startswith("v_mfma_f32_16x16x128_f8f6f4") for x in mfma), name
        assert len(mfma) == 4 * per_step, (name, len(mfma))
        ops_of = lambda x: [o.strip().split()[0] for o in x.split(None, 1)[1].split(",")]
        assert sum(1 for x in mfma if ops_of(x)[3] == "0") == per_step, name
        for x in mfma:
            ops = ops_of(x)
            assert ops[3] in (ops[0], "0"), x
        first = next(i for i, x in enumerate(text) if x.startswith("v_mfma"))
        last = max(i for i, x in enumerate(text) if x.startswith("v_mfma"))
        assert not [x for x in text[first:last]
                    if x.startswith(("v_accvgpr_write", "v_accvgpr_mov", "v_accvgpr_read"))], name
