"""The counted waits of the few-row kernel (gemm_skinny.hip), replayed.

Each wavefront of that kernel streams its K-steps of B into a ring of LDS
stages with direct-to-LDS loads and, before reading the stage of K-step j,
waits until at most `count` of its loads are still in flight.  That is right
only if at least `count` loads were issued after the last B load of step j.
The issue order differs between the prologue, the first round, the steady
rounds and the partial last round; this test replays it for every number of
K-steps per wavefront up to 40 and every configuration the launcher lists,
with the constants and the count formulas read from the source.  It also
checks that every step finds its own K-step's A fragments in its slot (they
are fetched kLeadA steps ahead, by the prologue or an earlier step).
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "dense_gemm_run_amd", "csrc", "gemm_skinny.hip")).read()


def const(name):
    return int(re.search(r"constexpr int %s = (\d+);" % name, SRC).group(1))


K_STAGES = const("kStages")
K_LEAD_A = const("kLeadA")
def _launch_list(text):
    return [tuple(int(x) for x in m.groups())
            for m in re.finditer(r"DGR_LAUNCH\((\d+), (\d+), (\d+), (\d+)\)", text)]


# (element bytes, rows, strip, K-step, wavefronts) of every instance the
# launcher lists: 16-bit ones before "} else {", 8-bit ones after it
_block = SRC[SRC.index("if constexpr (Elem<E>::BYTES == 2)"):SRC.index("#undef DGR_LAUNCH")]
_two, _one = _block.split("} else {")
CONFIGS = [(2,) + c for c in _launch_list(_two)] + [(1,) + c for c in _launch_list(_one)]


def loads_per_step(es, bms, bn, bk):
    """Direct-to-LDS B loads and 16-byte A loads of one K-step."""
    ki = 32 if es == 2 else 128            # K per MFMA
    frag = ki // 4 * es                    # fragment bytes per lane
    return bk * bn * es // 1024, (bk // ki) * (bms // 16) * (frag // 16)


def after_prologue(t, b_loads, a_loads):
    # the formula of the source's after_prologue()
    return (K_STAGES - 1 - t) * b_loads + min(K_STAGES - t, K_LEAD_A) * a_loads


def replay(per_wave, b_loads, a_loads):
    """Issue order of one wavefront and the waits it executes; returns the
    (step, count, loads issued after the step's last B load) of every wait."""
    L = b_loads + a_loads
    issued = []
    waits = []
    slot = {}                       # A slot -> the K-step whose fragments it holds

    def issue_b(j):
        issued.extend([("B", j)] * b_loads)

    def issue_a(j):
        issued.extend([("A", j)] * a_loads)
        slot[j % K_STAGES] = j

    def step(j, count, refill, fetch_a):
        last_b = max(i for i, e in enumerate(issued) if e == ("B", j))
        waits.append((j, count, len(issued) - 1 - last_b))
        # the MFMAs of step j read A slot j % kStages: it must hold step j
        assert slot.get(j % K_STAGES) == j, ("A slot", j, slot.get(j % K_STAGES))
        if refill:
            issue_b(j + K_STAGES)
        if refill or fetch_a:
            issue_a(j + K_LEAD_A)

    for s in range(-K_STAGES, 0):
        issue_b(s + K_STAGES)
        if s + K_LEAD_A >= 0:
            issue_a(s + K_LEAD_A)
    full, rem = divmod(per_wave, K_STAGES)
    steady = (K_STAGES - 1) * L + a_loads
    if full > 0:
        for t in range(K_STAGES):
            step(t, after_prologue(t, b_loads, a_loads) + t * L, True, True)
        for r in range(1, full):
            for t in range(K_STAGES):
                step(r * K_STAGES + t, steady, True, True)
    for t in range(rem):
        step(full * K_STAGES + t, after_prologue(t, b_loads, a_loads), False, t + K_LEAD_A < rem)
    return waits


def test_source_constants_and_configs_found():
    assert K_STAGES == 7 and 1 <= K_LEAD_A <= K_STAGES
    assert {c[0] for c in CONFIGS} == {1, 2}


@pytest.mark.parametrize("cfg", CONFIGS)
def test_every_wait_covers_its_b_loads(cfg):
    es, bms, bn, bk, w = cfg
    b_loads, a_loads = loads_per_step(es, bms, bn, bk)
    assert K_STAGES * (b_loads + a_loads) <= 63        # the vmcnt field
    for per_wave in range(1, 41):
        waits = replay(per_wave, b_loads, a_loads)
        assert [j for j, _, _ in waits] == list(range(per_wave))
        for j, count, after in waits:
            # vmcnt(count) lets `count` loads stay in flight: all of them must
            # have been issued after the B loads of step j
            assert after >= count, (cfg, per_wave, j, count, after)
        # and the steady rounds wait no more than they must
        if per_wave >= 2 * K_STAGES:
            j, count, after = waits[K_STAGES]
            assert count == after, (cfg, per_wave, count, after)
