"""CPU model of the GEMM cores' K pipeline (gemm_core.h, gemm_core8.h): the
order in which a wavefront issues its direct-to-LDS loads, reads stages and
passes the stage barriers, written out from the schedule the cores document,
and checked for every K length the kernels can see:

  * every K stage is loaded exactly once, LP / 2 instructions per wavefront;
  * the wait before each barrier (s_waitcnt vmcnt(N): at most N of this
    wavefront's loads still outstanding, loads completing in issue order) is
    exact: N equals the number of loads issued after the last load of the
    stage the barrier publishes (N larger would publish a stage not yet in
    LDS; smaller would wait longer than needed);
  * no LDS slot (stage mod 5) is refilled before the barrier that ends the
    last read of its previous stage;
  * every wait count used has a case in the core's wait_loads.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_optimizers_amd", "csrc")
NSTAGE = 5


def schedule(LP, nk):
    """Events of one wavefront: ('load', stage), ('read', stage),
    ('barrier', stage published, wait count)."""
    ev = []
    W_EVEN, W_ODD, W_FIRST = LP, 1 + LP // 2, 1 + LP

    def quarter(pair, q):
        l0, l1 = q * LP // 4, (q + 1) * LP // 4
        for l in range(l0, l1):
            ev.append(("load", pair + (l & 1)))

    for p in (0, 2):                      # prologue: pairs (0, 1) and (2, 3) whole
        for l in range(LP):
            ev.append(("load", p + (l & 1)))
    ev.append(("barrier", 0, W_FIRST))
    ev.append(("read", 0))                # (stage 0, substep 0)

    def step(ks, after, pa, qa, pb, qb):
        if pa >= 0:
            quarter(pa, qa)
        ev.append(("read", ks))           # (ks, substep 1), with the first substep's MFMAs
        ev.append(("barrier", ks + 1, after))
        if pb >= 0:
            quarter(pb, qb)
        ev.append(("read", ks + 1))       # (ks + 1, substep 0)

    step(0, W_EVEN, -1, 0, 4, 0)
    step(1, W_ODD, 4, 1, 4, 2)
    ks = 2
    while ks + 6 <= nk:
        step(ks, W_EVEN, ks + 2, 3, ks + 4, 0)
        step(ks + 1, W_ODD, ks + 4, 1, ks + 4, 2)
        ks += 2
    step(ks, W_EVEN, ks + 2, 3, -1, 0)
    step(ks + 1, 1, -1, 0, -1, 0)
    step(ks + 2, 0, -1, 0, -1, 0)
    ev.append(("read", nk - 1))           # (nk - 1, substep 1); the last substep reads nothing
    return ev


def check(LP, nk):
    ev = schedule(LP, nk)
    loads = [e[1] for e in ev if e[0] == "load"]
    assert sorted(loads) == sorted(s for s in range(nk) for _ in range(LP // 2)), (LP, nk)
    waits = set()
    n_loads = 0
    last_load = {}                        # stage -> index (in issue order) of its last load
    published = -1                        # highest stage published by a barrier
    unfenced = set()                      # stages read since the last barrier
    fenced = set()                        # stages whose every read is behind a barrier
    for e in ev:
        if e[0] == "load":
            prev = e[1] - NSTAGE
            if prev >= 0:
                assert prev in fenced and prev not in unfenced, ("slot reuse", LP, nk, e[1])
            last_load[e[1]] = n_loads
            n_loads += 1
        elif e[0] == "read":
            assert e[1] <= published, ("read before publish", LP, nk, e)
            unfenced.add(e[1])
            fenced.discard(e[1])
        else:
            _, stage, n = e
            after = n_loads - 1 - last_load[stage]
            assert n == after, (LP, nk, stage, n, after)
            waits.add(n)
            published = max(published, stage)
            fenced |= unfenced
            unfenced = set()
    return waits


def wait_cases(header):
    text = open(os.path.join(CSRC, header)).read()
    body = text[text.index("auto wait_loads"):]
    body = body[:body.index("};")]
    return {int(x) for x in re.findall(r"after == (\d+)", body)} | {0}


@pytest.mark.parametrize("header,LPs", [("gemm_core.h", [16, 12, 10]), ("gemm_core8.h", [8, 6])])
def test_pipeline_waits_are_exact_and_slots_safe(header, LPs):
    """4-wavefront core: LP = 2 (4 + NB) for tile widths NB = 4, 2, 1; 8-wavefront
    core: LP = 2 (2 + NB / 2) for NB = 4, 2.  K lengths: every even stage count
    from 8 (the 256-element minimum of bf16) to 600."""
    cases = wait_cases(header)
    for LP in LPs:
        used = set()
        for nk in range(8, 601, 2):
            used |= check(LP, nk)
        assert used <= cases, (header, LP, sorted(used - cases))


def test_model_catches_a_wrong_wait_and_an_early_refill(monkeypatch):
    """The checks themselves fire: an odd-step wait one too large, and a
    three-stage ring (a pair loaded into slots still being read)."""
    import sys
    mod = sys.modules[__name__]
    orig = mod.schedule

    def bad_wait(LP, nk):
        return [("barrier", e[1], e[2] + 1) if e[0] == "barrier" and e[2] == 1 + LP // 2 else e
                for e in orig(LP, nk)]
    monkeypatch.setattr(mod, "schedule", bad_wait)
    with pytest.raises(AssertionError):
        check(8, 16)
    monkeypatch.setattr(mod, "schedule", orig)
    monkeypatch.setattr(mod, "NSTAGE", 3)
    with pytest.raises(AssertionError):
        check(8, 16)
