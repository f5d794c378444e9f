"""The allocation-free Muon step captured in a HIP graph (torch.cuda.CUDAGraph):
its work list goes up through kernel arguments and it records no memset, so
each replay is one full step.  Three replays, with eager work and
synchronisations between them, must each equal, bit for bit, the same step
run eagerly on a second copy of the state."""
import pytest

import matrix_optimizers_amd as mo

from _parity import hp_kwargs, random_case, to_dev
from matrix_optimizers_amd import workloads as wlmod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ns", ["bf16", "f32"])
def test_graph_replays_match_eager_steps(gpu, ns):
    import torch
    hp = wlmod.MuonHP(ns_dtype=ns)
    dt = "bf16" if ns == "bf16" else "f32"
    shapes = [(256, 512), (300, 200), (512, 512)]
    cases = [random_case(r, c, dt, dt, seed=5 + i) for i, (r, c) in enumerate(shapes)]
    make = lambda: [(to_dev(c.W, dt, gpu), to_dev(c.G, dt, gpu), to_dev(c.M, "f32", gpu)) for c in cases]
    graphed, eager = make(), make()
    kw = hp_kwargs(hp)
    mo.muon_owner_step_noalloc(graphed, **kw)     # outside the capture: code objects, scratch address
    mo.muon_owner_step_noalloc(eager, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mo.muon_owner_step_noalloc(graphed, **kw)
    # capturing launches nothing: the captured step has not run yet
    for (Wg, _, Mg), (We, _, Me) in zip(graphed, eager):
        assert torch.equal(Wg, We) and torch.equal(Mg, Me)
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        mo.muon_owner_step_noalloc(eager, **kw)
        junk = torch.randn(1 << 20, device=gpu).sum()   # eager work between replays
        torch.cuda.synchronize()
        del junk
        for (Wg, _, Mg), (We, _, Me) in zip(graphed, eager):
            assert torch.equal(Wg, We) and torch.equal(Mg, Me), f"replay {r}"
