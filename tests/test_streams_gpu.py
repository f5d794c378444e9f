"""The one-shot entry points launched on a side stream, given as a torch stream
and as a raw HIP stream handle, with the workspace left to the binding: the
results must equal, bit for bit, those of the same step on the current stream
(every kernel sums in a fixed order).  Between the launch and the
synchronisation the current stream allocates and fills memory, which would
take over a workspace block that was not tied to the launch stream."""
import pytest

import matrix_optimizers_amd as mo

pytestmark = pytest.mark.gpu


def _inputs(torch, seed, shapes, extra):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for r, c in shapes:
        W = torch.randn((r, c), device="cuda", generator=g) * 0.02
        G = torch.randn((r, c), device="cuda", generator=g) * 1e-3
        out.append([W, G] + extra(r, c, g))
    return out


def _clone(mats):
    return [[t.clone() for t in m] for m in mats]


def _run_both(torch, step_fn, mats):
    ref = _clone(mats)
    step_fn(ref, None)
    torch.cuda.synchronize()
    results = []
    for as_handle in (False, True):
        side = torch.cuda.Stream()
        got = _clone(mats)
        side.wait_stream(torch.cuda.current_stream())
        step_fn(got, side.cuda_stream if as_handle else side)
        churn = [torch.full((1 << 22,), float(k), device="cuda") for k in range(8)]
        del churn
        torch.cuda.synchronize()
        results.append(got)
    for got in results:
        for a, b in zip(got, ref):
            for x, y in zip(a, b):
                assert torch.equal(x, y)


def test_muon_on_side_stream(gpu):
    import torch
    mats = _inputs(torch, 1, [(256, 512), (384, 256)], lambda r, c, g: [torch.zeros((r, c), device="cuda")])
    _run_both(torch, lambda m, s: mo.muon_owner_step([tuple(x) for x in m], stream=s, lr=0.02), mats)


def test_shampoo_on_side_stream(gpu):
    import torch
    eye = lambda n: torch.eye(n, device="cuda") * 1e-6
    mats = _inputs(torch, 2, [(128, 192), (96, 64)], lambda r, c, g: [eye(r), eye(c)])
    _run_both(torch, lambda m, s: mo.shampoo_owner_step([tuple(x) for x in m], stream=s, lr=1e-3), mats)


def test_soap_on_side_stream(gpu):
    import torch
    eye = lambda n: torch.eye(n, device="cuda") * 1e-6
    zeros = lambda r, c: torch.zeros((r, c), device="cuda")
    mats = _inputs(torch, 3, [(96, 160), (64, 64)], lambda r, c, g: [eye(r), eye(c), zeros(r, c), zeros(r, c)])
    _run_both(torch, lambda m, s: mo.soap_owner_step([tuple(x) for x in m], stream=s, step=1, lr=1e-3,
                                                    eps=1e-3), mats)


def test_reusable_step_dropped_after_side_stream_call(gpu):
    """A reusable step (workspace allocated once, on the current stream) called
    on a side stream and dropped at once, while the current stream allocates
    and fills memory: the launch stream is recorded on the workspace block, so
    the caching allocator keeps it until the side stream's work is done, and
    the results equal the same step run on the current stream."""
    import torch
    mats = _inputs(torch, 4, [(512, 768), (768, 256)], lambda r, c, g: [torch.zeros((r, c), device="cuda")])
    ref = _clone(mats)
    mo.MuonOwnerStep([tuple(x) for x in ref], lr=0.02)()
    torch.cuda.synchronize()
    for as_handle in (False, True):
        got = _clone(mats)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        step = mo.MuonOwnerStep([tuple(x) for x in got], lr=0.02)
        step(side.cuda_stream if as_handle else side)
        del step
        churn = [torch.full((1 << 22,), float(k), device="cuda") for k in range(16)]
        del churn
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            for x, y in zip(a, b):
                assert torch.equal(x, y)
