"""The allocation-free Muon entry point (muon_owner_step_noalloc), through the
C ABI: on the library's static scratch array it must give the same bits as
muon_owner_step with a caller workspace (same kernels, same work list), on
two calls in a row with the second bucket smaller than the first, and the
fp64 oracle's tolerances on a sampled matrix.  A bucket whose workspace
exceeds the array is refused before anything runs."""
import ctypes

import numpy as np
import pytest

import matrix_optimizers_amd as mo
from matrix_optimizers_amd import _binding as B

from _parity import check_case, hp_kwargs, random_case, to_dev, to_host
from matrix_optimizers_amd import workloads as wlmod

pytestmark = pytest.mark.gpu

BF = wlmod.MuonHP()


def _bucket(shapes, seed, device, dtype="bf16"):
    cases = [random_case(r, c, dtype, dtype, seed=seed + i) for i, (r, c) in enumerate(shapes)]
    mats = [(to_dev(c.W, dtype, device), to_dev(c.G, dtype, device), to_dev(c.M, "f32", device))
            for c in cases]
    return cases, mats


def _clone(mats):
    return [(W.clone(), G, M.clone()) for (W, G, M) in mats]


def _noalloc_raw(mats, ups, hp):
    """The new entry point called directly through ctypes (no binding logic)."""
    lib = mo.load_library()
    descs = [mo.tensor_descriptor(W, G, M, u) for (W, G, M), u in zip(mats, ups)]
    arr, n = B._array(descs)
    h = mo.hparams(**hp_kwargs(hp))
    import torch
    return lib.muon_owner_step_noalloc(arr, n, ctypes.byref(h),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("ns", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point_twice(gpu, ns):
    import torch
    hp = BF if ns == "bf16" else wlmod.MuonHP(ns_dtype="f32")
    dt = "bf16" if ns == "bf16" else "f32"
    # first call: a larger bucket; second: a smaller one (the array keeps the
    # first call's contents, which the second must not depend on)
    for shapes, seed in (([(512, 768), (768, 256), (300, 1000), (1024, 1024), (0, 7)], 11),
                         ([(200, 96), (64, 64)], 41)):
        cases, mats = _bucket(shapes, seed, gpu, dt)
        ref, got = _clone(mats), _clone(mats)
        ups_ref = [torch.empty(W.shape, dtype=torch.float32, device=gpu) for (W, _, _) in mats]
        ups_got = [torch.full(W.shape, float("nan"), dtype=torch.float32, device=gpu) for (W, _, _) in mats]
        mo.muon_owner_step(ref, update_out=ups_ref, **hp_kwargs(hp))
        assert _noalloc_raw(got, ups_got, hp) == 0
        torch.cuda.synchronize()
        for (W1, _, M1), (W2, _, M2), u1, u2 in zip(ref, got, ups_ref, ups_got):
            assert torch.equal(W1, W2) and torch.equal(M1, M2) and torch.equal(u1, u2)
        k = max(range(len(shapes)), key=lambda i: shapes[i][0] * shapes[i][1])
        print(ns, shapes[k], check_case(cases[k], (to_host(got[k][0]), to_host(got[k][2]),
                                                   to_host(ups_got[k])), hp), flush=True)


def test_noalloc_refuses_a_bucket_beyond_the_array(gpu):
    """8192 x 8192 bf16: X, its two transposes, A and B need 640 MiB > 512 MiB.
    The call fails with MO_ERR_WORKSPACE_TOO_SMALL and touches nothing."""
    import torch
    W = torch.full((8192, 8192), 0.5, dtype=torch.bfloat16, device=gpu)
    G = torch.ones((8192, 8192), dtype=torch.bfloat16, device=gpu)
    M = torch.zeros((8192, 8192), dtype=torch.float32, device=gpu)
    assert mo.muon_workspace_bytes([mo.tensor_descriptor(W, G, M)], mo.hparams()) > mo.NOALLOC_SCRATCH_BYTES
    assert _noalloc_raw([(W, G, M)], [None], BF) == -3
    with pytest.raises(mo.MoError):
        mo.muon_owner_step_noalloc([(W, G, M)], **hp_kwargs(BF))
    torch.cuda.synchronize()
    assert bool((W == 0.5).all()) and bool((M == 0).all())


def test_noalloc_binding_and_stream(gpu):
    """Through the binding, on a side stream: same bits as the workspace path."""
    import torch
    cases, mats = _bucket([(384, 640), (640, 384)], 71, gpu)
    ref, got = _clone(mats), _clone(mats)
    mo.muon_owner_step(ref, **hp_kwargs(BF))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    mo.muon_owner_step_noalloc(got, stream=side, **hp_kwargs(BF))
    torch.cuda.synchronize()
    for (W1, _, M1), (W2, _, M2) in zip(ref, got):
        assert torch.equal(W1, W2) and torch.equal(M1, M2)
