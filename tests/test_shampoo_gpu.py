"""GPU parity of the Shampoo owner step (C ABI, HIP kernels) against the fp64
oracle in oracle/shampoo.py, on seeded synthetic inputs.

Tolerances (relative Frobenius norm), fp32 throughout:
  * the update lr H_L G H_R: 1e-4 (the fp32 bar; a numpy fp32 run of the same
    iteration lands at 5e-6 .. 4e-5 on these condition numbers);
  * the statistics L', R': 1e-6 (one fp32 dot product per entry); sampled
    entries at full size: 4 sqrt(K) u sum |a_k b_k| each;
  * the written weight: decay W - delta_gpu rounded to W's dtype (1e-6 for
    fp32, one bf16 spacing plus operand rounding for bf16).
"""
import numpy as np
import pytest

import matrix_optimizers_amd as mo
from matrix_optimizers_amd import workloads as wlmod
from oracle import shampoo as osh
from shampoo_ref import svd_route_update

pytestmark = pytest.mark.gpu

TOL_U, TOL_STATS, TOL_W = 1e-4, 1e-6, 1e-6


def rel(a, b):
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / den if den > 0 else float(np.linalg.norm(a - b))


def f32(x):
    return float(np.float32(x))


def to_dev(x, dtype, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run(cases, hp, device, steps=1, strided=False, with_update=True):
    """cases: [(W, G, L, R, w_dtype, g_dtype)] host arrays; returns per case the
    host (W', L', R', delta) after `steps` steps with the same G."""
    import torch
    mats, ups, keep = [], [], []
    for W, G, L, R, wd, gd in cases:
        if strided and W.size:
            def view(x, dt, off):
                big = torch.zeros((x.shape[0], x.shape[1] + 24), dtype=to_dev(x[:1, :1], dt, device).dtype,
                                  device=device)
                v = big[:, off:off + x.shape[1]]
                v.copy_(to_dev(x, dt, device))
                keep.append(big)
                return v
            t = (view(W, wd, 3), view(G, gd, 5), view(L, "f32", 1), view(R, "f32", 7))
        else:
            t = (to_dev(W, wd, device), to_dev(G, gd, device), to_dev(L, "f32", device),
                 to_dev(R, "f32", device))
        mats.append(t)
        ups.append(torch.full(W.shape, float("nan"), dtype=torch.float32, device=device)
                   if with_update else None)
    for _ in range(steps):
        mo.shampoo_owner_step(mats, update_out=ups if with_update else None, lr=hp.lr,
                              weight_decay=hp.weight_decay, root_iters=hp.root_iters)
    torch.cuda.synchronize()
    return [tuple(to_host(x) for x in (m[0], m[2], m[3])) + ((to_host(u) if u is not None else None),)
            for m, u in zip(mats, ups)]


def check(case, got, hp, steps=1):
    W, G, L, R, wd, gd = case
    W1, L1, R1, D1 = got
    lr, wdec = f32(hp.lr), f32(hp.weight_decay)
    Wo, Lo, Ro = W.astype(np.float64), L.astype(np.float64), R.astype(np.float64)
    for _ in range(steps):
        Wo, Lo, Ro, Do = osh.shampoo_step(Wo, G.astype(np.float64), Lo, Ro, lr, wdec, "newton", hp.root_iters)
    out = {"L": rel(L1, Lo), "R": rel(R1, Ro)}
    assert out["L"] <= TOL_STATS and out["R"] <= TOL_STATS, out
    if D1 is not None:
        out["delta"] = rel(D1, Do)
        assert out["delta"] <= TOL_U, out
        if steps == 1:
            decay = np.float32(1.0 - np.float64(lr) * np.float64(wdec))
            want = (decay * W.astype(np.float32) - D1.astype(np.float32)).astype(np.float64)
            if wd == "bf16":
                ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
                allow = ulp + 4 * 2.0 ** -24 * np.maximum(np.abs(W), np.abs(D1))
                assert float((np.abs(W1 - want) / allow).max()) <= 1.0
            else:
                out["W"] = rel(W1, want)
                assert out["W"] <= TOL_W, out
    return out


def workload_cases(wl):
    return [wlmod.shampoo_inputs(wl, i) + (wl.w_dtype, wl.g_dtype) for i in range(len(wl.matrices))]


def test_mixed_small_bucket(gpu):
    """Five ragged fp32 matrices in one bucket (tails of tiles, a single row, a
    side of 1000 = 3 tiles + 232)."""
    wl = wlmod.SHAMPOO_WORKLOADS["shampoo_mixed_small"]
    cases = workload_cases(wl)
    got = run(cases, wl.hp, gpu)
    for c, g in zip(cases, got):
        print(c[0].shape, check(c, g, wl.hp))


@pytest.mark.parametrize("iters", [1, 2, 3, 7])
def test_root_iteration_counts(gpu, iters):
    """K = 1 (no product), 2 (the last H only), 3 and 7 coupled Newton steps."""
    wl = wlmod.SHAMPOO_WORKLOADS["shampoo_mixed_small"]
    hp = wlmod.ShampooHP(root_iters=iters)
    cases = [workload_cases(wl)[1], workload_cases(wl)[3]]
    for c, g in zip(cases, run(cases, hp, gpu)):
        print(iters, c[0].shape, check(c, g, hp))


def test_two_steps_accumulate(gpu):
    """The statistics carry over: the second step preconditions with
    eps I + 2 G G^T (the same G twice) and writes W twice."""
    wl = wlmod.SHAMPOO_WORKLOADS["shampoo_mixed_small"]
    hp = wlmod.ShampooHP(weight_decay=0.1)
    cases = [workload_cases(wl)[0], workload_cases(wl)[2]]
    for c, g in zip(cases, run(cases, hp, gpu, steps=2)):
        print(c[0].shape, check(c, g, hp, steps=2))


def test_bf16_strided_empty_and_no_update(gpu):
    """bf16 W and G, strided storage of every tensor, an empty shard in the
    bucket, and a matrix without update_out."""
    hp = wlmod.ShampooHP(weight_decay=0.05)
    rng = np.random.default_rng(5)
    def case(r, c, wd, gd):
        W = wlmod.store(rng.standard_normal((r, c)) * 0.02, wd)
        G = wlmod.store(rng.standard_normal((r, c)) * 1e-3, gd)
        return (W, G, (hp.eps * np.eye(r)).astype(np.float32), (hp.eps * np.eye(c)).astype(np.float32), wd, gd)
    cases = [case(260, 300, "bf16", "bf16"), case(128, 520, "f32", "bf16"), case(500, 64, "bf16", "f32")]
    got = run(cases, hp, gpu, strided=True)
    for c, g in zip(cases, got):
        print(c[0].shape, check(c, g, hp))
    # without update_out the weight is written bit-identically
    again = run(cases, hp, gpu, strided=True, with_update=False)
    for g, a in zip(got, again):
        assert np.array_equal(g[0], a[0])
    import torch
    e = [(torch.zeros((0, 5), device=gpu), torch.zeros((0, 5), device=gpu), torch.zeros((0, 0), device=gpu),
          torch.zeros((5, 5), device=gpu))]
    W, G, L, R, _, _ = cases[1]
    dev = [to_dev(x, "f32", gpu) for x in (W, G, L, R)]
    mo.shampoo_owner_step(e + [tuple(dev)], lr=hp.lr, weight_decay=hp.weight_decay, root_iters=hp.root_iters)
    torch.cuda.synchronize()
    Wo, _, _, _ = osh.shampoo_step(W, G, L, R, f32(hp.lr), f32(hp.weight_decay), "newton", hp.root_iters)
    assert rel(to_host(dev[0]) - W, Wo - W) <= TOL_U


def test_decoder_layer_full_size(gpu):
    """The bench's bucket (hidden 2048, FFN 5632) in the bench's launch
    configuration: every matrix's update against the SVD route of the oracle,
    and sampled statistics entries as fp64 dot products."""
    import torch
    wl = wlmod.SHAMPOO_WORKLOADS["shampoo_decoder_layer_h2048"]
    hp = wl.hp
    host = [wlmod.shampoo_inputs(wl, i) for i in range(len(wl.matrices))]
    mats = [tuple(to_dev(x, "f32", gpu) for x in h) for h in host]
    ups = [torch.empty(h[0].shape, dtype=torch.float32, device=gpu) for h in host]
    step = mo.ShampooOwnerStep(mats, update_out=ups, lr=hp.lr, weight_decay=hp.weight_decay,
                               root_iters=hp.root_iters)
    step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    for (W, G, L, R), (_, _, Ld, Rd), U, spec in zip(host, mats, ups, wl.matrices):
        G64 = G.astype(np.float64)
        for S, n, M in ((Ld, G.shape[0], G64), (Rd, G.shape[1], G64.T)):
            # 64 random entries and 16 diagonal ones.  An fp32 dot product of
            # length K has a rounding error of about lambda sqrt(K) u sum |a_k b_k|
            # (u = 2^-24; the probabilistic bound of Higham and Mary, 2019),
            # lambda = 4 here; the diagonal, a sum of positive terms, is where
            # it is reached.
            idx = rng.integers(0, n, size=(80, 2))
            idx[64:, 1] = idx[64:, 0]
            got = S[idx[:, 0], idx[:, 1]].cpu().numpy().astype(np.float64)
            a, b = M[idx[:, 0]], M[idx[:, 1]]
            want = np.einsum("ij,ij->i", a, b) + np.float32(hp.eps) * (idx[:, 0] == idx[:, 1])
            scale = np.einsum("ij,ij->i", np.abs(a), np.abs(b)) + np.float32(hp.eps) * (idx[:, 0] == idx[:, 1])
            bound = 4 * np.sqrt(M.shape[1]) * 2.0 ** -24 * scale
            worst = float(np.max(np.abs(got - want) / bound))
            assert worst <= 1.0, (spec.name, worst)
        d = rel(to_host(U) / f32(hp.lr), svd_route_update(G64, f32(hp.eps), hp.root_iters))
        print(spec.name, spec.rows, spec.cols, "delta rel", d)
        assert d <= TOL_U, spec


def test_paper_layer_full_size(gpu):
    """One layer of the paper's model (roots of side 4096 and 16384): sampled
    statistics entries of every matrix, a finite update everywhere, and the
    first 4096 x 4096 matrix's update against the SVD route."""
    import torch
    wl = wlmod.SHAMPOO_WORKLOADS["shampoo_paper_layer"]
    hp = wl.hp
    host = [wlmod.shampoo_inputs(wl, i) for i in range(len(wl.matrices))]
    mats = [tuple(to_dev(x, "f32", gpu) for x in h) for h in host]
    ups = [torch.empty(h[0].shape, dtype=torch.float32, device=gpu) for h in host]
    mo.shampoo_owner_step(mats, update_out=ups, lr=hp.lr, weight_decay=hp.weight_decay, root_iters=hp.root_iters)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    for (W, G, L, R), (_, _, Ld, Rd), U, spec in zip(host, mats, ups, wl.matrices):
        assert bool(torch.isfinite(U).all()), spec.name
        G64 = G.astype(np.float64)
        for S, n, M in ((Ld, G.shape[0], G64), (Rd, G.shape[1], G64.T)):
            idx = rng.integers(0, n, size=(48, 2))
            idx[32:, 1] = idx[32:, 0]
            got = S[idx[:, 0], idx[:, 1]].cpu().numpy().astype(np.float64)
            a, b = M[idx[:, 0]], M[idx[:, 1]]
            diag = np.float32(hp.eps) * (idx[:, 0] == idx[:, 1])
            want = np.einsum("ij,ij->i", a, b) + diag
            scale = np.einsum("ij,ij->i", np.abs(a), np.abs(b)) + diag
            assert np.all(np.abs(got - want) <= 4 * np.sqrt(M.shape[1]) * 2.0 ** -24 * scale), spec.name
    d = rel(to_host(ups[0]) / f32(hp.lr), svd_route_update(host[0][1].astype(np.float64), f32(hp.eps), hp.root_iters))
    print("q 4096 x 4096 delta rel", d)
    assert d <= TOL_U
