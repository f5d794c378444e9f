"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Sizes here run the oracle in seconds and span several 128-tiles plus ragged
edges; the full-size workloads are covered in test_fullsize_gpu.py.
"""
import dataclasses

import numpy as np
import pytest

from matrix_optimizers_amd import workloads as wlmod
from oracle import adamw as oadamw

from _parity import Case, check_case, hp_kwargs, random_case, rel, run_gpu, to_dev, to_host

pytestmark = pytest.mark.gpu

BF = wlmod.MuonHP()                         # bf16 Newton-Schulz, torch.optim.Muon defaults
F32HP = wlmod.MuonHP(ns_dtype="f32")


def test_single_256x512_f32_workload(gpu):
    """The one-matrix fp32 workload in full: fp32 NS, zero momentum, G ~ N(0, 1)."""
    wl = wlmod.get("single_256x512_f32")
    x = wlmod.matrix_inputs(wl, 0)
    c = Case(x.W, x.G, x.M, wl.w_dtype, wl.g_dtype)
    got = run_gpu([c], wl.hp, gpu)[0]
    errs = check_case(c, got, wl.hp)
    print("single_256x512_f32", errs)


SHAPES = [(1, 1), (1, 300), (300, 1), (33, 17), (17, 33), (100, 257), (257, 100),
          (384, 640), (640, 384), (300, 700), (700, 300), (129, 129)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("ns", ["bf16", "f32"])
def test_ragged_shapes(gpu, shape, ns):
    """Tiny, ragged and multi-tile shapes, tall and wide, both NS precisions."""
    hp = dataclasses.replace(BF, ns_dtype=ns)
    c = random_case(*shape, "bf16" if ns == "bf16" else "f32", "bf16" if ns == "bf16" else "f32",
                    seed=hash(shape) & 0xFFFF)
    errs = check_case(c, run_gpu([c], hp, gpu)[0], hp)
    print(shape, ns, errs)


def test_mixed_bucket_with_empty_shards(gpu):
    """One grouped launch over differently shaped matrices, with empty shards
    (a non-owner's view) that must be skipped."""
    shapes = [(256, 256), (0, 5), (128, 512), (512, 128), (5, 0), (70, 190), (190, 70)]
    cases = [random_case(r, c, "bf16", "bf16", seed=i + 11) for i, (r, c) in enumerate(shapes)]
    got = run_gpu(cases, BF, gpu)
    for c, g in zip(cases, got):
        print(c.W.shape, check_case(c, g, BF))


def test_strided_tensors(gpu):
    """Row strides larger than the row length (views into wider tensors)."""
    cases = [random_case(200, 96, "bf16", "bf16", seed=3), random_case(96, 200, "f32", "bf16", seed=4)]
    got = run_gpu(cases, BF, gpu, strided=True)
    for c, g in zip(cases, got):
        print(c.W.shape, check_case(c, g, BF))


@pytest.mark.parametrize("w_dtype,g_dtype,ns", [("f32", "bf16", "bf16"), ("bf16", "f32", "f32"),
                                                 ("f32", "f32", "bf16"), ("bf16", "bf16", "f32")])
def test_dtype_combinations(gpu, w_dtype, g_dtype, ns):
    hp = dataclasses.replace(BF, ns_dtype=ns)
    c = random_case(160, 416, w_dtype, g_dtype, seed=21)
    print(w_dtype, g_dtype, ns, check_case(c, run_gpu([c], hp, gpu)[0], hp))


@pytest.mark.parametrize("variant", [
    dict(ns_steps=0), dict(ns_steps=1), dict(ns_steps=2, momentum=0.5, lr_adjust="match_rms_adamw"),
    dict(nesterov=False), dict(lr_adjust="none"), dict(lr_adjust="match_rms_adamw"),
    dict(weight_decay=0.0), dict(ns_a=1.5, ns_b=-0.5, ns_c=0.0, ns_steps=8),
])
def test_hyperparameter_variants(gpu, variant):
    hp = dataclasses.replace(BF, **variant)
    cases = [random_case(192, 320, "bf16", "bf16", seed=5), random_case(320, 192, "bf16", "bf16", seed=6)]
    got = run_gpu(cases, hp, gpu)
    for c, g in zip(cases, got):
        print(variant, c.W.shape, check_case(c, g, hp))


def test_zero_gradient_and_eps_clamp(gpu):
    """G = M = 0 gives W' = (1 - lr wd) W exactly; a tiny gradient (||U|| < eps)
    is divided by eps, not by its norm."""
    z = random_case(130, 70, "f32", "f32", seed=8)
    z.G[:] = 0
    z.M[:] = 0
    W1, M1, D1 = run_gpu([z], F32HP, gpu)[0]
    assert not M1.any() and not D1.any()
    decay = np.float32(1 - np.float32(F32HP.lr) * np.float32(F32HP.weight_decay))
    np.testing.assert_allclose(W1, (decay * z.W).astype(np.float64), rtol=1e-7, atol=0)
    tiny = random_case(64, 96, "f32", "f32", seed=9, g_std=1e-12, m_std=0.0)
    print("tiny", check_case(tiny, run_gpu([tiny], F32HP, gpu)[0], F32HP))


def test_without_update_out_is_identical(gpu):
    """The optional update output does not change what is written to W and M."""
    cases = [random_case(200, 520, "bf16", "bf16", seed=12), random_case(520, 200, "bf16", "bf16", seed=13)]
    a = run_gpu(cases, BF, gpu, with_update=True)
    b = run_gpu(cases, BF, gpu, with_update=False)
    for (Wa, Ma, _), (Wb, Mb, _) in zip(a, b):
        np.testing.assert_array_equal(Wa, Wb)
        np.testing.assert_array_equal(Ma, Mb)


def test_deterministic_and_bucket_independent(gpu):
    """Same inputs give bit-identical outputs; a matrix's result does not depend
    on the rest of its bucket."""
    cases = [random_case(256, 768, "bf16", "bf16", seed=14), random_case(384, 128, "bf16", "bf16", seed=15),
             random_case(1000, 300, "bf16", "bf16", seed=16)]
    a = run_gpu(cases, BF, gpu)
    b = run_gpu(cases, BF, gpu)
    alone = run_gpu([cases[1]], BF, gpu)[0]
    for x, y in zip(a, b):
        for u, v in zip(x, y):
            np.testing.assert_array_equal(u, v)
    for u, v in zip(a[1], alone):
        np.testing.assert_array_equal(u, v)


def test_power_of_two_scale_invariance_bit_exact(gpu):
    """NS(alpha X) = NS(X): scaling G and M by 4 scales U, its norm and every
    partial exactly, so the update is bit-identical."""
    c = random_case(384, 640, "f32", "f32", seed=17)
    c4 = Case(c.W.copy(), c.G * 4, c.M * 4, "f32", "f32")
    a = run_gpu([c], BF, gpu)[0]
    b = run_gpu([c4], BF, gpu)[0]
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[2], b[2])


def test_decoder_layer_bucket_full(gpu):
    """The hidden-2048 decoder-layer owner bucket in full (7 matrices) plus its
    AdamW tail."""
    wl = wlmod.get("decoder_layer_h2048")
    cases = []
    for i in range(len(wl.matrices)):
        x = wlmod.matrix_inputs(wl, i)
        cases.append(Case(x.W, x.G, x.M, wl.w_dtype, wl.g_dtype))
    got = run_gpu(cases, wl.hp, gpu)
    for spec, c, g in zip(wl.matrices, cases, got):
        print(spec.name, check_case(c, g, wl.hp))
    check_tail(gpu, wl.seed, wl.tail_numel, wl.adamw)


def check_tail(device, seed, n, a: wlmod.AdamWHP):
    import matrix_optimizers_amd as mo
    t = wlmod.tail_inputs(seed, n)
    p, g, m, v = (to_dev(x, "f32", device) for x in (t.p, t.g, t.m, t.v))
    mo.adamw_tail_step(p, g, m, v, a.step, lr=a.lr, beta1=a.beta1, beta2=a.beta2, eps=a.eps,
                       weight_decay=a.weight_decay)
    f = lambda x: float(np.float32(x))
    po, mo_, vo = oadamw.adamw_step(t.p, t.g, t.m, t.v, a.step, f(a.lr), f(a.beta1), f(a.beta2),
                                    f(a.eps), f(a.weight_decay))
    errs = (rel(to_host(p), po), rel(to_host(m), mo_), rel(to_host(v), vo))
    print("adamw", n, errs)
    assert max(errs) <= 1e-6, errs


# 517 and 2051: a last partial group of 16-byte accesses plus ragged elements;
# 2^25 + 4099: a grid of 16387 workgroups with both.
@pytest.mark.parametrize("n", [0, 1, 3, 4, 517, 1023, 2051, 4096, 32768, 1 << 20, (1 << 25) + 4099])
def test_adamw_tail(gpu, n):
    check_tail(gpu, 40 + n % 7, n, wlmod.AdamWHP())


def test_adamw_tail_beyond_one_pass(gpu):
    """More elements than one pass of the largest grid covers (131072
    workgroups of 2048 elements, 2^28): the first workgroups loop once more,
    one ends in a partial 16-byte group, and the last n % 4 elements take the
    element-wise path.  Inputs are drawn on the device; AdamW is elementwise,
    so the oracle evaluated on sampled elements (both ends, both sides of the
    pass boundary, and random ones), from their inputs as stored, is exact for
    those elements."""
    import torch
    import matrix_optimizers_amd as mo
    n = (1 << 28) + (1 << 20) + 4099
    gen = torch.Generator(device=gpu).manual_seed(71)
    p = torch.randn(n, device=gpu, generator=gen) * 0.02
    g = torch.randn(n, device=gpu, generator=gen) * 1e-3
    m = torch.randn(n, device=gpu, generator=gen) * 1e-3
    v = (torch.randn(n, device=gpu, generator=gen) * 1e-3) ** 2
    edge = 1 << 28
    idx = torch.cat([torch.arange(0, 8192), torch.arange(edge - 8192, edge + 8192), torch.arange(n - 16384, n),
                     torch.randint(0, n, (200000,), generator=torch.Generator().manual_seed(72))]).unique()
    idx_d = idx.to(gpu)
    before = [t[idx_d].double().cpu().numpy() for t in (p, g, m, v)]
    a = wlmod.AdamWHP()
    mo.adamw_tail_step(p, g, m, v, a.step, lr=a.lr, beta1=a.beta1, beta2=a.beta2, eps=a.eps,
                       weight_decay=a.weight_decay)
    after = [t[idx_d].double().cpu().numpy() for t in (p, m, v)]
    f = lambda x: float(np.float32(x))
    want = oadamw.adamw_step(*before, a.step, f(a.lr), f(a.beta1), f(a.beta2), f(a.eps), f(a.weight_decay))
    errs = [rel(x, w) for x, w in zip(after, want)]
    print("adamw beyond one pass", n, len(idx), errs)
    assert max(errs) <= 1e-6, errs


@pytest.mark.parametrize("step", [1, 2, 1000])
def test_adamw_steps(gpu, step):
    check_tail(gpu, 50, 5000, dataclasses.replace(wlmod.AdamWHP(), step=step))


def test_adamw_misaligned_views(gpu):
    """Tail tensors that start 4 bytes off a 16-byte boundary take the scalar path."""
    import torch
    import matrix_optimizers_amd as mo
    n = 1001
    t = wlmod.tail_inputs(60, n)
    bufs = [torch.zeros(n + 1, dtype=torch.float32, device=gpu) for _ in range(4)]
    views = [b[1:] for b in bufs]
    for v_, x in zip(views, (t.p, t.g, t.m, t.v)):
        v_.copy_(torch.from_numpy(x))
    a = wlmod.AdamWHP()
    mo.adamw_tail_step(*views, a.step, lr=a.lr, beta1=a.beta1, beta2=a.beta2, eps=a.eps,
                       weight_decay=a.weight_decay)
    f = lambda x: float(np.float32(x))
    po, _, _ = oadamw.adamw_step(t.p, t.g, t.m, t.v, a.step, f(a.lr), f(a.beta1), f(a.beta2),
                                 f(a.eps), f(a.weight_decay))
    assert rel(to_host(views[0]), po) <= 1e-6


# (2 << 30) + (64 << 20) + 4080: more than one pass of the largest grid (2 GiB)
@pytest.mark.parametrize("nbytes", [16, 48, 4096 + 16, 3 * 4096 * 16 + 1008, (64 << 20) + 4080,
                                    (2 << 30) + (64 << 20) + 4080])
def test_device_copy(gpu, nbytes):
    """The copy that calibrates the byte counters copies every byte, including
    a last partial group of 16-byte accesses and, past 2 GiB, a second pass of
    the grid."""
    import torch
    import matrix_optimizers_amd as mo
    gen = torch.Generator(device=gpu).manual_seed(nbytes % 1000)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=gpu, generator=gen)
    dst = torch.zeros_like(src)
    mo.device_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def _widths(shapes, hp, mat):
    """Tile widths (nb -> count) of matrix `mat` in each phase's dispatch list."""
    import collections
    import matrix_optimizers_amd as mo
    from worklist_cases import parse_worklist
    descs = [mo.descriptor(r, c, W=(1 << 40) + 3 * i * (1 << 34), G=(1 << 40) + (3 * i + 1) * (1 << 34),
                           M=(1 << 40) + (3 * i + 2) * (1 << 34)) for i, (r, c) in enumerate(shapes)]
    wl = mo.build_worklist(descs, mo.hparams(**hp_kwargs(hp)))
    _, lists = parse_worklist(wl)
    return [dict(collections.Counter(nb for m, _, _, nb in items if m == mat)) for items in lists]


@pytest.mark.parametrize("shape,count,in_bucket,alone", [
    ((1024, 1024), 30, [{4: 10}, {4: 10}, {4: 16}], [{2: 20}, {2: 20}, {2: 32}]),
    ((3072, 1024), 12, [{2: 20}, {2: 20}, {4: 48}], [{2: 20}, {2: 20}, {2: 96}]),
])
def test_tile_widths_give_bit_identical_results(gpu, shape, count, in_bucket, alone):
    """Where full tiles would leave CUs idle the host splits them into half
    widths.  Matrix 0 runs at full width inside a large bucket (or half, for
    the Gram and Poly of the tall case) and at half width alone; every output
    element is summed over the same K in the same order either way, so the
    results are bit-identical."""
    assert _widths([shape] * count, BF, 0) == in_bucket
    assert _widths([shape], BF, 0) == alone
    cases = [random_case(shape[0], shape[1], "bf16", "bf16", seed=70 + i) for i in range(count)]
    a = run_gpu(cases, BF, gpu)[0]
    b = run_gpu([cases[0]], BF, gpu)[0]
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    print(shape, check_case(cases[0], b, BF))


@pytest.mark.parametrize("ns", ["bf16", "f32"])
def test_half_width_tiles_parity(gpu, ns):
    """Eight 1024 x 1024 matrices: every phase runs half-width tiles."""
    hp = dataclasses.replace(BF, ns_dtype=ns)
    assert _widths([(1024, 1024)] * 8, hp, 3) == [{2: 20}, {2: 20}, {2: 32}]
    cases = [random_case(1024, 1024, "bf16", "bf16", seed=90 + i) for i in range(8)]
    got = run_gpu(cases, hp, gpu)
    for k in (0, 5):
        print(ns, k, check_case(cases[k], got[k], hp))


@pytest.mark.parametrize("ns", ["bf16", "f32"])
def test_two_consecutive_steps_carry_state(gpu, ns):
    """Two consecutive owner steps on one bucket, carrying W and M between them
    ([P §3], [P §4.4]: the owner keeps its Muon state from step to step), against
    two chained oracle steps.  Step 2's update and momentum are compared with
    the oracle's own second step; the written weights with decay W1 - delta2 of
    the GPU's own W1.  Then the second step is run again from a saved copy of
    the state after step 1, on a fresh workspace: it must give the same bits
    as the consecutive run (a saved and restored state is the same state)."""
    import torch
    import matrix_optimizers_amd as mo
    from _parity import hp_f32, bf16_ulp
    from oracle import muon as omuon
    hp = dataclasses.replace(BF, ns_dtype=ns)
    wd = "bf16" if ns == "bf16" else "f32"
    shapes = [(192, 320), (320, 192), (256, 256)]
    cases = [random_case(r, c, wd, wd, seed=40 + i) for i, (r, c) in enumerate(shapes)]
    g2s = [random_case(r, c, wd, wd, seed=80 + i).G for i, (r, c) in enumerate(shapes)]
    mats = [(to_dev(c.W, wd, gpu), to_dev(c.G, wd, gpu), to_dev(c.M, "f32", gpu)) for c in cases]
    ups = [torch.empty(W.shape, dtype=torch.float32, device=gpu) for (W, _, _) in mats]
    mo.muon_owner_step(mats, update_out=ups, **hp_kwargs(hp))
    # step 2: new gradients, the state carried in place
    mats2 = [(W, to_dev(g2, wd, gpu), M) for (W, _, M), g2 in zip(mats, g2s)]
    saved = [(W.clone(), M.clone()) for (W, _, M) in mats2]
    mo.muon_owner_step(mats2, update_out=ups, **hp_kwargs(hp))
    torch.cuda.synchronize()
    hpo = hp_f32(hp)
    tol = 3e-2 if ns == "bf16" else 1e-4
    for c, g2, (W2, _, M2), U2, (W1s, _) in zip(cases, g2s, mats2, ups, saved):
        W1o, M1o, _ = omuon.muon_step(c.W, c.G, c.M, hpo)
        _, M2o, D2o = omuon.muon_step(W1o, g2.astype(np.float64), M1o, hpo)
        e_d, e_m = rel(to_host(U2), D2o), rel(to_host(M2), M2o)
        decay = np.float32(1.0 - np.float64(np.float32(hp.lr)) * np.float64(np.float32(hp.weight_decay)))
        want = (decay * to_host(W1s).astype(np.float32) - to_host(U2).astype(np.float32)).astype(np.float64)
        got = to_host(W2)
        if wd == "bf16":
            # one bf16 spacing plus the fp32 rounding of the two operands, as in
            # check_case (the operands can cancel)
            op = np.maximum(np.abs(np.float64(decay) * to_host(W1s)), np.abs(to_host(U2)))
            allow = bf16_ulp(np.maximum(np.abs(got), np.abs(want))) + 4 * 2.0 ** -24 * op
            w_err = float((np.abs(got - want) / allow).max())
            assert w_err <= 1.0, w_err
        else:
            w_err = rel(got, want)
            assert w_err <= 1e-6, w_err
        print(c.W.shape, ns, f"step-2 delta {e_d:.2e} momentum {e_m:.2e} weights {w_err:.2e}")
        assert e_d <= tol and e_m <= 1e-6
    # the second step again, from the saved state, on a fresh workspace
    mats3 = [(W1s.clone(), G2, M1s.clone()) for (W1s, M1s), (_, G2, _) in zip(saved, mats2)]
    ups3 = [torch.empty_like(u) for u in ups]
    mo.muon_owner_step(mats3, update_out=ups3, **hp_kwargs(hp))
    torch.cuda.synchronize()
    for (W2, _, M2), (W3, _, M3), u2, u3 in zip(mats2, mats3, ups, ups3):
        assert torch.equal(W2, W3) and torch.equal(M2, M3) and torch.equal(u2, u3)
