"""SOAP owner step on the GPU (soap_owner_step through the C ABI) against the
fp64 oracle (oracle/soap.py), on the same stored inputs.

Tolerance.  The step stores fp32 and accumulates its products in fp64; its
eigensolver is fp64.  Its update
depends on the eigenvectors of the fp32 statistics, and where two eigenvalues
are closer than the fp32 rounding of L' or R' can separate, the fp32
statistics alone move those eigenvectors: the error of an fp32 step has a
floor set by the conditioning of each input, not by the implementation.  The
test measures that floor on the same stored inputs with a plain fp32 model of
the step whose eigenvectors are exact (numpy's fp64 eigh of the fp32
statistics, rounded once), and requires the GPU update within
max(1e-4, 4 x floor) relative Frobenius of the oracle's; on most draws the
floor is 2e-6 .. 2e-5, so the bar is the 1e-4 of the fp32 Muon path.  The
statistics and the first moment are plain fp32 sums (1e-6); the warm second
moment is dominated by b2 V (1e-6), the first one is (1 - b2) G~^2 (twice the
update's bar).

Workload: warm states (statistics summed over ten earlier gradients, M and V
drawn as state, t = 10), where the step is well posed in fp32 (every shape
keeps both statistics of full rank: a repeated eigenvalue with non-zero
moments in its eigenspace would make the update depend on the basis chosen
inside it); and a first
step from zero moments with an Adam eps of 1e-3 (with a small eps the first
step is a sign function of the rotated gradient, whose fp32 rounding of
exactly-zero entries no fp32 implementation reproduces).
"""
import numpy as np
import pytest

from oracle import soap as osoap

pytestmark = pytest.mark.gpu

F32 = np.float32


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def seeded(seed, *key):
    return np.random.default_rng(np.random.SeedSequence([seed, *key]))


def warm_state(seed, r, c, history=10):
    """Stored (fp32-rounded) inputs of one warm matrix, as fp64 arrays."""
    rng = seeded(seed, r, c)
    q = lambda x: np.asarray(x, F32).astype(np.float64)
    W = q(rng.normal(0, 0.02, (r, c)))
    G = q(rng.normal(0, 1e-3, (r, c)))
    L = 1e-6 * np.eye(r)
    R = 1e-6 * np.eye(c)
    for _ in range(history):
        Gp = rng.normal(0, 1e-3, (r, c))
        L += Gp @ Gp.T
        R += Gp.T @ Gp
    M = q(rng.normal(0, 1e-3, (r, c)))
    V = q(rng.normal(0, 1e-3, (r, c)) ** 2)
    return dict(W=W, G=G, L=q(L), R=q(R), M=M, V=V)


def first_state(seed, r, c, eps_stat=1e-6):
    rng = seeded(seed, r, c, 1)
    q = lambda x: np.asarray(x, F32).astype(np.float64)
    return dict(W=q(rng.normal(0, 0.02, (r, c))), G=q(rng.normal(0, 1e-3, (r, c))),
                L=q(eps_stat * np.eye(r)), R=q(eps_stat * np.eye(c)), M=np.zeros((r, c)), V=np.zeros((r, c)))


def fp32_floor(st, step, hp):
    """Relative error of an fp32 step whose eigenvectors are exact (rounded once)."""
    G = st["G"].astype(F32)
    L1 = st["L"].astype(F32) + G @ G.T
    R1 = st["R"].astype(F32) + G.T @ G
    EL = np.linalg.eigh(L1.astype(np.float64))[1].T.astype(F32)
    ER = np.linalg.eigh(R1.astype(np.float64))[1].T.astype(F32)
    b1, b2 = F32(hp["beta1"]), F32(hp["beta2"])
    M1 = b1 * st["M"].astype(F32) + (F32(1) - b1) * G
    Gr = EL @ G @ ER.T
    Mr = EL @ M1 @ ER.T
    V1 = b2 * st["V"].astype(F32) + (F32(1) - b2) * Gr * Gr
    N = (Mr / F32(1 - hp["beta1"] ** step)) / (np.sqrt(V1 / F32(1 - hp["beta2"] ** step)) + F32(hp["eps"]))
    return F32(hp["lr"]) * (EL.T @ N @ ER)


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def run_gpu(states, step, hp, w_dtype="f32", g_dtype="f32", sweeps=14):
    import torch
    import matrix_optimizers_amd as mo
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    dev = torch.device("cuda:0")
    mats, ups = [], []
    for st in states:
        t = lambda x, d=torch.float32: torch.tensor(np.asarray(x, F32), device=dev).to(d).contiguous()
        mats.append((t(st["W"], dt[w_dtype]), t(st["G"], dt[g_dtype]), t(st["L"]), t(st["R"]), t(st["M"]),
                     t(st["V"])))
        ups.append(torch.empty(st["W"].shape, dtype=torch.float32, device=dev))
    mo.soap_owner_step(mats, update_out=ups, step=step, sweeps=sweeps, **hp)
    torch.cuda.synchronize()
    to = lambda x: x.float().cpu().numpy().astype(np.float64)
    return [dict(W=to(m[0]), L=to(m[2]), R=to(m[3]), M=to(m[4]), V=to(m[5]), U=to(u)) for m, u in zip(mats, ups)]


def check(st, out, step, hp, label):
    W1, L1, R1, M1, V1, D = osoap.soap_step(st["W"], st["G"], st["L"], st["R"], st["M"], st["V"], step,
                                            hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    floor = rel(fp32_floor(st, step, hp), D)
    tol = max(1e-4, 4 * floor)
    err = rel(out["U"], D)
    print(f"{label}: update {err:.2e} (fp32 floor {floor:.2e}, tol {tol:.2e}); "
          f"L {rel(out['L'], L1):.1e} R {rel(out['R'], R1):.1e} M {rel(out['M'], M1):.1e} "
          f"V {rel(out['V'], V1):.1e}", flush=True)
    assert np.all(np.isfinite(out["U"]))
    assert err <= tol
    assert rel(out["L"], L1) <= 1e-6 and rel(out["R"], R1) <= 1e-6
    assert rel(out["M"], M1) <= 1e-6
    # V' = b2 V + (1 - b2) G~^2: near b2 V's rounding when V is warm; from V = 0
    # it carries twice the relative error of the rotated gradient, which is of
    # the update's kind
    assert rel(out["V"], V1) <= max(1e-6, 2 * tol)
    # W' = (1 - lr wd) W - update, in fp32
    decay = F32(1 - hp["lr"] * hp["weight_decay"])
    Wexp = (decay * st["W"].astype(F32) - out["U"].astype(F32)).astype(np.float64)
    assert np.max(np.abs(out["W"] - Wexp)) <= 4 * np.finfo(F32).eps * np.max(np.abs(Wexp))


@pytest.mark.parametrize("shape", [(96, 160), (200, 136), (64, 64), (2, 16), (33, 5)])
def test_warm_step(gpu, shape):
    st = warm_state(11, *shape)
    out = run_gpu([st], 10, HP)[0]
    check(st, out, 10, HP, f"warm {shape}")


@pytest.mark.parametrize("log2s", [40, -40])
def test_statistics_scale(gpu, log2s):
    """The eigensolver's rotations hold far from fp64's range ends: a gradient
    scaled by s (moments and Adam eps with it, statistics by s^2) gives, in
    exact arithmetic, the same update; the step must match the oracle there as
    at unit scale, and the scaled update must equal the unscaled one to the bar."""
    s = 2.0 ** log2s
    base = warm_state(23, 96, 160)
    st = dict(base, G=base["G"] * s, M=base["M"] * s, L=base["L"] * s * s, R=base["R"] * s * s,
              V=base["V"] * s * s)
    hp = dict(HP, eps=HP["eps"] * s)
    out, ref = run_gpu([st], 10, hp)[0], run_gpu([base], 10, HP)[0]
    check(st, out, 10, hp, f"scale 2^{log2s}")
    assert rel(out["U"], ref["U"]) <= 2e-4


def test_mixed_bucket_with_empty_shard(gpu):
    """One launch sequence over several shapes; each matrix's result is the one
    it gets alone (rows = 0 marks a skipped shard)."""
    import torch
    import matrix_optimizers_amd as mo
    shapes = [(128, 192), (70, 130), (256, 64)]
    states = [warm_state(21, *s) for s in shapes]
    outs = run_gpu(states, 10, HP)
    for s, st, out in zip(shapes, states, outs):
        check(st, out, 10, HP, f"bucket {s}")
    alone = run_gpu([states[1]], 10, HP)[0]
    assert np.array_equal(alone["U"], outs[1]["U"])
    # an empty shard in the descriptor list changes nothing
    dev = torch.device("cuda:0")
    e = torch.empty((0, 5), device=dev)
    mo.soap_owner_step([(e, e, torch.empty((0, 0), device=dev), torch.empty((5, 5), device=dev), e, e)],
                       step=1, **HP)
    torch.cuda.synchronize()


def test_first_step_large_eps(gpu):
    hp = dict(HP, eps=1e-3)
    st = first_state(31, 120, 200)
    out = run_gpu([st], 1, hp)[0]
    check(st, out, 1, hp, "first step (eps 1e-3)")


def test_bf16_weight_and_gradient(gpu):
    st = warm_state(41, 96, 160)
    q = lambda x: np.asarray(x, np.float64)
    import torch
    bf = lambda a: torch.tensor(np.asarray(a, F32)).to(torch.bfloat16).float().numpy().astype(np.float64)
    st = dict(st, W=bf(st["W"]), G=bf(st["G"]))
    out = run_gpu([st], 10, HP, w_dtype="bf16", g_dtype="bf16")[0]
    W1, L1, R1, M1, V1, D = osoap.soap_step(st["W"], st["G"], st["L"], st["R"], st["M"], st["V"], 10,
                                            HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
    floor = rel(fp32_floor(st, 10, HP), D)
    assert rel(out["U"], D) <= max(1e-4, 4 * floor)
    # W' is rounded once into bf16: within half a bf16 unit of decay W - update
    Wexp = (1 - HP["lr"] * HP["weight_decay"]) * st["W"] - out["U"]
    assert np.all(np.abs(out["W"] - Wexp) <= 2.0 ** -8 * np.abs(Wexp) + 1e-30)
    assert q(out["M"]).shape == st["M"].shape


def test_two_steps_carry_state(gpu):
    """The state written by one call is the input of the next."""
    import torch
    import matrix_optimizers_amd as mo
    st = warm_state(51, 80, 144)
    rng = seeded(51, 2)
    G2 = np.asarray(rng.normal(0, 1e-3, st["G"].shape), F32).astype(np.float64)
    dev = torch.device("cuda:0")
    t = lambda x: torch.tensor(np.asarray(x, F32), device=dev).contiguous()
    W, G, L, R, M, V = (t(st[k]) for k in ("W", "G", "L", "R", "M", "V"))
    U = torch.empty_like(W)
    step = mo.SoapOwnerStep([(W, G, L, R, M, V)], update_out=[U], sweeps=14, **HP)
    step(10)
    G.copy_(t(G2))
    step(11)
    torch.cuda.synchronize()
    o1 = osoap.soap_step(st["W"], st["G"], st["L"], st["R"], st["M"], st["V"], 10, HP["lr"], HP["beta1"],
                         HP["beta2"], HP["eps"], HP["weight_decay"])
    o2 = osoap.soap_step(o1[0], G2, o1[1], o1[2], o1[3], o1[4], 11, HP["lr"], HP["beta1"], HP["beta2"],
                         HP["eps"], HP["weight_decay"])
    err = rel(U.cpu().numpy(), o2[5])
    st2 = dict(W=o1[0], G=G2, L=o1[1], R=o1[2], M=o1[3], V=o1[4])
    floor = rel(fp32_floor(st2, 11, HP), o2[5])
    print(f"two steps: update {err:.2e} (fp32 floor of the second step {floor:.2e})", flush=True)
    # the second step also carries the first step's fp32 state
    assert err <= max(2e-4, 8 * floor)
    assert rel(L.cpu().numpy(), o2[1]) <= 1e-6


def test_chained_steps_stay_at_the_floor(gpu):
    """Six chained steps on a ragged shape, a fresh gradient each time: every
    step's update stays within the bar of its own fp32 floor against the fp64
    oracle chained on its own state, so nothing builds up across steps (the
    eigenvectors are recomputed each step, E accumulated in fp32 within it)."""
    import torch
    import matrix_optimizers_amd as mo
    st = warm_state(71, 130, 200)
    dev = torch.device("cuda:0")
    t = lambda x: torch.tensor(np.asarray(x, F32), device=dev).contiguous()
    W, G, L, R, M, V = (t(st[k]) for k in ("W", "G", "L", "R", "M", "V"))
    U = torch.empty_like(W)
    step = mo.SoapOwnerStep([(W, G, L, R, M, V)], update_out=[U], sweeps=14, **HP)
    ref = dict(st)
    errs = []
    for k in range(6):
        if k:
            rng = seeded(71, 3 + k)
            ref["G"] = np.asarray(rng.normal(0, 1e-3, st["G"].shape), F32).astype(np.float64)
            G.copy_(t(ref["G"]))
        step(10 + k)
        torch.cuda.synchronize()
        o = osoap.soap_step(ref["W"], ref["G"], ref["L"], ref["R"], ref["M"], ref["V"], 10 + k, HP["lr"],
                            HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
        floor = rel(fp32_floor(ref, 10 + k, HP), o[5])
        err = rel(U.cpu().numpy(), o[5])
        errs.append(err)
        print(f"chained step {k}: update {err:.2e} (fp32 floor {floor:.2e})", flush=True)
        assert err <= max(2e-4, 8 * floor)
        ref = dict(W=o[0], G=ref["G"], L=o[1], R=o[2], M=o[3], V=o[4])
    assert rel(L.cpu().numpy(), ref["L"]) <= 1e-6 and rel(R.cpu().numpy(), ref["R"]) <= 1e-6


def test_warm_start_chained_steps(gpu):
    """Steps after the first start the eigensolver from the previous step's
    bases: six chained steps on a ragged shape, every one within the bar of
    its own fp32 floor against the fp64 oracle (which recomputes each
    eigendecomposition from scratch), and every step converged."""
    import torch
    import matrix_optimizers_amd as mo
    st = warm_state(73, 130, 200)
    dev = torch.device("cuda:0")
    t = lambda x: torch.tensor(np.asarray(x, F32), device=dev).contiguous()
    W, G, L, R, M, V = (t(st[k]) for k in ("W", "G", "L", "R", "M", "V"))
    U = torch.empty_like(W)
    step = mo.SoapOwnerStep([(W, G, L, R, M, V)], update_out=[U], warm_start=True, sweeps=14, **HP)
    ref = dict(st)
    for k in range(6):
        if k:
            rng = seeded(73, 3 + k)
            ref["G"] = np.asarray(rng.normal(0, 1e-3, st["G"].shape), F32).astype(np.float64)
            G.copy_(t(ref["G"]))
        step(10 + k)
        assert step.hp.warm_start == (1 if k else 0)
        torch.cuda.synchronize()
        o = osoap.soap_step(ref["W"], ref["G"], ref["L"], ref["R"], ref["M"], ref["V"], 10 + k, HP["lr"],
                            HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
        floor = rel(fp32_floor(ref, 10 + k, HP), o[5])
        err = rel(U.cpu().numpy(), o[5])
        print(f"warm chained step {k}: update {err:.2e} (fp32 floor {floor:.2e})", flush=True)
        assert err <= max(2e-4, 8 * floor)
        assert step.rotating_pairs() == [(0, 0)]
        ref = dict(W=o[0], G=ref["G"], L=o[1], R=o[2], M=o[3], V=o[4])


def test_warm_start_full_size(gpu):
    """A 2048 x 2048 and a 5632 x 2048 matrix of the decoder-layer shapes: a
    cold step, then a warm one on a fresh gradient, the warm step against the
    oracle on the state the cold one left, at its fp32 floor; both converged."""
    import torch
    import matrix_optimizers_amd as mo
    dev = torch.device("cuda:0")
    mats = []
    for i, (r, c) in enumerate(((2048, 2048), (5632, 2048))):
        gen = torch.Generator(device=dev)
        gen.manual_seed(7100 + i)
        rnd = lambda std: torch.randn((r, c), device=dev, generator=gen) * std
        W, G = rnd(0.02), rnd(1e-3)
        L = torch.eye(r, device=dev) * 1e-6
        R = torch.eye(c, device=dev) * 1e-6
        for _ in range(10):
            Gp = rnd(1e-3)
            L += Gp @ Gp.T
            R += Gp.T @ Gp
        mats.append((W, G, L, R, rnd(1e-3), rnd(1e-3) ** 2))
    ups = [torch.empty_like(m[0]) for m in mats]
    hp = dict(HP, weight_decay=0.01)
    step = mo.SoapOwnerStep(mats, update_out=ups, warm_start=True, sweeps=14, **hp)
    step(10)
    assert step.rotating_pairs() == [(0, 0), (0, 0)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(7200)
    for m in mats:
        m[1].copy_(torch.randn(m[1].shape, device=dev, generator=gen) * 1e-3)
    torch.cuda.synchronize()
    host = [{k: m[j].double().cpu().numpy() for j, k in enumerate(("W", "G", "L", "R", "M", "V"))}
            for m in mats]
    step(11)
    assert step.hp.warm_start == 1
    assert step.rotating_pairs() == [(0, 0), (0, 0)]
    for i, label in enumerate(("warm 2048x2048", "warm 5632x2048")):
        out = {k: mats[i][j].double().cpu().numpy() for j, k in enumerate(("W", "G", "L", "R", "M", "V"))}
        out["U"] = ups[i].double().cpu().numpy()
        check(host[i], out, 11, hp, label)


def test_warm_start_without_previous_bases(gpu):
    """warm_start=1 on a workspace that never held this bucket's bases (bytes
    of 0xFF) runs cold; on one holding another matrix's bases of the same
    size, those orthonormal bases are a valid start too; on one holding the
    bases of a smaller matrix whose sides pad to the same sizes (so the same
    workspace layout), those lack directions and the step runs cold.  All
    match the oracle at the floor and converge."""
    import torch
    import matrix_optimizers_amd as mo
    dev = torch.device("cuda:0")
    t = lambda x: torch.tensor(np.asarray(x, F32), device=dev).contiguous()
    st = warm_state(77, 150, 90)
    other = warm_state(78, 150, 90)
    smaller = warm_state(79, 140, 70)   # sides 140 and 70 pad to 192 and 128, as 150 and 90 do

    def mats_of(s):
        return [tuple(t(s[k]) for k in ("W", "G", "L", "R", "M", "V"))]
    ref = mats_of(st)
    need = mo.soap_workspace_bytes([mo.soap_tensor_descriptor(*ref[0])], mo.soap_hparams())
    for label, prev in (("fresh workspace", None), ("another matrix's bases", other),
                        ("a smaller matrix's bases", smaller)):
        if prev is None:
            ws = torch.full((need,), 255, dtype=torch.uint8, device=dev)
        else:
            pmats = mats_of(prev)
            assert mo.soap_workspace_bytes([mo.soap_tensor_descriptor(*pmats[0])], mo.soap_hparams()) == need
            ostep = mo.SoapOwnerStep(pmats, sweeps=14, **HP)
            ostep(10)
            ws = ostep.workspace
        mats = mats_of(st)
        U = torch.empty_like(mats[0][0])
        mo.soap_owner_step(mats, update_out=[U], workspace=ws, step=10, sweeps=14, warm_start=1, **HP)
        torch.cuda.synchronize()
        assert mo.soap_converged(mats, ws, step=10, sweeps=14, **HP) == [(0, 0)], label
        out = {k: mats[0][j].double().cpu().numpy() for j, k in enumerate(("W", "G", "L", "R", "M", "V"))}
        out["U"] = U.double().cpu().numpy()
        check(st, out, 10, HP, f"warm start, {label}")


def test_deterministic(gpu):
    st = warm_state(61, 100, 100)
    a = run_gpu([st], 10, HP)[0]
    b = run_gpu([st], 10, HP)[0]
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_decoder_layer_full_size(gpu):
    """The decoder-layer bucket (hidden 2048, FFN 5632) in one call at the
    default 14 sweeps, from a warm state drawn on the device with torch: the
    2048 x 2048 and one 5632 x 2048 matrix against the oracle at their fp32
    floors, sampled rows of the
    5632-sided statistics in fp64, every output finite, and the eigensolver
    converged (16 sweeps change no update by more than 1e-5 relative)."""
    import torch
    import matrix_optimizers_amd as mo
    from matrix_optimizers_amd import workloads as wlmod
    wl = wlmod.SOAP_WORKLOADS["soap_decoder_layer_h2048"]
    dev = torch.device("cuda:0")
    base = []
    for i, sp in enumerate(wl.matrices):
        gen = torch.Generator(device=dev)
        gen.manual_seed(7000 + i)
        rnd = lambda std: torch.randn((sp.rows, sp.cols), device=dev, generator=gen) * std
        W, G = rnd(0.02), rnd(1e-3)
        L = torch.eye(sp.rows, device=dev) * wl.hp.stat_eps
        R = torch.eye(sp.cols, device=dev) * wl.hp.stat_eps
        for _ in range(10):
            Gp = rnd(1e-3)
            L += Gp @ Gp.T
            R += Gp.T @ Gp
        base.append((W, G, L, R, rnd(1e-3), rnd(1e-3) ** 2))
    torch.cuda.synchronize()
    host = [tuple(t.double().cpu().numpy() for t in m) for m in base]

    def run(sweeps):
        mats = [tuple(t.clone() for t in m) for m in base]
        ups = [torch.empty_like(m[0]) for m in mats]
        mo.soap_owner_step(mats, update_out=ups, step=10, sweeps=sweeps, lr=1e-3, beta1=0.9, beta2=0.999,
                           eps=1e-8, weight_decay=0.01)
        torch.cuda.synchronize()
        return mats, ups

    mats, ups = run(14)
    _, ups16 = run(16)
    for i, (u, u16) in enumerate(zip(ups, ups16)):
        assert torch.isfinite(u).all() and torch.isfinite(mats[i][0]).all(), i
        d = float((u - u16).norm() / u16.norm())
        print(f"matrix {i} {tuple(u.shape)}: 14 vs 16 sweeps {d:.1e}", flush=True)
        assert d <= 1e-5, i
    # matrix 0 (2048 x 2048) against the oracle
    W, G, L, R, M, V = host[0]
    st = dict(W=W, G=G, L=L, R=R, M=M, V=V)
    out = {k: mats[0][j].double().cpu().numpy() for j, k in enumerate(("W", "G", "L", "R", "M", "V"))}
    out["U"] = ups[0].double().cpu().numpy()
    check(st, out, 10, dict(HP, weight_decay=0.01), "decoder 2048x2048")
    # matrix 4 (5632 x 2048: a 5632-sided L) against the oracle
    W, G, L, R, M, V = host[4]
    st = dict(W=W, G=G, L=L, R=R, M=M, V=V)
    out = {k: mats[4][j].double().cpu().numpy() for j, k in enumerate(("W", "G", "L", "R", "M", "V"))}
    out["U"] = ups[4].double().cpu().numpy()
    check(st, out, 10, dict(HP, weight_decay=0.01), "decoder 5632x2048")
    # sampled statistics rows of every 5632-sided matrix, in fp64
    rng = np.random.default_rng(5)
    for i, (W, G, L, R, M, V) in enumerate(host):
        rows = rng.choice(G.shape[0], 4, replace=False)
        Lr = L[rows] + G[rows] @ G.T
        assert rel(mats[i][2][rows].double().cpu().numpy(), Lr) <= 1e-6, i
        cols = rng.choice(G.shape[1], 4, replace=False)
        Rc = R[cols] + G[:, cols].T @ G
        assert rel(mats[i][3][cols].double().cpu().numpy(), Rc) <= 1e-6, i


def test_strided_views_and_mixed_dtypes(gpu):
    """Every tensor as a view into a wider buffer (row stride above its column
    count), bf16 W with fp32 G: the same update as the contiguous call."""
    import torch
    import matrix_optimizers_amd as mo
    st = warm_state(71, 72, 104)
    dev = torch.device("cuda:0")
    r, c = st["W"].shape

    def view(x, extra, dtype=torch.float32):
        rows, cols = x.shape
        big = torch.full((rows, cols + extra), float("nan"), device=dev, dtype=dtype)
        big[:, :cols] = torch.tensor(np.asarray(x, F32), device=dev).to(dtype)
        return big[:, :cols]

    W = view(st["W"], 24, torch.bfloat16)
    G = view(st["G"], 8)
    L, R = view(st["L"], 16), view(st["R"], 40)
    M, V = view(st["M"], 4), view(st["V"], 12)
    U = view(np.zeros((r, c)), 36)
    mo.soap_owner_step([(W, G, L, R, M, V)], update_out=[U], step=10, **HP)
    torch.cuda.synchronize()
    ref = run_gpu([st], 10, HP, w_dtype="bf16")[0]
    assert np.array_equal(U.cpu().numpy(), ref["U"].astype(F32))
    assert np.array_equal(M.cpu().numpy(), ref["M"].astype(F32))
    assert np.array_equal(V.cpu().numpy(), ref["V"].astype(F32))
    assert np.array_equal(L.cpu().numpy(), ref["L"].astype(F32))
    assert np.array_equal(W.float().cpu().numpy(), ref["W"].astype(F32))
    # the padding columns of every buffer are untouched
    for t in (W, G, L, R, M, V, U):
        base = t.as_strided((t.shape[0], t.stride(0)), (t.stride(0), 1))
        assert torch.isnan(base[:, t.shape[1]:].float()).all()


def test_zero_state_and_gradient(gpu):
    """G = L = R = M = V = 0: no rotation happens (the threshold is zero and so
    is every entry), the update is exactly zero and W' = (1 - lr wd) W."""
    import torch
    import matrix_optimizers_amd as mo
    dev = torch.device("cuda:0")
    r, c = 70, 130
    W = torch.randn((r, c), device=dev) * 0.02
    W0 = W.clone()
    z = lambda *s: torch.zeros(s, device=dev)
    U = torch.full((r, c), float("nan"), device=dev)
    hp = dict(HP, weight_decay=0.1)
    mo.soap_owner_step([(W, z(r, c), z(r, r), z(c, c), z(r, c), z(r, c))], update_out=[U], step=1, **hp)
    torch.cuda.synchronize()
    assert torch.equal(U, torch.zeros_like(U))
    decay = np.float32(1 - hp["lr"] * hp["weight_decay"])
    assert torch.equal(W, W0 * float(decay))


@pytest.mark.parametrize("rows, bar", [(9000, 1e-3), (16384, 2e-4)])
def test_long_side_first_step_closed_form(gpu, rows, bar):
    """A long-sided statistic (rows x 64 matrix: 9000 pads to 9024, 141 block
    pairs; 16384, the largest side the library takes, is 256 pairs): one step
    from eps I and zero moments.  With G = U S W^T (thin SVD), the eigenbases
    are U (plus the eps-eigenspace, where G, M' and V' vanish) and W, so G~ is
    S in those bases and the update is lr U diag(s / (s + eps)) W^T (t = 1:
    the bias corrections cancel b1 and b2), the oracle's step in closed form
    (it matches the oracle to 6e-13 at 900 x 64).  The first step divides the
    rotated gradient's small entries by eps, so it amplifies the fp32
    rounding of the statistics by 1 / eps; Adam's eps is 1e-2 here (the
    singular values are about 0.09 and 0.13).  The bar is the fp32 floor of
    each input: the fp32 model of the step with exact eigenvectors
    (fp32_floor) measures 1.04e-3 (9000) and 1.41e-4 (16384) against the
    closed form; the GPU, which accumulates its products in fp64, must stay
    within 1e-3 and 2e-4."""
    r, c = rows, 64
    st = first_state(81, r, c)
    hp = dict(HP, eps=1e-2, weight_decay=0.0)
    out = run_gpu([st], 1, hp)[0]
    U, sv, Wt = np.linalg.svd(st["G"], full_matrices=False)
    D = hp["lr"] * (U * (sv / (sv + hp["eps"]))) @ Wt
    err = rel(out["U"], D)
    print(f"{r} x {c} first step: update {err:.2e} against the closed form", flush=True)
    assert np.all(np.isfinite(out["U"]))
    assert err <= bar


def test_convergence_report(gpu):
    """soap_converged after a step: a single sweep leaves a warm 256 x 384 pair
    of statistics unconverged (pair problems still rotate in the final sweep),
    the default sweep count converges it (a final sweep without rotations),
    and the converged step passes the parity check."""
    import torch
    import matrix_optimizers_amd as mo
    st = warm_state(91, 256, 384)
    dev = torch.device("cuda:0")
    res = {}
    for sweeps in (1, 14):
        t = lambda x: torch.tensor(np.asarray(x, F32), device=dev).contiguous()
        mats = [(t(st["W"]), t(st["G"]), t(st["L"]), t(st["R"]), t(st["M"]), t(st["V"]))]
        ups = [torch.empty(st["W"].shape, dtype=torch.float32, device=dev)]
        step = mo.SoapOwnerStep(mats, update_out=ups, sweeps=sweeps, **HP)
        step(10)
        res[sweeps] = step.rotating_pairs()
        torch.cuda.synchronize()
        if sweeps == 14:
            to = lambda x: x.float().cpu().numpy().astype(np.float64)
            m = mats[0]
            check(st, dict(W=to(m[0]), L=to(m[2]), R=to(m[3]), M=to(m[4]), V=to(m[5]), U=to(ups[0])), 10, HP,
                  "converged 256x384")
    print("rotating pair slots in the final sweep:", res, flush=True)
    assert min(res[1][0]) > 0
    assert res[14] == [(0, 0)]
