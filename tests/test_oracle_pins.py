"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names the kind of pin: SVD brute force, exact closed forms, an
invariant of the mathematics, or an independent library routine (numpy/scipy
SVD and polar decomposition, torch.optim.Muon, torch.optim.AdamW).  A plausible
mistake in the oracle (dropped b or c term, wrong sign, A A vs A, skipped
transpose, eps added instead of clamped, heavy-ball instead of EMA momentum,
wrong lr multiplier, decay with the adjusted lr) fails at least one of them.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import scipy.linalg

from matrix_optimizers_amd.workloads import MuonHP, AdamWHP
from oracle import adamw as oadamw
from oracle import muon as omuon

A5 = (3.4445, -4.7750, 2.0315)


def scalar_chain(s: float, coeffs, steps: int) -> float:
    a, b, c = coeffs
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def exact_chain(s: Fraction, coeffs, steps: int) -> Fraction:
    a, b, c = (Fraction(str(x)) for x in coeffs)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def svd_brute_force(X: np.ndarray, coeffs, steps: int, eps: float) -> np.ndarray:
    """U p^K(S / max(||X||_F, eps)) V^T via numpy's fp64 SVD."""
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    nrm = max(float(np.sqrt(np.sum(S ** 2))), eps)
    P = np.array([scalar_chain(float(s) / nrm, coeffs, steps) for s in S])
    return (U * P) @ Vt


@pytest.mark.parametrize("shape", [(1, 1), (2, 3), (3, 2), (4, 8), (8, 4), (16, 32), (33, 17)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_ns_equals_svd_brute_force(shape, steps):
    """Pin: the iteration acts on singular values by the scalar quintic."""
    rng = np.random.default_rng(hash((shape, steps)) & 0xFFFF)
    X = rng.standard_normal(shape)
    hp = MuonHP(ns_steps=steps)
    got = omuon.orthogonalize(X, hp)
    want = svd_brute_force(X, A5, steps, hp.eps)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_ns_svd_brute_force_other_coefficients():
    """Pin with coefficients where a b/c swap or sign slip changes the answer."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((6, 11))
    coeffs = (2.0, -1.5, 0.5)
    got = omuon.newton_schulz(X, *coeffs, steps=3, eps=1e-7)
    want = svd_brute_force(X, coeffs, 3, 1e-7)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_rank_one_closed_form():
    """Pin: rank-1 G = u v^T has one singular value; after normalisation it is 1,
    so O = p^5(1) * (u/|u|)(v/|v|)^T, with p^5(1) from exact rational arithmetic."""
    rng = np.random.default_rng(3)
    u, v = rng.standard_normal(5), rng.standard_normal(9)
    O = omuon.newton_schulz(np.outer(u, v), *A5, steps=5, eps=1e-7)
    k = float(exact_chain(Fraction(1), A5, 5))
    assert abs(k - 0.6964364094697522) < 1e-15
    want = k * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    np.testing.assert_allclose(O, want, rtol=0, atol=1e-13)


def test_scaled_partial_identity_closed_form():
    """Pin: kappa [I_4 | 0] has four singular values kappa, Frobenius norm 2 kappa,
    so every normalised singular value is 1/2 and O = p^5(1/2) [I_4 | 0]."""
    X = np.zeros((4, 8))
    X[:, :4] = 3.7 * np.eye(4)
    O = omuon.newton_schulz(X, *A5, steps=5, eps=1e-7)
    k = float(exact_chain(Fraction(1, 2), A5, 5))
    assert abs(k - 0.7654385304543384) < 1e-15
    want = np.zeros((4, 8))
    want[:, :4] = k * np.eye(4)
    np.testing.assert_allclose(O, want, rtol=0, atol=1e-14)


def test_diagonal_acts_entrywise():
    """Pin: a diagonal input stays diagonal; each entry follows the scalar chain
    from |d_i| / ||d||_2 with the sign of d_i."""
    d = np.array([0.3, -1.2, 2.5, 0.01, -0.7])
    O = omuon.newton_schulz(np.diag(d), *A5, steps=5, eps=1e-7)
    nrm = float(np.sqrt(np.sum(d ** 2)))
    want = np.diag([math.copysign(float(exact_chain(Fraction(abs(x)) / Fraction(nrm), A5, 5)), x)
                    for x in d])
    np.testing.assert_allclose(O, want, rtol=0, atol=1e-14)


def test_quintic_band_after_five_steps():
    """Pin: five quintic steps map normalised singular values in [1e-3, 1] into a
    band around 1 (the property that makes the update spectrum-balanced)."""
    s = np.logspace(-3, 0, 2000)
    out = np.array([scalar_chain(x, A5, 5) for x in s])
    assert out.min() > 0.45 and out.max() < 1.21
    # and the matrix iteration inherits it
    rng = np.random.default_rng(11)
    O = omuon.newton_schulz(rng.standard_normal((32, 64)), *A5, steps=5, eps=1e-7)
    sv = np.linalg.svd(O, compute_uv=False)
    assert sv.min() > 0.45 and sv.max() < 1.21


def test_cubic_variant_converges_to_polar_factor():
    """Pin: with (a, b, c) = (1.5, -0.5, 0) the iteration is the classical cubic
    Newton-Schulz and converges to the polar factor U V^T (scipy.linalg.polar)."""
    rng = np.random.default_rng(5)
    m, n = 12, 20
    Q1, _ = np.linalg.qr(rng.standard_normal((m, m)))
    Q2, _ = np.linalg.qr(rng.standard_normal((n, m)))
    s = np.linspace(1.0, 3.0, m)            # normalised sigma_min = 1/||s|| > 0.1
    X = (Q1 * s) @ Q2.T
    O = omuon.newton_schulz(X, 1.5, -0.5, 0.0, steps=40, eps=1e-7)
    Up, _ = scipy.linalg.polar(X.T)         # X^T = Up P, Up n x m
    np.testing.assert_allclose(O, Up.T, rtol=0, atol=1e-12)


def haar(rng, k):
    Q, R = np.linalg.qr(rng.standard_normal((k, k)))
    return Q * np.sign(np.diag(R))


def test_orthogonal_scale_transpose_equivariance():
    """Invariants: NS(Q1 X Q2) = Q1 NS(X) Q2, NS(alpha X) = NS(X), NS(X^T) = NS(X)^T."""
    rng = np.random.default_rng(9)
    X = rng.standard_normal((10, 24))
    Q1, Q2 = haar(rng, 10), haar(rng, 24)
    ns = lambda Y: omuon.newton_schulz(Y, *A5, steps=5, eps=1e-7)
    base = ns(X)
    np.testing.assert_allclose(ns(Q1 @ X @ Q2), Q1 @ base @ Q2, atol=1e-12)
    np.testing.assert_allclose(ns(7.3 * X), base, atol=1e-12)
    hp = MuonHP()
    np.testing.assert_allclose(omuon.orthogonalize(X.T, hp), omuon.orthogonalize(X, hp).T,
                               atol=1e-12)


def test_eps_is_a_clamp():
    """Pin: below eps the divisor is eps itself: O = U p^5(S/eps) V^T."""
    rng = np.random.default_rng(2)
    X = rng.standard_normal((6, 9))
    X *= 2e-9 / np.linalg.norm(X)           # ||X||_F = 2e-9 < eps = 1e-7
    got = omuon.newton_schulz(X, *A5, steps=5, eps=1e-7)
    want = svd_brute_force(X, A5, 5, 1e-7)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    # an added eps would give a visibly different scale
    wrong = svd_brute_force(X / (2e-9 + 1e-7) * 1e-7, A5, 5, 1e-7)
    assert np.abs(got - wrong).max() > 1e-4 * np.abs(got).max()


def test_zero_gradient_closed_form():
    """Closed form: G = M = 0 gives O = 0, so W' = (1 - lr*wd) W and M' = 0."""
    hp = MuonHP(lr=0.02, weight_decay=0.5)
    W = np.random.default_rng(1).standard_normal((7, 3))
    Wn, Mn, D = omuon.muon_step(W, np.zeros((7, 3)), np.zeros((7, 3)), hp)
    np.testing.assert_array_equal(Wn, (1 - 0.02 * 0.5) * W)
    assert not Mn.any() and not D.any()


def test_empty_matrix_is_skipped():
    hp = MuonHP()
    for shape in [(0, 5), (5, 0), (0, 0)]:
        W = np.zeros(shape)
        Wn, Mn, D = omuon.muon_step(W, W, W, hp)
        assert Wn.shape == shape and Mn.shape == shape


def test_lr_multiplier_values():
    """The three adjustments at shapes where they differ."""
    assert omuon.lr_multiplier(8, 2, "original") == 2.0
    assert omuon.lr_multiplier(2, 8, "original") == 1.0
    assert omuon.lr_multiplier(128256, 4096, "original") == pytest.approx(5.5958, abs=1e-4)
    assert omuon.lr_multiplier(8, 2, "match_rms_adamw") == pytest.approx(0.2 * math.sqrt(8))
    assert omuon.lr_multiplier(8, 2, "none") == 1.0


# ---------------------------------------------------------------------------
# library witnesses
# ---------------------------------------------------------------------------

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("shape", [(64, 128), (128, 64), (96, 96)])
@pytest.mark.parametrize("nesterov", [True, False])
@pytest.mark.parametrize("adjust", ["original", "match_rms_adamw"])
def test_torch_muon_witness(shape, nesterov, adjust):
    """Witness: torch.optim.Muon (named by the paper's §5.1 as its optimizer).
    Its Newton-Schulz runs in bf16, so the update agrees only to ~1e-2; its
    momentum buffer is fp32 and agrees to fp32 rounding.  Two steps, so the
    second step sees a nonzero buffer."""
    rng = np.random.default_rng(abs(hash((shape, nesterov, adjust))) & 0xFFFF)
    W0 = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    G1 = (rng.standard_normal(shape) * 1e-3).astype(np.float32)
    G2 = (rng.standard_normal(shape) * 1e-3).astype(np.float32)
    hp = MuonHP(lr=0.02, weight_decay=0.1, momentum=0.9, nesterov=nesterov, lr_adjust=adjust)
    p = torch.nn.Parameter(torch.from_numpy(W0.copy()))
    opt = torch.optim.Muon([p], lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                           nesterov=nesterov, adjust_lr_fn=adjust)
    W, M = W0.astype(np.float64), np.zeros(shape)
    for G in (G1, G2):
        before = p.detach().numpy().astype(np.float64).copy()
        p.grad = torch.from_numpy(G.copy())
        opt.step()
        W_o, M_o, D_o = omuon.muon_step(before, G, M, hp)
        d_torch = (1 - hp.lr * hp.weight_decay) * before - p.detach().numpy().astype(np.float64)
        rel = np.linalg.norm(d_torch - D_o) / np.linalg.norm(D_o)
        assert rel < 3e-2, rel
        buf = opt.state[p]["momentum_buffer"].numpy().astype(np.float64)
        assert np.linalg.norm(buf - M_o) / np.linalg.norm(M_o) < 1e-6
        M = buf  # continue from torch's buffer (fp32 rounding only)


def test_torch_adamw_witness():
    """Witness: torch.optim.AdamW in fp64 over several steps."""
    rng = np.random.default_rng(4)
    n = 1000
    p0 = rng.standard_normal(n) * 0.02
    hp = AdamWHP()
    p = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                            weight_decay=hp.weight_decay)
    m = np.zeros(n)
    v = np.zeros(n)
    pp = p0.copy()
    for t in range(1, 6):
        g = rng.standard_normal(n) * 1e-3
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        pp, m, v = oadamw.adamw_step(pp, g, m, v, t, hp.lr, hp.beta1, hp.beta2, hp.eps,
                                     hp.weight_decay)
        np.testing.assert_allclose(p.detach().numpy(), pp, rtol=1e-13, atol=0)
        # torch forms m' by lerp, a different fp64 rounding order than beta*m + (1-beta)*g
        np.testing.assert_allclose(opt.state[p]["exp_avg"].numpy(), m, rtol=1e-11, atol=0)
        np.testing.assert_allclose(opt.state[p]["exp_avg_sq"].numpy(), v, rtol=1e-11, atol=0)


def test_adamw_first_step_closed_form():
    """Closed form at t = 1 from m = v = 0: m' = (1-b1) g, v' = (1-b2) g^2, the
    bias corrections cancel, p' = p(1 - lr wd) - lr g / (|g| + eps)."""
    rng = np.random.default_rng(8)
    p, g = rng.standard_normal(50), rng.standard_normal(50) * 1e-3
    hp = AdamWHP()
    pn, mn, vn = oadamw.adamw_step(p, g, np.zeros(50), np.zeros(50), 1, hp.lr, hp.beta1,
                                   hp.beta2, hp.eps, hp.weight_decay)
    want = p * (1 - hp.lr * hp.weight_decay) - hp.lr * g / (np.abs(g) + hp.eps)
    np.testing.assert_allclose(pn, want, rtol=1e-12, atol=0)
    np.testing.assert_allclose(mn, (1 - hp.beta1) * g, rtol=1e-15)
    np.testing.assert_allclose(vn, (1 - hp.beta2) * g * g, rtol=1e-15)
