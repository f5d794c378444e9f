"""Pins of the fp64 SOAP oracle (oracle/soap.py) against things other than itself,
CPU only: torch.optim.Adam where the eigenbasis is the coordinate basis, the
polar factor (scipy.linalg.polar) for the first step, orthogonal equivariance,
and invariance to the eigenvectors' signs and order.  A plausible mistake (the
second moment in the weight frame, a missing rotation back, Q_R for Q_R^T, a
bias correction dropped, the decay applied to the update) fails one of them.
"""
import numpy as np
import pytest
import scipy.linalg
import scipy.stats
import torch

from oracle import soap as osoap


def zeros_state(m, n, eps):
    return eps * np.eye(m), eps * np.eye(n), np.zeros((m, n)), np.zeros((m, n))


def axis_gradient(rng, m, n, base):
    """A gradient whose G G^T and G^T G are diagonal with a fixed order of
    values: entries only at (i, i), magnitudes base[i] times a factor near 1."""
    G = np.zeros((m, n))
    k = min(m, n)
    G[np.arange(k), np.arange(k)] = base * (1 + 0.05 * rng.uniform(-1, 1, k)) * rng.choice([-1, 1], k)
    return G


def test_axis_aligned_gradients_are_adam():
    """With G G^T and G^T G diagonal at every step (and the order of their
    entries fixed), the eigenbasis is the coordinate basis and SOAP is Adam:
    three steps against torch.optim.Adam (fp64, weight decay 0)."""
    rng = np.random.default_rng(0)
    m, n, lr, b1, b2, eps = 4, 6, 1e-2, 0.9, 0.99, 1e-8
    base = np.array([3.0, 1.5, 0.7, 0.2])
    W = rng.standard_normal((m, n))
    L, R, M, V = zeros_state(m, n, 1e-3)
    Wt = torch.tensor(W.copy(), requires_grad=True)
    opt = torch.optim.Adam([Wt], lr=lr, betas=(b1, b2), eps=eps)
    for t in range(1, 4):
        G = axis_gradient(rng, m, n, base)
        W, L, R, M, V, _ = osoap.soap_step(W, G, L, R, M, V, t, lr, b1, b2, eps)
        Wt.grad = torch.tensor(G)
        opt.step()
        np.testing.assert_allclose(W, Wt.detach().numpy(), rtol=0, atol=1e-12)


def test_first_step_is_the_polar_factor():
    """From zero moments, step 1: M~ / sqrt(V~) = sign(Q_L^T G Q_R), and in G's
    singular bases that matrix has +-s_i at matching singular vectors and zeros
    elsewhere, so the update is U V^T, the orthogonal polar factor of G.  Adam's
    eps must sit far below the singular values and far above fp64 rounding of
    the zero entries (which the elementwise division would otherwise lift)."""
    rng = np.random.default_rng(1)
    for m, n in ((5, 9), (9, 5), (6, 6)):
        G = rng.standard_normal((m, n))
        L, R, M, V = zeros_state(m, n, 1e-12)
        _, _, _, _, _, D = osoap.soap_step(np.zeros((m, n)), G, L, R, M, V, 1, 1.0, eps=1e-7)
        if m <= n:
            Up, _ = scipy.linalg.polar(G.T)
            want = Up.T
        else:
            want, _ = scipy.linalg.polar(G)
        np.testing.assert_allclose(D, want, rtol=0, atol=1e-5)


def test_orthogonal_equivariance():
    """Rotating the gradient (and the statistics it came from) on both sides
    rotates the update the same way: SOAP(U G Z^T) = U SOAP(G) Z^T, for two
    steps with the second step's state carried.  Adam's eps is 1e-3 here: the
    rotated gradient is diagonal in the singular bases, and a small eps would
    lift the fp64 rounding of its zero entries (the step is a sign function
    there) above the pin's tolerance."""
    rng = np.random.default_rng(2)
    m, n = 5, 7
    U = scipy.stats.ortho_group.rvs(m, random_state=3)
    Z = scipy.stats.ortho_group.rvs(n, random_state=4)
    G1, G2 = rng.standard_normal((m, n)), rng.standard_normal((m, n))
    L, R, M, V = zeros_state(m, n, 0.1)
    a = osoap.soap_step(np.zeros((m, n)), G1, L, R, M, V, 1, 1.0, eps=1e-3)
    b = osoap.soap_step(np.zeros((m, n)), U @ G1 @ Z.T, U @ L @ U.T, Z @ R @ Z.T, M, V, 1, 1.0, eps=1e-3)
    np.testing.assert_allclose(b[5], U @ a[5] @ Z.T, rtol=0, atol=1e-10)
    a2 = osoap.soap_step(a[0], G2, a[1], a[2], a[3], a[4], 2, 1.0, eps=1e-3)
    b2 = osoap.soap_step(b[0], U @ G2 @ Z.T, b[1], b[2], b[3], b[4], 2, 1.0, eps=1e-3)
    np.testing.assert_allclose(b2[5], U @ a2[5] @ Z.T, rtol=0, atol=1e-10)


def test_eigenvector_sign_and_order_do_not_matter(monkeypatch):
    """Flipping the signs and reversing the order of the eigenvectors leaves
    the update unchanged (one step and, with the moments carried, two)."""
    rng = np.random.default_rng(5)
    m, n = 4, 6
    G1, G2 = rng.standard_normal((m, n)), rng.standard_normal((m, n))
    L, R, M, V = zeros_state(m, n, 0.1)
    ref1 = osoap.soap_step(np.zeros((m, n)), G1, L, R, M, V, 1, 1.0, eps=1e-3)
    ref2 = osoap.soap_step(ref1[0], G2, *ref1[1:5], 2, 1.0, eps=1e-3)
    plain = osoap.eigenbasis

    def flipped(S):
        Q = plain(S)[:, ::-1]
        return Q * np.where(np.arange(Q.shape[1]) % 2 == 0, -1.0, 1.0)
    monkeypatch.setattr(osoap, "eigenbasis", flipped)
    got1 = osoap.soap_step(np.zeros((m, n)), G1, L, R, M, V, 1, 1.0, eps=1e-3)
    np.testing.assert_allclose(got1[5], ref1[5], rtol=0, atol=1e-12)
    # the second moment lives in the (reordered) eigenbasis: carry this run's own
    got2 = osoap.soap_step(got1[0], G2, *got1[1:5], 2, 1.0, eps=1e-3)
    np.testing.assert_allclose(got2[5], ref2[5], rtol=0, atol=1e-12)


def test_statistics_and_decay():
    """L', R' accumulate like Shampoo's, and the decay multiplies the old W."""
    G = np.array([[1.0, 2.0, 0.0], [0.0, 1.0, -1.0]])
    L, R, M, V = zeros_state(2, 3, 1.0)
    W = np.ones((2, 3))
    W1, L1, R1, _, _, D = osoap.soap_step(W, G, L, R, M, V, 1, 0.1, weight_decay=0.5)
    np.testing.assert_array_equal(L1, [[6.0, 2.0], [2.0, 3.0]])
    np.testing.assert_array_equal(R1, [[2.0, 2.0, 0.0], [2.0, 6.0, -1.0], [0.0, -1.0, 2.0]])
    np.testing.assert_allclose(W1, 0.95 * W - D, rtol=0, atol=1e-15)


def test_eigenvector_order_matters_once_v_is_warm(monkeypatch):
    """The second moment V is indexed by the eigenbasis, so with a warm V the
    update depends on the eigenvectors' order (the reading fixes ascending
    eigenvalue order, numpy's eigh), while their signs still do not matter:
    reversing the order changes the update, flipping signs does not."""
    rng = np.random.default_rng(9)
    m, n = 5, 7
    G = rng.standard_normal((m, n))
    L = 0.1 * np.eye(m) + (lambda A: A @ A.T)(rng.standard_normal((m, 2 * m)))
    R = 0.1 * np.eye(n) + (lambda A: A @ A.T)(rng.standard_normal((n, 2 * n)))
    M = rng.standard_normal((m, n))
    V = rng.standard_normal((m, n)) ** 2
    ref = osoap.soap_step(np.zeros((m, n)), G, L, R, M, V, 5, 1.0, eps=1e-3)[5]
    plain = osoap.eigenbasis

    def signs(S):
        Q = plain(S)
        return Q * np.where(np.arange(Q.shape[1]) % 2 == 0, -1.0, 1.0)
    monkeypatch.setattr(osoap, "eigenbasis", signs)
    flipped = osoap.soap_step(np.zeros((m, n)), G, L, R, M, V, 5, 1.0, eps=1e-3)[5]
    np.testing.assert_allclose(flipped, ref, rtol=0, atol=1e-12)
    monkeypatch.setattr(osoap, "eigenbasis", lambda S: plain(S)[:, ::-1])
    reordered = osoap.soap_step(np.zeros((m, n)), G, L, R, M, V, 5, 1.0, eps=1e-3)[5]
    assert np.linalg.norm(reordered - ref) > 1e-2 * np.linalg.norm(ref)
