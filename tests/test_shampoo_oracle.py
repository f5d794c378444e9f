"""Pins of the fp64 Shampoo oracle (oracle/shampoo.py) against things other than
itself, CPU only: closed forms of the inverse fourth root, convergence of the
coupled Newton iteration to the eigendecomposition definition, its action on
each eigenvalue, Shampoo's one-step identity with the polar factor (a textbook
routine), hand-computed statistics and the weight-decay write.  A plausible
mistake (a -1/2 power for -1/4, G^T G for G G^T, a transposed operand, H_0 = I,
a spectral instead of a Frobenius scale, the identity term dropped or not
divided by p, the decay applied to the update) fails at least one of them.
"""
import numpy as np
import pytest
import scipy.linalg
import scipy.stats

from oracle import shampoo as osh
from shampoo_ref import svd_route_update


def random_orthogonal(n, seed):
    return scipy.stats.ortho_group.rvs(n, random_state=seed) if n > 1 else np.ones((1, 1))


def spd_with_spectrum(lam, seed):
    V = random_orthogonal(len(lam), seed)
    return (V * np.asarray(lam, np.float64)) @ V.T, V


def test_inverse_fourth_root_closed_forms():
    """c I -> c^{-1/4} I; eps I + s^2 u u^T -> eps^{-1/4} (I - u u^T) + (eps + s^2)^{-1/4} u u^T."""
    np.testing.assert_allclose(osh.inverse_fourth_root(16.0 * np.eye(5)), 0.5 * np.eye(5), rtol=0, atol=1e-14)
    rng = np.random.default_rng(1)
    u = rng.standard_normal(7)
    u /= np.linalg.norm(u)
    eps, s2 = 1e-3, 4.0
    A = eps * np.eye(7) + s2 * np.outer(u, u)
    P = np.outer(u, u)
    want = eps ** -0.25 * (np.eye(7) - P) + (eps + s2) ** -0.25 * P
    np.testing.assert_allclose(osh.inverse_fourth_root(A), want, rtol=1e-12, atol=1e-12)


def test_inverse_fourth_root_on_a_known_eigenbasis():
    """V diag(lam) V^T with V built here (not from eigh) -> V diag(lam^{-1/4}) V^T,
    and its fourth power inverts A."""
    lam = np.array([0.01, 0.3, 1.0, 2.0, 7.5, 40.0])
    A, V = spd_with_spectrum(lam, 3)
    want = (V * lam ** -0.25) @ V.T
    got = osh.inverse_fourth_root(A)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.matrix_power(got, 4) @ A, np.eye(6), rtol=0, atol=1e-10)


@pytest.mark.parametrize("cond", [1.0, 10.0, 1e3])
def test_coupled_newton_converges_to_the_definition(cond):
    """Enough steps reach A^{-1/4} itself (from the constructed eigenbasis)."""
    lam = np.geomspace(1.0, cond, 9) * 3e-2
    A, V = spd_with_spectrum(lam, 5)
    want = (V * lam ** -0.25) @ V.T
    got = osh.coupled_newton_root(A, 40)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-11 * np.abs(want).max())


def test_coupled_newton_acts_per_eigenvalue():
    """Every iterate is a polynomial in A: on V diag(lam) V^T it is V diag(h_K(lam)) V^T
    with h_K the scalar recurrence, for converged and unconverged step counts,
    and the scalar h_K tends to lam^{-1/4}."""
    lam = np.array([1e-6, 1e-3, 0.02, 0.5, 1.0, 3.0])
    A, V = spd_with_spectrum(lam, 7)
    z = osh.newton_scale(A)
    np.testing.assert_allclose(z, 2.5 / np.sqrt(np.sum(lam ** 2)), rtol=1e-14)   # Frobenius = sqrt(sum lam^2)
    for K in (1, 2, 5, 30):
        h = osh.scalar_newton_root(lam, z, K)
        np.testing.assert_allclose(osh.coupled_newton_root(A, K), (V * h) @ V.T, rtol=0, atol=1e-10 * h.max())
    h60 = osh.scalar_newton_root(lam, z, 60)
    np.testing.assert_allclose(h60, lam ** -0.25, rtol=1e-12)


def test_coupled_newton_one_step_by_hand():
    """1 x 1, a = 4: z = 5/8, H_1 = z^{1/4} (5 - z a) / 4 = z^{1/4} * 0.625;
    2 steps: M_1 = 0.625^4 * 2.5, H_2 = H_1 (5 - M_1) / 4."""
    A = np.array([[4.0]])
    z = 5.0 / 8.0
    h1 = z ** 0.25 * 0.625
    np.testing.assert_allclose(osh.coupled_newton_root(A, 1), [[h1]], rtol=1e-15)
    m1 = 0.625 ** 4 * 2.5
    np.testing.assert_allclose(osh.coupled_newton_root(A, 2), [[h1 * (5 - m1) / 4]], rtol=1e-15)


def test_statistics_by_hand():
    G = np.array([[1.0, 2.0, 0.0], [0.0, 1.0, -1.0]])
    L, R = osh.statistics(G, np.eye(2), 2 * np.eye(3))
    np.testing.assert_array_equal(L, [[6.0, 2.0], [2.0, 3.0]])
    np.testing.assert_array_equal(R, [[3.0, 2.0, 0.0], [2.0, 7.0, -1.0], [0.0, -1.0, 3.0]])


@pytest.mark.parametrize("how", ["exact", "newton"])
def test_orthogonal_gradient_closed_form(how):
    """G = s Q (Q orthogonal): L' = R' = (eps + s^2) I, U = s (eps + s^2)^{-1/2} Q."""
    Q = random_orthogonal(6, 11)
    s, eps = 0.3, 0.01
    L0, R0 = osh.initial_statistics(6, 6, eps)
    W = np.zeros((6, 6))
    _, L1, R1, dU = osh.shampoo_step(W, s * Q, L0, R0, lr=1.0, how=how, iters=40)
    np.testing.assert_allclose(L1, (eps + s * s) * np.eye(6), atol=1e-15)
    np.testing.assert_allclose(dU, s / np.sqrt(eps + s * s) * Q, rtol=0, atol=1e-12)


@pytest.mark.parametrize("how", ["exact", "newton"])
def test_rank_one_closed_form(how):
    """G = sigma u v^T (unit u in R^5, v in R^9): U = sigma (eps + sigma^2)^{-1/2} u v^T.
    The sides differ, so a transposed operand or swapped L/R fails on shape or value."""
    rng = np.random.default_rng(2)
    u, v = rng.standard_normal(5), rng.standard_normal(9)
    u /= np.linalg.norm(u)
    v /= np.linalg.norm(v)
    sig, eps = 2.0, 0.5
    L0, R0 = osh.initial_statistics(5, 9, eps)
    _, _, _, dU = osh.shampoo_step(np.zeros((5, 9)), sig * np.outer(u, v), L0, R0, lr=1.0, how=how, iters=40)
    np.testing.assert_allclose(dU, sig / np.sqrt(eps + sig * sig) * np.outer(u, v), rtol=0, atol=1e-12)


def test_one_step_is_the_polar_factor():
    """From eps I with eps -> 0, one Shampoo step is (G G^T)^{-1/4} G (G^T G)^{-1/4}
    = U V^T, the orthogonal polar factor of G (scipy.linalg.polar)."""
    rng = np.random.default_rng(4)
    G = rng.standard_normal((5, 9))
    L0, R0 = osh.initial_statistics(5, 9, 1e-14)
    _, _, _, dU = osh.shampoo_step(np.zeros((5, 9)), G, L0, R0, lr=1.0, how="exact")
    Up, _ = scipy.linalg.polar(G.T)   # G^T = Up P: Up is 9 x 5 with orthonormal columns
    np.testing.assert_allclose(dU, Up.T, rtol=0, atol=1e-6)


def test_second_step_accumulates():
    """Step 2 preconditions with eps I + G1 G1^T + G2 G2^T, not with G2 alone."""
    rng = np.random.default_rng(6)
    G1, G2 = rng.standard_normal((4, 6)), rng.standard_normal((4, 6))
    L0, R0 = osh.initial_statistics(4, 6, 0.1)
    _, L1, R1, _ = osh.shampoo_step(np.zeros((4, 6)), G1, L0, R0, lr=1.0, how="exact")
    _, L2, R2, dU = osh.shampoo_step(np.zeros((4, 6)), G2, L1, R1, lr=1.0, how="exact")
    np.testing.assert_allclose(L2, 0.1 * np.eye(4) + G1 @ G1.T + G2 @ G2.T, atol=1e-13)
    np.testing.assert_allclose(R2, 0.1 * np.eye(6) + G1.T @ G1 + G2.T @ G2, atol=1e-13)
    want = scipy.linalg.fractional_matrix_power(L2, -0.25) @ G2 @ scipy.linalg.fractional_matrix_power(R2, -0.25)
    np.testing.assert_allclose(dU, np.real(want), rtol=0, atol=1e-10)


def test_weight_write():
    """W' = (1 - lr wd) W - lr U, with U from the closed form of an orthogonal G."""
    Q = random_orthogonal(4, 8)
    W = np.arange(16.0).reshape(4, 4) / 10
    eps, lr, wd = 0.0, 0.1, 0.5
    L0, R0 = osh.initial_statistics(4, 4, eps)
    W1, _, _, dU = osh.shampoo_step(W, Q, L0, R0, lr=lr, weight_decay=wd, how="exact")
    np.testing.assert_allclose(W1, 0.95 * W - 0.1 * Q, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dU, 0.1 * Q, rtol=0, atol=1e-13)


def test_svd_route_matches_the_oracle():
    """The full-size reference route of the GPU tests agrees with the oracle."""
    rng = np.random.default_rng(9)
    for r, c in ((40, 70), (70, 40), (33, 33)):
        G = rng.standard_normal((r, c)) * 1e-3
        L0, R0 = osh.initial_statistics(r, c, 1e-6)
        _, _, _, D = osh.shampoo_step(np.zeros((r, c)), G, L0, R0, 1.0, 0.0, "newton", 20)
        U = svd_route_update(G, 1e-6, 20)
        assert np.linalg.norm(U - D) <= 1e-9 * np.linalg.norm(D)
