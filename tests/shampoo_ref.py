"""A full-size reference route for the Shampoo step, built from the oracle's
pinned pieces (test infrastructure).

For one step from eps I, the thin SVD G = P S Q^T gives L' = P (S^2 + eps) P^T +
eps (I - P P^T) and R' likewise, and every coupled Newton iterate acts on each
eigenvalue by the scalar recurrence (pinned in test_shampoo_oracle.py), so the
lr = 1 update is U = P diag(h_L(s^2 + eps) s h_R(s^2 + eps)) Q^T, with the
Frobenius scales taken over all eigenvalues (the rows - k, resp. cols - k,
eigenvalues equal to eps included).  It costs one SVD instead of 4 K products
of each side, so it reaches the full workload sizes.
"""
import numpy as np

from oracle import shampoo as osh


def svd_route_update(G, eps, iters):
    r, c = G.shape
    P, s, Qt = np.linalg.svd(np.asarray(G, np.float64), full_matrices=False)
    k = len(s)
    lam = s ** 2 + eps
    zl = (osh.P_ROOT + 1) / (2 * np.sqrt(np.sum(lam ** 2) + (r - k) * eps ** 2))
    zr = (osh.P_ROOT + 1) / (2 * np.sqrt(np.sum(lam ** 2) + (c - k) * eps ** 2))
    d = osh.scalar_newton_root(lam, zl, iters) * s * osh.scalar_newton_root(lam, zr, iters)
    return (P * d) @ Qt
