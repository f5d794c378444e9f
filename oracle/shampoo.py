"""Plain fp64 Shampoo owner step.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's CPU baseline, never by the library or its binding.

"MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
sharding", §5.7: because every 2D matrix is whole on its owner, the owner can
run any single-device matrix optimizer; the paper swaps owner-Muon for Shampoo
with full left / right preconditioners and an inverse fourth root, in float32.
The pages name the method but print none of its formulas.  The readings here
(each also stated beside the C entry point):

  Statistics (the published Shampoo update for a matrix, Gupta, Koren and
  Singer, 2018, Algorithm 1; the caller starts L and R at eps I):
      L' = L + G G^T        R' = R + G^T G
  Preconditioned direction and the weight write (decoupled weight decay, as
  the Muon path of the same owner writes it):
      U  = L'^{-1/4} G R'^{-1/4}
      W' = (1 - lr wd) W - lr U
  The inverse fourth root, "root" = "exact": V diag(lambda^{-1/4}) V^T from a
  symmetric eigendecomposition (the definition).  "root" = "newton": the
  coupled Newton iteration for the inverse p-th root (Guo and Higham, 2006),
  p = 4, with the Frobenius-norm scaling used by the large-scale Shampoo
  implementation of Anil et al. (2020):
      z = (p + 1) / (2 ||A||_F),   M_0 = z A,   H_0 = z^{1/p} I
      for k = 1 .. K:   X = ((p + 1) I - M) / p,   H <- H X,   M <- X^p M
      A^{-1/p} ~ H_K
  (H^p A = M holds at every step and M -> I, so H -> A^{-1/p}.)  The HIP path
  runs this iteration in fp32 for a caller-chosen K; parity compares it with
  the same K here.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

P_ROOT = 4


def inverse_fourth_root(A: np.ndarray) -> np.ndarray:
    """A^{-1/4} for a symmetric positive definite A, by definition.
    Pins: the closed forms of tests/test_shampoo_oracle.py (scaled identity,
    rank-one updates), (A^{-1/4})^4 A = I."""
    A = np.asarray(A, np.float64)
    lam, V = np.linalg.eigh((A + A.T) / 2)
    return (V * lam ** -0.25) @ V.T


def newton_scale(A: np.ndarray) -> float:
    """z = (p + 1) / (2 ||A||_F)."""
    return (P_ROOT + 1) / (2.0 * float(np.linalg.norm(np.asarray(A, np.float64))))


def coupled_newton_root(A: np.ndarray, iters: int) -> np.ndarray:
    """H_K of the coupled Newton iteration for A^{-1/4} (module docstring).
    Pins: converges to inverse_fourth_root on well-conditioned A; acts on each
    eigenvalue as the scalar recurrence (scalar_newton_root); 1x1 hand values."""
    A = np.asarray(A, np.float64)
    n = A.shape[0]
    eye = np.eye(n)
    z = newton_scale(A)
    M = z * A
    H = z ** (1.0 / P_ROOT) * eye
    for _ in range(iters):
        X = ((P_ROOT + 1) * eye - M) / P_ROOT
        H = H @ X
        M = np.linalg.matrix_power(X, P_ROOT) @ M
    return H


def scalar_newton_root(lam: np.ndarray, z: float, iters: int) -> np.ndarray:
    """The same iteration on scalars: h_K for each eigenvalue lam, scale z."""
    m = z * np.asarray(lam, np.float64)
    h = np.full_like(m, z ** (1.0 / P_ROOT))
    for _ in range(iters):
        x = ((P_ROOT + 1) - m) / P_ROOT
        h = h * x
        m = x ** P_ROOT * m
    return h


def statistics(G: np.ndarray, L: np.ndarray, R: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """L + G G^T and R + G^T G."""
    G = np.asarray(G, np.float64)
    return np.asarray(L, np.float64) + G @ G.T, np.asarray(R, np.float64) + G.T @ G


def root(A: np.ndarray, how: str, iters: int) -> np.ndarray:
    if how == "exact":
        return inverse_fourth_root(A)
    if how == "newton":
        return coupled_newton_root(A, iters)
    raise ValueError(how)


def shampoo_step(W, G, L, R, lr: float, weight_decay: float = 0.0, how: str = "newton",
                 iters: int = 20):
    """One owner step on one matrix; returns (W', L', R', lr * U) in fp64."""
    L1, R1 = statistics(G, L, R)
    U = root(L1, how, iters) @ np.asarray(G, np.float64) @ root(R1, how, iters)
    W1 = (1.0 - lr * weight_decay) * np.asarray(W, np.float64) - lr * U
    return W1, L1, R1, lr * U


def initial_statistics(rows: int, cols: int, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """L_0 = eps I_rows, R_0 = eps I_cols."""
    return eps * np.eye(rows), eps * np.eye(cols)
