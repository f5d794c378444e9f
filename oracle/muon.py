"""fp64 oracle of the owner-side Muon step (test infrastructure; see package header).

Every value is carried in float64 on the exact stored input values.  Matrix
products use numpy's fp64 ``@`` as a library primitive; there is no blocking,
fusion or reordering beyond the algorithm's own order.

Readings taken where the pages are silent (the paper prints no update formula and
no Newton-Schulz coefficients; it names torch.optim.Muon as its optimizer in
§5.1 Setup, so that optimizer's documented behaviour fills the gaps):
  * momentum is an exponential moving average, M' = beta*M + (1-beta)*G;
  * the Nesterov blend is U = (1-beta)*G + beta*M';
  * the Gram side is the short side: a tall matrix (rows > cols) is transposed
    before the iteration and transposed back after it; ties are not transposed;
  * normalisation divides by max(||X||_F, eps) (a clamp, not an added eps);
  * the learning-rate multiplier is sqrt(max(1, rows/cols)) ("original"),
    0.2*sqrt(max(rows, cols)) ("match_rms_adamw", the setting of §5.1), or 1;
  * decoupled decay multiplies the old weight by (1 - lr*wd) with the
    unadjusted lr.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np


def momentum(G: np.ndarray, M: np.ndarray, beta: float, nesterov: bool):
    """Momentum smoothing of the owner's full gradient.

    [A] describes Muon's orthogonalised input as the momentum-averaged gradient;
    [P §5.1] gives the momentum coefficient as a hyperparameter.
    Returns (M', U): the new momentum buffer and the matrix handed to the
    orthogonalisation.
    Pins: torch.optim.Muon's momentum buffer (library witness).
    """
    G = np.asarray(G, np.float64)
    M = np.asarray(M, np.float64)
    M_new = beta * M + (1.0 - beta) * G
    if nesterov:
        U = (1.0 - beta) * G + beta * M_new
    else:
        U = M_new.copy()
    return M_new, U


def frobenius_norm(X: np.ndarray) -> float:
    """sqrt of the sum of squares (numpy's fp64 sum as the library primitive)."""
    X = np.asarray(X, np.float64)
    return math.sqrt(float(np.sum(X * X)))


def newton_schulz(X: np.ndarray, a: float, b: float, c: float, steps: int,
                  eps: float, on_step=None) -> np.ndarray:
    """Frobenius normalisation, then `steps` quintic Newton-Schulz iterations.

    [P §2]: the orthogonalisation's steps are built from products X X^T, which
    couple the rows of the whole matrix.  Each iteration here is
        A = X X^T;  B = b*A + c*(A A);  X <- a*X + B X,
    i.e. the odd polynomial p(s) = a s + b s^3 + c s^5 applied to every singular
    value of X.  X is m x n with the Gram side m (callers pass the short side
    first).
    Pins: SVD brute force (U p^K(S/||X||) V^T), rank-1 and scaled-identity
    closed forms, the cubic (1.5, -0.5) variant converging to the polar factor,
    orthogonal / scale / transpose equivariance.
    on_step: optional callable(k) run after iteration k (progress reporting
    for large inputs; it does not touch the arithmetic).
    """
    X = np.array(X, dtype=np.float64, copy=True)
    if X.size == 0:
        return X
    X = X / max(frobenius_norm(X), eps)
    for k in range(int(steps)):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
        if on_step is not None:
            on_step(k + 1)
    return X


def lr_multiplier(rows: int, cols: int, lr_adjust: str) -> float:
    """Shape-dependent factor on lr (torch.optim.Muon's adjust_lr_fn; the paper
    uses match_rms_adamw in §5.1 Setup)."""
    if lr_adjust == "original":
        return math.sqrt(max(1.0, rows / cols))
    if lr_adjust == "match_rms_adamw":
        return 0.2 * math.sqrt(max(rows, cols))
    if lr_adjust == "none":
        return 1.0
    raise ValueError(f"unknown lr_adjust {lr_adjust!r}")


def orthogonalize(U: np.ndarray, hp, on_step=None) -> np.ndarray:
    """Newton-Schulz in the short-side frame, returned in U's own frame."""
    rows, cols = U.shape
    transposed = rows > cols
    X = U.T if transposed else U
    O = newton_schulz(X, hp.ns_a, hp.ns_b, hp.ns_c, hp.ns_steps, hp.eps, on_step)
    return O.T if transposed else O


def muon_step(W: np.ndarray, G: np.ndarray, M: np.ndarray, hp, on_step=None):
    """One owner-side Muon step on one whole matrix.

    [P §3]: the owner holds the full reduced gradient, applies the Newton-Schulz
    update to the full matrix and updates its local weight and Muon state;
    [P §4.4]: ranks with an empty shard do nothing for it (an empty matrix is
    returned unchanged here).
    Returns (W', M', delta) with delta = lr_eff * O, so W' = (1-lr*wd)*W - delta.
    Pins: zero-gradient closed form W' = (1-lr*wd) W; torch.optim.Muon witness
    (bf16 Newton-Schulz, so only to 3e-2); the pins of newton_schulz.
    on_step: passed to newton_schulz (progress only).
    """
    W = np.asarray(W, np.float64)
    rows, cols = W.shape
    if rows == 0 or cols == 0:
        return W.copy(), np.asarray(M, np.float64).copy(), np.zeros_like(W)
    M_new, U = momentum(G, M, hp.momentum, hp.nesterov)
    O = orthogonalize(U, hp, on_step)
    lr_eff = hp.lr * lr_multiplier(rows, cols, hp.lr_adjust)
    delta = lr_eff * O
    W_new = (1.0 - hp.lr * hp.weight_decay) * W - delta
    return W_new, M_new, delta


def muon_bucket(mats: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]], hp):
    """The owner step over a bucket: every matrix is independent [P §3]."""
    return [muon_step(W, G, M, hp) for (W, G, M) in mats]
