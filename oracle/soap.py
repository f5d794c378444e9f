"""Plain fp64 SOAP owner step.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's CPU baseline, never by the library or its binding.

"MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
sharding", §5.7: next to Shampoo, the paper runs SOAP on the owners, which it
describes as Adam in the Shampoo eigenbasis.  The pages print no formulas.
The reading here follows the published SOAP algorithm (Vyas et al., 2024) with
the same statistics as the Shampoo reading of this package, and every choice
that algorithm leaves to its implementation taken in its plainest form:

  L' = L + G G^T,  R' = R + G^T G            Shampoo statistics (caller starts at eps I)
  Q_L, Q_R = eigenvectors of L', R'          the eigenbasis, recomputed every step
  M' = b1 M + (1 - b1) G                     first moment, kept in the weight's own frame
  G~ = Q_L^T G Q_R,  M~ = Q_L^T M' Q_R       gradient and first moment in the eigenbasis
  V' = b2 V + (1 - b2) G~ * G~               second moment, kept in the eigenbasis
  N~ = (M~ / (1 - b1^t)) / (sqrt(V' / (1 - b2^t)) + eps)
  W' = (1 - lr wd) W - lr Q_L N~ Q_R^T       decoupled decay

The update does not depend on the sign of the eigenvectors.  Once V is
non-zero it depends on their order (V is indexed by it): the eigenbasis is
taken in ascending eigenvalue order, numpy's eigh order.  It also depends on
the basis chosen inside a repeated eigenvalue wherever the rotated moments are
non-zero there (one step from eps I keeps them zero in the eps-eigenspace,
since G has no component there).
"""
from __future__ import annotations

import numpy as np


def eigenbasis(S: np.ndarray) -> np.ndarray:
    """Orthonormal eigenvectors of the symmetric S, ascending eigenvalues."""
    S = np.asarray(S, np.float64)
    _, V = np.linalg.eigh((S + S.T) / 2)
    return V


def soap_step(W, G, L, R, M, V, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
              eps: float = 1e-8, weight_decay: float = 0.0):
    """One owner step on one matrix; returns (W', L', R', M', V', lr * update) in fp64."""
    G = np.asarray(G, np.float64)
    L1 = np.asarray(L, np.float64) + G @ G.T
    R1 = np.asarray(R, np.float64) + G.T @ G
    QL, QR = eigenbasis(L1), eigenbasis(R1)
    M1 = beta1 * np.asarray(M, np.float64) + (1 - beta1) * G
    Gr = QL.T @ G @ QR
    Mr = QL.T @ M1 @ QR
    V1 = beta2 * np.asarray(V, np.float64) + (1 - beta2) * Gr * Gr
    Nr = (Mr / (1 - beta1 ** step)) / (np.sqrt(V1 / (1 - beta2 ** step)) + eps)
    D = lr * (QL @ Nr @ QR.T)
    W1 = (1 - lr * weight_decay) * np.asarray(W, np.float64) - D
    return W1, L1, R1, M1, V1, D
