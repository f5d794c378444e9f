"""fp64 oracle of the AdamW step on the packed non-2D tail (test infrastructure).

[P §3]: the non-2D tensors of an FSDP unit are packed into one tail role that
stays on the AdamW path; [P §5.1 Setup] gives its hyperparameters (lr, weight
decay, betas, eps).  AdamW is coordinate-wise, so packing changes nothing.

The update is decoupled-weight-decay Adam as published by Loshchilov and Hutter
(the paper's reference for AdamW), with bias correction folded into the step
size and eps added outside the square root, as torch.optim.AdamW does:
    p  <- p * (1 - lr*wd)
    m  <- beta1*m + (1-beta1)*g
    v  <- beta2*v + (1-beta2)*g^2
    p  <- p - (lr / bc1) * m / (sqrt(v) / sqrt(bc2) + eps),  bc_i = 1 - beta_i^t
Pins: torch.optim.AdamW in fp64 (library witness); the t = 1, m = v = 0 closed
form p' = p(1 - lr*wd) - lr * g / (|g| + eps).
"""
from __future__ import annotations

import math

import numpy as np


def adamw_step(p, g, m, v, step: int, lr: float, beta1: float, beta2: float,
               eps: float, weight_decay: float):
    p = np.asarray(p, np.float64)
    g = np.asarray(g, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    if step < 1:
        raise ValueError("step counts from 1")
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    p = p - (lr / bc1) * m / (np.sqrt(v) / math.sqrt(bc2) + eps)
    return p, m, v
