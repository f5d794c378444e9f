"""Helpers for the GPU parity tests: run the HIP path through the C ABI (via the
binding) and the fp64 oracle on the same stored inputs, and compare.

Tolerances (relative Frobenius norm):
  * the update delta = lr_eff * O: 3e-2 with bf16 Newton-Schulz operands, 1e-4
    with fp32 ones;
  * the momentum buffer M': 1e-6 (one fp32 fma chain per element);
  * W': the written weight must equal round(decay * W - delta_gpu) in W's dtype
    to within one unit in the last place per element plus the fp32 rounding of
    the two operands (the fp32 evaluation order may differ, and the operands can
    cancel), and delta_gpu is checked against the oracle above.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from matrix_optimizers_amd import workloads as wlmod
from oracle import muon as omuon

TOL = {"bf16": 3e-2, "f32": 1e-4}
TOL_M = 1e-6


def f32(x: float) -> float:
    return float(np.float32(x))


def hp_f32(hp: wlmod.MuonHP) -> wlmod.MuonHP:
    """The hyperparameters as the fp32 values the library receives."""
    return dataclasses.replace(hp, lr=f32(hp.lr), weight_decay=f32(hp.weight_decay),
                               momentum=f32(hp.momentum), ns_a=f32(hp.ns_a), ns_b=f32(hp.ns_b),
                               ns_c=f32(hp.ns_c), eps=f32(hp.eps))


def hp_kwargs(hp: wlmod.MuonHP) -> dict:
    return dict(lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                nesterov=hp.nesterov, ns_steps=hp.ns_steps,
                ns_coefficients=(hp.ns_a, hp.ns_b, hp.ns_c), eps=hp.eps,
                adjust_lr_fn=hp.lr_adjust, ns_dtype=hp.ns_dtype)


def torch_dtype(name: str):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_dev(x: np.ndarray, dtype: str, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device).to(torch_dtype(dtype))


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel(a: np.ndarray, b: np.ndarray) -> float:
    den = float(np.linalg.norm(b))
    num = float(np.linalg.norm(a - b))
    return num / den if den > 0 else num


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


@dataclasses.dataclass
class Case:
    W: np.ndarray
    G: np.ndarray
    M: np.ndarray
    w_dtype: str
    g_dtype: str


def random_case(rows: int, cols: int, w_dtype: str, g_dtype: str, seed: int,
                g_std: float = 1e-3, m_std: float = 1e-3) -> Case:
    W = wlmod.normal(seed, 0, wlmod.ROLE_W, (rows, cols), 0.02, w_dtype)
    G = wlmod.normal(seed, 0, wlmod.ROLE_G, (rows, cols), g_std, g_dtype)
    M = wlmod.normal(seed, 0, wlmod.ROLE_M, (rows, cols), m_std, "f32")
    return Case(W, G, M, w_dtype, g_dtype)


def run_gpu(cases: Sequence[Case], hp: wlmod.MuonHP, device, with_update: bool = True,
            strided: bool = False):
    """Returns [(W', M', delta or None)] as fp64 host arrays."""
    import torch
    import matrix_optimizers_amd as mo
    mats, ups, keep = [], [], []
    for c in cases:
        if strided and c.W.size:
            pad = 24
            rows, cols = c.W.shape
            bigW = torch.zeros((rows, cols + pad), dtype=torch_dtype(c.w_dtype), device=device)
            bigG = torch.zeros((rows, cols + pad), dtype=torch_dtype(c.g_dtype), device=device)
            bigM = torch.zeros((rows, cols + pad), dtype=torch.float32, device=device)
            W = bigW[:, 3:3 + cols]
            G = bigG[:, 5:5 + cols]
            M = bigM[:, 1:1 + cols]
            W.copy_(to_dev(c.W, c.w_dtype, device))
            G.copy_(to_dev(c.G, c.g_dtype, device))
            M.copy_(to_dev(c.M, "f32", device))
            keep += [bigW, bigG, bigM]
        else:
            W = to_dev(c.W, c.w_dtype, device)
            G = to_dev(c.G, c.g_dtype, device)
            M = to_dev(c.M, "f32", device)
        mats.append((W, G, M))
        ups.append(torch.full(c.W.shape, float("nan"), dtype=torch.float32, device=device)
                   if with_update else None)
    mo.muon_owner_step(mats, update_out=ups if with_update else None, **hp_kwargs(hp))
    torch.cuda.synchronize()
    return [(to_host(W), to_host(M), to_host(U) if U is not None else None)
            for (W, G, M), U in zip(mats, ups)]


def check_case(c: Case, got, hp: wlmod.MuonHP, tol: Optional[float] = None, on_step=None) -> dict:
    """Compare one GPU result with the oracle; returns the measured errors.
    on_step: progress callback of the oracle's Newton-Schulz loop."""
    W1, M1, D1 = got
    hpo = hp_f32(hp)
    Wo, Mo, Do = omuon.muon_step(c.W.astype(np.float64), c.G.astype(np.float64),
                                 c.M.astype(np.float64), hpo, on_step=on_step)
    tol = TOL[hp.ns_dtype] if tol is None else tol
    out = {}
    if c.W.size == 0:
        assert W1.shape == c.W.shape
        return out
    out["delta"] = rel(D1, Do)
    out["momentum"] = rel(M1, Mo)
    assert out["momentum"] <= TOL_M, out
    assert out["delta"] <= tol, out
    # the weight write is decay * W - delta in fp32, rounded to W's dtype
    decay = np.float32(1.0 - np.float64(np.float32(hp.lr)) * np.float64(np.float32(hp.weight_decay)))
    want = (decay * c.W.astype(np.float32) - D1.astype(np.float32)).astype(np.float64)
    if c.w_dtype == "bf16":
        # One bf16 spacing at the larger magnitude (a 1-ulp difference of the
        # fp32 evaluation can cross a rounding boundary or a binade), plus the
        # fp32 rounding of the two operands, which dominates when they cancel.
        op = np.maximum(np.abs(decay * c.W.astype(np.float64)), np.abs(D1))
        allow = bf16_ulp(np.maximum(np.abs(W1), np.abs(want))) + 4 * 2.0 ** -24 * op
        err = np.abs(W1 - want) / allow
        out["w_ulps"] = float(err.max())
        if out["w_ulps"] > 1.0:
            worst = np.argsort(err.ravel())[-4:]
            rows = [(int(k) // W1.shape[1], int(k) % W1.shape[1], float(c.W.ravel()[k]),
                     float(D1.ravel()[k]), float(want.ravel()[k]), float(W1.ravel()[k]))
                    for k in worst]
            out["worst(row,col,W,delta,want,got)"] = rows
        assert out["w_ulps"] <= 1.0, out
    else:
        out["w_rel"] = rel(W1, want)
        assert out["w_rel"] <= 1e-6, out
    return out
