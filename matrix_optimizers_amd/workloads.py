"""Seeded synthetic workloads for the owner-side Muon step and the AdamW tail.

This module only describes shapes, storage dtypes, hyperparameter values and how
the random inputs are drawn.  It holds none of the optimizer's arithmetic, so both
the HIP path's tests/bench and the fp64 oracle can take their inputs from here.

Shapes follow the decoder-transformer matrices the MatrixFSDP paper trains
("MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
sharding", §5.1 Setup: every 2D weight of a block is one Muon role, the non-2D
tensors form the AdamW tail, §3).  The pages print no input distributions; the
ones below are the plain reading used throughout: weights N(0, 0.02^2), gradients
and momenta N(0, 1e-3^2), values drawn in fp64 and rounded to nearest-even into
the storage dtype.

Random streams: numpy ``default_rng(SeedSequence([workload_seed, matrix_index,
role]))`` with role 0 = W, 1 = G, 2 = M, 3 = per-matrix gradient scale,
4..7 = AdamW tail p, g, m, v.  For the multi-GB workloads a GPU generator
(``torch.Generator`` seeded the same way, hashed to one integer) is offered for
benchmarking; parity tests at those sizes read the generated tensors back.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

F32 = "f32"
BF16 = "bf16"

ROLE_W, ROLE_G, ROLE_M, ROLE_SCALE = 0, 1, 2, 3
ROLE_P, ROLE_TG, ROLE_TM, ROLE_TV = 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class MuonHP:
    """Muon hyperparameters.  Defaults are torch.optim.Muon's documented defaults,
    the optimizer the paper runs on its owners (§5.1 Setup names torch.optim.Muon)."""
    lr: float = 0.02
    weight_decay: float = 0.01
    momentum: float = 0.95
    nesterov: bool = True
    ns_steps: int = 5
    ns_a: float = 3.4445
    ns_b: float = -4.7750
    ns_c: float = 2.0315
    eps: float = 1e-7
    lr_adjust: str = "original"      # "original" | "match_rms_adamw" | "none"
    ns_dtype: str = BF16             # "bf16" | "f32"


@dataclasses.dataclass(frozen=True)
class AdamWHP:
    """AdamW hyperparameters of the paper's non-matrix tail (§5.1 Setup)."""
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 1e-2
    step: int = 10


@dataclasses.dataclass(frozen=True)
class MatrixSpec:
    rows: int
    cols: int
    name: str = ""


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    seed: int
    matrices: Tuple[MatrixSpec, ...]
    w_dtype: str
    g_dtype: str
    hp: MuonHP
    w_std: float = 0.02
    g_std: float = 1e-3
    m_std: float = 1e-3            # 0.0 => momentum starts at zero
    g_scale_loguniform: Optional[Tuple[float, float]] = None
    tail: Tuple[int, ...] = ()     # lengths of the fp32 non-2D tail tensors
    adamw: AdamWHP = AdamWHP()
    description: str = ""

    @property
    def tail_numel(self) -> int:
        return int(sum(self.tail))


def _decoder_layer(h: int, ffn: int, kv: int) -> List[MatrixSpec]:
    return [MatrixSpec(h, h, "wq"), MatrixSpec(kv, h, "wk"), MatrixSpec(kv, h, "wv"),
            MatrixSpec(h, h, "wo"), MatrixSpec(ffn, h, "w_gate"), MatrixSpec(ffn, h, "w_up"),
            MatrixSpec(h, ffn, "w_down")]


def _build() -> dict:
    w = {}
    w["single_256x512_f32"] = Workload(
        key="single_256x512_f32", seed=1, matrices=(MatrixSpec(256, 512, "w"),),
        w_dtype=F32, g_dtype=F32, hp=MuonHP(ns_dtype=F32), g_std=1.0, m_std=0.0,
        description="one 256x512 fp32 matrix, fp32 Newton-Schulz, zero momentum")
    w["decoder_layer_h2048"] = Workload(
        key="decoder_layer_h2048", seed=2, matrices=tuple(_decoder_layer(2048, 5632, 2048)),
        w_dtype=BF16, g_dtype=BF16, hp=MuonHP(), tail=(2048, 2048),
        description="one decoder-layer owner bucket, hidden 2048, FFN 5632, tail 2x2048 fp32")
    mats = [MatrixSpec(1024, 1024, f"sq{i}") for i in range(64)] + \
           [MatrixSpec(1024, 4096, f"wide{i}") for i in range(64)]
    w["batched_1024"] = Workload(
        key="batched_1024", seed=3, matrices=tuple(mats), w_dtype=BF16, g_dtype=BF16,
        hp=MuonHP(), g_scale_loguniform=(1e-4, 1e-1),
        description="64x(1024x1024) + 64x(1024x4096), per-matrix log-uniform gradient scale")
    layers = []
    for _ in range(4):
        layers += _decoder_layer(4096, 14336, 1024)
    w["llama8b_4layers"] = Workload(
        key="llama8b_4layers", seed=4, matrices=tuple(layers), w_dtype=BF16, g_dtype=BF16,
        hp=MuonHP(), tail=(4096,) * 8,
        description="Llama-3-8B-shaped owner share of 4 layers (GQA kv 1024), tail 8x4096 fp32")
    w["large_single"] = Workload(
        key="large_single", seed=5,
        matrices=(MatrixSpec(28672, 8192, "mlp_up"), MatrixSpec(8192, 28672, "mlp_down"),
                  MatrixSpec(128256, 4096, "head")),
        w_dtype=BF16, g_dtype=BF16, hp=MuonHP(),
        description="28672x8192, 8192x28672 and a 128256x4096 output head")
    # The paper's own timing settings (§5.1 Setup): momentum 0.5, two NS steps,
    # match_rms_adamw lr adjustment, lr 1e-3, wd 1e-2; on one rank's share of the
    # 16-layer hidden-4096 / intermediate-16384 model (4 square + 2 MLP matrices per
    # layer, 16 layers over 8 ranks = 2 layers per rank).
    paper = []
    for _ in range(2):
        paper += [MatrixSpec(4096, 4096, "q"), MatrixSpec(4096, 4096, "k"),
                  MatrixSpec(4096, 4096, "v"), MatrixSpec(4096, 4096, "o"),
                  MatrixSpec(16384, 4096, "up"), MatrixSpec(4096, 16384, "down")]
    w["paper_owner_share"] = Workload(
        key="paper_owner_share", seed=6, matrices=tuple(paper), w_dtype=BF16, g_dtype=BF16,
        hp=MuonHP(lr=1e-3, weight_decay=1e-2, momentum=0.5, ns_steps=2,
                  lr_adjust="match_rms_adamw"),
        description="one rank's share of the paper's 16-layer 3.2B timing model, paper settings")
    return w


WORKLOADS = _build()
WORKLOAD_ORDER = ["single_256x512_f32", "decoder_layer_h2048", "batched_1024",
                  "llama8b_4layers", "large_single"]

# The paper's timing and ablation model (§5.1 Setup): Qwen-style decoder layers,
# hidden 4096, intermediate 16384, 32 heads; per layer 4 square attention
# matrices, the MLP up (16384 x 4096) and down (4096 x 16384) matrices, and the
# layer's two hidden-size norm vectors packed into its tail role (§3).  16 layers
# give the 3.2B model of §5.2, 64 the 12.9B model of §5.6.
PAPER_LAYER = ((4096, 4096, "q"), (4096, 4096, "k"), (4096, 4096, "v"), (4096, 4096, "o"),
               (16384, 4096, "up"), (4096, 16384, "down"))
PAPER_LAYER_TAIL = 2 * 4096
ROLE_MATRIX, ROLE_TAIL = 0, 1


def paper_model_roles(layers: int) -> List[Tuple[int, int, int, int]]:
    """Planner roles (block, kind, rows, cols) of the paper's model, one block per layer."""
    roles = []
    for b in range(layers):
        roles += [(b, ROLE_MATRIX, r, c) for r, c, _ in PAPER_LAYER]
        roles.append((b, ROLE_TAIL, PAPER_LAYER_TAIL, 1))
    return roles


def planned_max_rank(layers: int, world: int, policy: str = "role_greedy") -> Workload:
    """The bucket of the rank with the most Newton-Schulz work when the library's
    owner planner places the paper's model over `world` ranks: the step time of
    the whole data-parallel group is that rank's.  Paper settings (§5.1)."""
    from . import _binding as B   # the C++ planner of libmo.so
    roles = paper_model_roles(layers)
    owner = B.plan_owners(roles, world, policy)
    flops = B.plan_score(roles, world, owner)["rank_flops"]
    top = max(range(world), key=lambda r: (flops[r], -r))
    names = {(b, k): name for b in range(layers) for k, (_, _, name) in enumerate(PAPER_LAYER)}
    mats, tail, k_in_block = [], [], {}
    for i, ((b, kind, rows, cols), o) in enumerate(zip(roles, owner)):
        if kind == ROLE_MATRIX:
            k = k_in_block.get(b, 0)
            k_in_block[b] = k + 1
            if o == top:
                mats.append(MatrixSpec(rows, cols, f"L{b}.{names[(b, k)]}"))
        elif o == top:
            tail.append(rows)
    return Workload(
        key=f"paper_planned_max_rank", seed=7, matrices=tuple(mats), w_dtype=BF16, g_dtype=BF16,
        hp=MuonHP(lr=1e-3, weight_decay=1e-2, momentum=0.5, ns_steps=2, lr_adjust="match_rms_adamw"),
        tail=tuple(tail),
        description=f"rank {top}'s bucket (most NS work) of the paper's {layers}-layer model over "
                    f"{world} ranks, {policy} owner plan, paper settings")


def get(key: str) -> Workload:
    if key == "paper_planned_max_rank":
        if key not in WORKLOADS:
            WORKLOADS[key] = planned_max_rank(16, 8)
        return WORKLOADS[key]
    return WORKLOADS[key]


# ----------------------------------------------------------------------------
# Shampoo on the owners (§5.7)
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ShampooHP:
    """Shampoo settings.  The pages run Shampoo on the owners in float32 (§5.7)
    without printing its settings; the plain reading used here: lr 1e-3 (the
    paper's Muon timing lr), no weight decay, statistics started at eps I with
    eps = 1e-6 (about 1e-4 of the largest eigenvalue of G G^T for N(0, 1e-3^2)
    gradients with a side of 1024 to 2048), and 20 coupled Newton steps per
    inverse root."""
    lr: float = 1e-3
    weight_decay: float = 0.0
    eps: float = 1e-6
    root_iters: int = 20


@dataclasses.dataclass(frozen=True)
class ShampooWorkload:
    key: str
    seed: int
    matrices: Tuple[MatrixSpec, ...]
    w_dtype: str = F32
    g_dtype: str = F32
    hp: ShampooHP = ShampooHP()
    w_std: float = 0.02
    g_std: float = 1e-3
    description: str = ""


SHAMPOO_WORKLOADS = {
    "shampoo_mixed_small": ShampooWorkload(
        key="shampoo_mixed_small", seed=11,
        matrices=(MatrixSpec(256, 512, "a"), MatrixSpec(300, 200, "b"), MatrixSpec(77, 1000, "c"),
                  MatrixSpec(513, 513, "d"), MatrixSpec(1, 300, "e")),
        description="five small fp32 matrices with ragged sides (tiles, tails and a single row)"),
    "shampoo_decoder_layer_h2048": ShampooWorkload(
        key="shampoo_decoder_layer_h2048", seed=12, matrices=tuple(_decoder_layer(2048, 5632, 2048)),
        description="one decoder-layer owner bucket, hidden 2048, FFN 5632, fp32 weights and gradients"),
    # One layer of the paper's model (§5.1: hidden 4096, intermediate 16384;
    # 4 square attention matrices, MLP up and down), the shapes of its Shampoo
    # run (§5.7); the up/down roots are 16384-sided.
    "shampoo_paper_layer": ShampooWorkload(
        key="shampoo_paper_layer", seed=13,
        matrices=(MatrixSpec(4096, 4096, "q"), MatrixSpec(4096, 4096, "k"), MatrixSpec(4096, 4096, "v"),
                  MatrixSpec(4096, 4096, "o"), MatrixSpec(16384, 4096, "up"), MatrixSpec(4096, 16384, "down")),
        description="one layer of the paper's hidden-4096 / intermediate-16384 model, fp32"),
}


def shampoo_inputs(wl: ShampooWorkload, index: int):
    """(W, G) for matrix `index` (fp32 arrays holding the storage dtype's values)
    and the initial statistics eps I_rows, eps I_cols."""
    spec = wl.matrices[index]
    shape = (spec.rows, spec.cols)
    W = normal(wl.seed, index, ROLE_W, shape, wl.w_std, wl.w_dtype)
    G = normal(wl.seed, index, ROLE_G, shape, wl.g_std, wl.g_dtype)
    L = (wl.hp.eps * np.eye(spec.rows)).astype(np.float32)
    R = (wl.hp.eps * np.eye(spec.cols)).astype(np.float32)
    return W, G, L, R


def shampoo_flops_algorithmic(rows: int, cols: int, root_iters: int) -> dict:
    """Per product kind, the flops one step spends on one matrix as the library
    computes it: one triangle of a symmetric product (m^3 for an m x m root
    product, m^2 k for a statistics product with K extent k), 2 m n k for a
    full one.  Per root and coupled Newton step after the first: S2, S4 and M
    symmetric, H full (5 m^3)."""
    out = {"stats": float(rows) ** 2 * cols + float(cols) ** 2 * rows,
           "root": 0.0, "left": 2.0 * rows * rows * cols, "right": 2.0 * rows * cols * cols}
    for m in (rows, cols):
        out["root"] += 5.0 * (root_iters - 1) * float(m) ** 3
    return out


@dataclasses.dataclass(frozen=True)
class SoapHP:
    """SOAP settings.  The pages run SOAP on the owners (§5.7) without printing
    its settings; the plain reading: Adam's defaults (lr 1e-3, betas 0.9 and
    0.999, eps 1e-8), no weight decay, statistics started at eps I with
    eps = 1e-6 (as the Shampoo workloads), 14 outer Jacobi sweeps (the
    decoder-layer sides converge to fp32 resolution within 12)."""
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    stat_eps: float = 1e-6
    sweeps: int = 14


@dataclasses.dataclass(frozen=True)
class SoapWorkload:
    key: str
    seed: int
    matrices: Tuple[MatrixSpec, ...]
    w_dtype: str = F32
    g_dtype: str = F32
    hp: SoapHP = SoapHP()
    w_std: float = 0.02
    g_std: float = 1e-3
    description: str = ""


SOAP_WORKLOADS = {
    "soap_decoder_layer_h2048": SoapWorkload(
        key="soap_decoder_layer_h2048", seed=14, matrices=tuple(_decoder_layer(2048, 5632, 2048)),
        description="one decoder-layer owner bucket, hidden 2048, FFN 5632, fp32 weights and gradients"),
    # One layer of the paper's model (hidden 4096, intermediate 16384), as in
    # the Shampoo workload of the same name: two 16384-sided statistics.
    "soap_paper_layer": SoapWorkload(
        key="soap_paper_layer", seed=15,
        matrices=(MatrixSpec(4096, 4096, "q"), MatrixSpec(4096, 4096, "k"), MatrixSpec(4096, 4096, "v"),
                  MatrixSpec(4096, 4096, "o"), MatrixSpec(16384, 4096, "up"), MatrixSpec(4096, 16384, "down")),
        description="one layer of the paper's hidden-4096 / intermediate-16384 model, fp32"),
}


def soap_jacobi_flops(m: int, sweeps: int) -> dict:
    """Flops of the blocked Jacobi eigensolver on one side m as built: per round,
    every upper 64 x 64 tile pair of A takes two 64^3 products (C = X + X D_J,
    A' = C + D_I^T C) and every 64 x 64 tile of E one; the pair problems take
    one scalar sweep of 63 steps over a 64 x 64 matrix, each step about 6 flops
    per element of S and of D (counted as 12 * 64^2 per step)."""
    P = (m + 63) // 64
    rounds = sweeps * (2 * P - 1)
    t3 = 2.0 * 64 ** 3
    apply = rounds * P * (P + 1) / 2 * 2 * t3
    etile = rounds * P * P * t3
    solve = rounds * P * 63 * 12.0 * 64 * 64
    return {"apply": apply, "etile": etile, "solve": solve, "rounds": rounds}


def soap_jacobi_bytes(m: int, sweeps: int) -> dict:
    """Algorithmic HBM bytes of the rotation launches on one side m: every round
    reads and writes the upper 32 x 32 blocks of A (fp64, 2P (2P + 1) / 2
    blocks) and all of E (fp32, m_pad x m_pad); the pair rotations D, 64 x 64
    each, are small and L2-resident."""
    P = (m + 63) // 64
    nb = 2 * P
    rounds = sweeps * (nb - 1)
    a_bytes = nb * (nb + 1) / 2 * 32 * 32 * 8
    e_bytes = (64.0 * P) ** 2 * 4
    return {"per_round": 2 * (a_bytes + e_bytes), "rounds": rounds}


def soap_product_flops(rows: int, cols: int) -> float:
    """The two statistics products and the six eigenbasis products (fp32), as
    computed on the padded sides."""
    r = (rows + 63) // 64 * 64
    c = (cols + 63) // 64 * 64
    return 2.0 * r * r * c + 2.0 * c * c * r + 3 * (2.0 * r * r * c + 2.0 * r * c * c)


# ----------------------------------------------------------------------------
# value generation
# ----------------------------------------------------------------------------

def rng_for(seed: int, index: int, role: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, index, role]))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 storage."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def store(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 draw -> value held in the storage dtype (returned as fp32 array)."""
    x32 = x64.astype(np.float32)          # round to nearest fp32
    return round_to_bf16(x32) if dtype == BF16 else x32


def normal(seed: int, index: int, role: int, shape, std: float, dtype: str) -> np.ndarray:
    if std == 0.0:
        return np.zeros(shape, np.float32)
    g = rng_for(seed, index, role).standard_normal(size=shape) * std
    return store(g, dtype)


def grad_scale(wl: Workload, index: int) -> float:
    if wl.g_scale_loguniform is None:
        return 1.0
    lo, hi = wl.g_scale_loguniform
    u = rng_for(wl.seed, index, ROLE_SCALE).uniform()
    return float(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))


@dataclasses.dataclass
class MatrixInputs:
    W: np.ndarray     # fp32 array holding values of wl.w_dtype
    G: np.ndarray     # fp32 array holding values of wl.g_dtype
    M: np.ndarray     # fp32 momentum


def matrix_inputs(wl: Workload, index: int, spec: Optional[MatrixSpec] = None) -> MatrixInputs:
    spec = spec or wl.matrices[index]
    shape = (spec.rows, spec.cols)
    W = normal(wl.seed, index, ROLE_W, shape, wl.w_std, wl.w_dtype)
    s = grad_scale(wl, index)
    if s == 1.0:
        G = normal(wl.seed, index, ROLE_G, shape, wl.g_std, wl.g_dtype)
    else:
        g = rng_for(wl.seed, index, ROLE_G).standard_normal(size=shape) * (wl.g_std * s)
        G = store(g, wl.g_dtype)
    M = normal(wl.seed, index, ROLE_M, shape, wl.m_std, F32)
    return MatrixInputs(W, G, M)


@dataclasses.dataclass
class TailInputs:
    p: np.ndarray
    g: np.ndarray
    m: np.ndarray
    v: np.ndarray


def tail_inputs(seed: int, n: int) -> TailInputs:
    """AdamW tail state: p ~ N(0, 0.02^2), g, m ~ N(0, 1e-3^2), v = N(0, 1e-3^2)^2."""
    shape = (n,)
    p = normal(seed, 0, ROLE_P, shape, 0.02, F32)
    g = normal(seed, 0, ROLE_TG, shape, 1e-3, F32)
    m = normal(seed, 0, ROLE_TM, shape, 1e-3, F32)
    v = normal(seed, 0, ROLE_TV, shape, 1e-3, F32)
    v = (v * v).astype(np.float32)
    return TailInputs(p, g, m, v)


def torch_seed(seed: int, index: int, role: int) -> int:
    """One integer seed for torch.Generator, derived from the same triple."""
    ss = np.random.SeedSequence([seed, index, role])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def ns_flops_nominal(rows: int, cols: int, steps: int) -> float:
    """4 m^2 n + 2 m^3 per Newton-Schulz step, m = min side (dense GEMM count)."""
    m, n = min(rows, cols), max(rows, cols)
    return float(steps) * (4.0 * m * m * n + 2.0 * m ** 3)


def ns_flops_algorithmic(rows: int, cols: int, steps: int) -> float:
    """Symmetry-aware count: X X^T and A A need only one triangle (m^2 n, m^3),
    B X is dense (2 m^2 n)."""
    m, n = min(rows, cols), max(rows, cols)
    return float(steps) * (3.0 * m * m * n + 1.0 * m ** 3)


# ----------------------------------------------------------------------------
# on-device generation for the multi-GB workloads (benchmarks and full-size
# property tests); same distributions, torch's Philox stream instead of numpy's
# ----------------------------------------------------------------------------

def torch_normal(seed: int, index: int, role: int, shape, std: float, dtype: str, device):
    import torch
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    if std == 0.0:
        return torch.zeros(shape, dtype=tdt, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, index, role))
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    x.mul_(std)
    return x.to(tdt)          # round to nearest even into the storage dtype


def torch_matrix_inputs(wl: Workload, index: int, device, spec: Optional[MatrixSpec] = None):
    """(W, G, M) device tensors for matrix `index` of `wl`, drawn on the device."""
    spec = spec or wl.matrices[index]
    shape = (spec.rows, spec.cols)
    W = torch_normal(wl.seed, index, ROLE_W, shape, wl.w_std, wl.w_dtype, device)
    G = torch_normal(wl.seed, index, ROLE_G, shape, wl.g_std * grad_scale(wl, index),
                     wl.g_dtype, device)
    M = torch_normal(wl.seed, index, ROLE_M, shape, wl.m_std, F32, device)
    return W, G, M


def torch_tail_inputs(seed: int, n: int, device):
    import torch
    p = torch_normal(seed, 0, ROLE_P, (n,), 0.02, F32, device)
    g = torch_normal(seed, 0, ROLE_TG, (n,), 1e-3, F32, device)
    m = torch_normal(seed, 0, ROLE_TM, (n,), 1e-3, F32, device)
    v = torch_normal(seed, 0, ROLE_TV, (n,), 1e-3, F32, device)
    v.mul_(v)
    return p, g, m, v
