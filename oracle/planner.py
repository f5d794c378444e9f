"""Plain Python owner planner (test infrastructure only: imported by tests/ and
never by the library or its binding).

Follows "MatrixFSDP: communication-free matrix optimizers under ZeRO-3
parameter sharding":
  * §3 / §4.1: every FSDP block becomes roles, one per 2D matrix and one packed
    tail of its non-2D tensors; a greedy over each role's owner-resident numel
    picks the owner rank; RoleGreedy is the default, ScopeGreedy pools the roles
    of all blocks, CostAware takes the scope plan only within a workspace cap.
  * §4.2, the equations of the bandwidth model: gamma_B = max_r O_{B,r} /
    (P_B / W) and C_owner_B = (W - 1) max_r O_{B,r}.
The pages do not print the algorithm.  The readings (the same as the C ABI
documents): largest role first, ties in input order; each role to the rank with
the least numel so far, ties to the lowest rank; RoleGreedy walks the blocks in
increasing index with the load carried over; CostAware's cap applies to the
largest per-block owner share and defaults to the role plan's.  Roles are
(block, kind, rows, cols) tuples, kind 0 = matrix, 1 = tail (rows = numel).
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

Role = Tuple[int, int, int, int]


def numel(role: Role) -> int:
    return role[2] * role[3]


def _greedy(roles: Sequence[Role], indices: List[int], load: List[int], owner: List[int]) -> None:
    # largest first; Python's sort is stable, so equal sizes keep input order
    for i in sorted(indices, key=lambda k: -numel(roles[k])):
        best = 0
        for r in range(1, len(load)):
            if load[r] < load[best]:
                best = r
        owner[i] = best
        load[best] += numel(roles[i])


def role_greedy(roles: Sequence[Role], world: int) -> List[int]:
    owner = [-1] * len(roles)
    load = [0] * world
    for b in sorted({r[0] for r in roles}):
        _greedy(roles, [i for i, r in enumerate(roles) if r[0] == b], load, owner)
    return owner


def scope_greedy(roles: Sequence[Role], world: int) -> List[int]:
    owner = [-1] * len(roles)
    _greedy(roles, list(range(len(roles))), [0] * world, owner)
    return owner


def block_shares(roles: Sequence[Role], owner: Sequence[int]) -> Dict[Tuple[int, int], int]:
    """O_{B,r}: numel rank r owns in block B."""
    out: Dict[Tuple[int, int], int] = {}
    for role, r in zip(roles, owner):
        out[(role[0], r)] = out.get((role[0], r), 0) + numel(role)
    return out


def cost_aware(roles: Sequence[Role], world: int, block_cap: int = 0) -> List[int]:
    scope = scope_greedy(roles, world)
    role = role_greedy(roles, world)
    cap = block_cap if block_cap > 0 else max(block_shares(roles, role).values(), default=0)
    return scope if max(block_shares(roles, scope).values(), default=0) <= cap else role


def plan(roles: Sequence[Role], world: int, policy: str, block_cap: int = 0) -> List[int]:
    if policy == "role_greedy":
        return role_greedy(roles, world)
    if policy == "scope_greedy":
        return scope_greedy(roles, world)
    if policy == "cost_aware":
        return cost_aware(roles, world, block_cap)
    raise ValueError(policy)


def ns_flops(role: Role) -> float:
    """Nominal flops of one Newton-Schulz iteration (4 m^2 n + 2 m^3); 0 for a tail."""
    if role[1] != 0:
        return 0.0
    m, n = min(role[2], role[3]), max(role[2], role[3])
    return 4.0 * m * m * n + 2.0 * m ** 3


def score(roles: Sequence[Role], world: int, owner: Sequence[int]) -> dict:
    rank_numel = [0.0] * world
    rank_flops = [0.0] * world
    for role, r in zip(roles, owner):
        rank_numel[r] += numel(role)
        rank_flops[r] += ns_flops(role)
    n_blocks = 1 + max((role[0] for role in roles), default=-1)
    total = [0.0] * n_blocks
    for role in roles:
        total[role[0]] += numel(role)
    peak = [0.0] * n_blocks
    for (b, _), v in block_shares(roles, owner).items():
        peak[b] = max(peak[b], float(v))
    gamma = [peak[b] / (total[b] / world) if total[b] > 0 else 0.0 for b in range(n_blocks)]
    comm = [(world - 1) * peak[b] for b in range(n_blocks)]
    return {"rank_numel": rank_numel, "rank_flops": rank_flops, "block_gamma": gamma,
            "block_owner_comm": comm}


def layout(roles: Sequence[Role], owner: Sequence[int]) -> List[int]:
    """Offset of each role in its owner's block-local buffer, roles back to back
    in input order."""
    cursor: Dict[Tuple[int, int], int] = {}
    out = []
    for role, r in zip(roles, owner):
        key = (role[0], r)
        out.append(cursor.get(key, 0))
        cursor[key] = cursor.get(key, 0) + numel(role)
    return out
