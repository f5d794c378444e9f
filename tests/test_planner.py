"""The owner planner (C ABI, host only) against the plain Python planner in
oracle/planner.py, and both against what the paper fixes: its model sizes, the
balance figures of its planner ablation, the bandwidth-model equations, and the
greedy's scheduling bound.  CPU only."""
import itertools
import random

import pytest

import matrix_optimizers_amd as mo
from matrix_optimizers_amd import workloads as wlmod
from oracle import planner as oplan

POLICIES = ["role_greedy", "scope_greedy", "cost_aware"]


def random_model(seed, blocks, world_hint=8):
    rng = random.Random(seed)
    roles = []
    for b in range(blocks):
        for _ in range(rng.randint(0, 7)):
            roles.append((b, 0, rng.choice([1, 64, 512, 1024, 4096, 5000]), rng.choice([1, 256, 1024, 4096, 14336])))
        if rng.random() < 0.8:
            roles.append((b, 1, rng.randint(0, 20000), 1))
    rng.shuffle(roles)   # blocks interleaved in the array
    return roles


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("policy", POLICIES)
def test_matches_python_planner(seed, policy):
    roles = random_model(seed, blocks=1 + seed % 9)
    for world in (1, 2, 3, 8, 13):
        cap = [0, 10 ** 7][seed % 2]
        assert mo.plan_owners(roles, world, policy, cap) == oplan.plan(roles, world, policy, cap)


@pytest.mark.parametrize("layers,world", [(16, 8), (64, 8), (64, 16), (64, 32), (64, 64)])
@pytest.mark.parametrize("policy", POLICIES)
def test_paper_model_plans_and_scores_match(layers, world, policy):
    roles = wlmod.paper_model_roles(layers)
    owner = mo.plan_owners(roles, world, policy)
    assert owner == oplan.plan(roles, world, policy)
    got, want = mo.plan_score(roles, world, owner), oplan.score(roles, world, owner)
    for k in want:
        assert got[k] == pytest.approx(want[k], rel=1e-12, abs=0), k
    assert mo.plan_layout(roles, world, owner) == oplan.layout(roles, owner)


def test_paper_model_sizes():
    """§5.2 and §5.6 name a 16-layer 3.2B and a 64-layer 12.9B model of these
    layers: the role shapes reproduce both parameter counts."""
    count = lambda L: sum(r * c for _, _, r, c in wlmod.paper_model_roles(L))
    assert round(count(16) / 1e9, 1) == 3.2
    assert round(count(64) / 1e9, 1) == 12.9


# §5.8 Table 5: per-rank optimizer-compute max/avg imbalance of the role-,
# scope- and cost-aware planners on the 64-layer model, by shard span.
TABLE5 = {8: (1.07, 1.02, 1.07), 16: (1.05, 1.02, 1.05), 32: (1.12, 1.03, 1.11), 64: (1.27, 1.04, 1.27)}


@pytest.mark.parametrize("world", sorted(TABLE5))
def test_table5_balance(world):
    """The pages report measured step-time ratios; the planner's modeled compute
    ratio (NS flops per rank, max / mean) should land within 0.05 of the role
    and cost-aware columns, and the scope plan should be at least as flat as
    measured."""
    roles = wlmod.paper_model_roles(64)
    ratio = {}
    for policy in POLICIES:
        fl = oplan.score(roles, world, oplan.plan(roles, world, policy))["rank_flops"]
        ratio[policy] = max(fl) / (sum(fl) / world)
    r, s, c = TABLE5[world]
    assert abs(ratio["role_greedy"] - r) <= 0.05, ratio
    assert abs(ratio["cost_aware"] - c) <= 0.05, ratio
    assert ratio["scope_greedy"] <= s, ratio
    assert ratio["scope_greedy"] <= ratio["role_greedy"]


def test_scope_plan_is_flatter_but_concentrates_blocks():
    """§4.1: ScopeGreedy improves global balance, RoleGreedy is the
    memory-conservative default: the scope plan has the lower rank imbalance
    and the higher per-block owner imbalance gamma_B."""
    roles = wlmod.paper_model_roles(16)
    sc = {p: oplan.score(roles, 8, oplan.plan(roles, 8, p)) for p in ("role_greedy", "scope_greedy")}
    imb = {p: max(v["rank_numel"]) / (sum(v["rank_numel"]) / 8) for p, v in sc.items()}
    assert imb["scope_greedy"] < imb["role_greedy"]
    assert max(sc["scope_greedy"]["block_gamma"]) > max(sc["role_greedy"]["block_gamma"])


def _makespan(roles, world, owner):
    load = [0] * world
    for role, o in zip(roles, owner):
        load[o] += oplan.numel(role)
    return max(load)


@pytest.mark.parametrize("seed", range(40))
def test_scope_greedy_within_graham_bound(seed):
    """ScopeGreedy is largest-first list scheduling: its largest rank load is at
    most (4/3 - 1/(3W)) of the optimum (Graham 1969), checked against brute
    force on small instances; it also never exceeds mean + largest role."""
    rng = random.Random(seed)
    world = rng.choice([2, 3])
    roles = [(0, 0, rng.randint(1, 40), rng.randint(1, 40)) for _ in range(rng.randint(1, 8))]
    for owner in (mo.plan_owners(roles, world, "scope_greedy"), oplan.scope_greedy(roles, world)):
        got = _makespan(roles, world, owner)
        opt = min(_makespan(roles, world, a) for a in itertools.product(range(world), repeat=len(roles)))
        assert got <= (4 / 3 - 1 / (3 * world)) * opt + 1e-9
        total = sum(oplan.numel(r) for r in roles)
        assert got <= total / world + max(oplan.numel(r) for r in roles)


def test_bandwidth_model_equations():
    """§4.2: gamma_B = max_r O_{B,r} / (P_B / W) and C_owner = (W - 1) max_r O_{B,r},
    on a hand-made block: P_B = 100 over W = 4, one rank owning 70."""
    roles = [(0, 0, 10, 7), (0, 0, 10, 2), (0, 1, 10, 1), (1, 0, 5, 8)]
    owner = [2, 0, 1, 3]
    sc = mo.plan_score(roles, 4, owner)
    assert sc["block_gamma"][0] == pytest.approx(70 / 25)
    assert sc["block_owner_comm"][0] == 3 * 70
    assert sc["block_gamma"][1] == pytest.approx(40 / 10)
    assert sc["rank_numel"] == [20, 10, 70, 40]
    assert sc["rank_flops"][2] == 4 * 7 * 7 * 10 + 2 * 7 ** 3   # m = 7, n = 10
    assert sc["rank_flops"][1] == 0                               # a tail has no NS work


def test_ties_go_round_robin_in_input_order():
    roles = [(0, 0, 8, 8)] * 5 + [(1, 0, 8, 8)] * 3
    assert mo.plan_owners(roles, 3, "scope_greedy") == [0, 1, 2, 0, 1, 2, 0, 1]
    assert mo.plan_owners(roles, 3, "role_greedy") == [0, 1, 2, 0, 1, 2, 0, 1]


def test_cost_aware_cap():
    roles = wlmod.paper_model_roles(8)
    scope, role = oplan.scope_greedy(roles, 8), oplan.role_greedy(roles, 8)
    peak = max(oplan.block_shares(roles, scope).values())
    assert mo.plan_owners(roles, 8, "cost_aware", peak) == scope
    assert mo.plan_owners(roles, 8, "cost_aware", peak - 1) == role


@pytest.mark.parametrize("policy", POLICIES)
def test_layout_is_one_contiguous_segment_per_parameter(policy):
    """§4.1: each emitted block layout holds one contiguous local segment per
    parameter: a rank's owned roles of a block tile its block buffer back to
    back, and a role it does not own has no segment there."""
    roles = random_model(99, blocks=6)
    owner = mo.plan_owners(roles, 5, policy)
    offs = mo.plan_layout(roles, 5, owner)
    spans = {}
    for role, o, off in zip(roles, owner, offs):
        spans.setdefault((role[0], o), []).append((off, oplan.numel(role)))
    for seg in spans.values():
        pos = 0
        for off, n in seg:          # input order
            assert off == pos
            pos += n


def test_planned_workload_is_the_busiest_rank():
    wl = wlmod.get("paper_planned_max_rank")
    roles = wlmod.paper_model_roles(16)
    owner = oplan.role_greedy(roles, 8)
    fl = oplan.score(roles, 8, owner)["rank_flops"]
    top = max(range(8), key=lambda r: (fl[r], -r))
    assert sorted((m.rows, m.cols) for m in wl.matrices) == \
        sorted((r, c) for (b, k, r, c), o in zip(roles, owner) if o == top and k == 0)
    assert sum(oplan.ns_flops((0, 0, m.rows, m.cols)) for m in wl.matrices) == max(fl)


def test_argument_checks():
    lib = mo.load_library()
    import ctypes
    bad = [
        dict(roles=[(0, 0, 4, 4)], world=0),
        dict(roles=[(-1, 0, 4, 4)], world=2),
        dict(roles=[(0, 0, -4, 4)], world=2),
        dict(roles=[(0, 1, 4, 4)], world=2),           # a tail with cols != 1
        dict(roles=[(0, 7, 4, 4)], world=2),           # unknown kind
        dict(roles=[(0, 0, 1 << 31, 4)], world=2),     # side beyond the int64-safe range
    ]
    for b in bad:
        with pytest.raises(mo.MoError):
            mo.plan_owners(b["roles"], b["world"])
    with pytest.raises(ValueError):
        mo.plan_owners([(0, 0, 4, 4)], 2, "other")
    with pytest.raises(mo.MoError):
        mo.plan_owners([(0, 0, 4, 4)], 2, "role_greedy", -1)
    with pytest.raises(mo.MoError):
        mo.plan_score([(0, 0, 4, 4)], 2, [2])           # owner outside [0, world)
    arr, n = mo._binding._roles([(0, 0, 4, 4)])
    assert lib.mo_plan_owners(arr, n, 2, 0, 0, None) == -1
    assert lib.mo_plan_owners(None, 0, 2, 0, 0, None) == 0
    assert lib.mo_plan_owners(arr, n, 2, 5, 0, (ctypes.c_int32 * 1)()) == -1
