"""CPU model of the SOAP pair solve's step order (soap_kernels.hip,
so_jac_solve_kernel): one scalar cyclic Jacobi sweep over a 64 x 64 symmetric
pair problem, 63 steps of 32 disjoint rotations in the circle ordering, with
one barrier per step.  Threads 0 .. 31 update the 2 x 2 blocks that hold the
next step's pivots, apply the diagonal updates those pivots need and compute
the next rotations; the other threads update the other blocks and waves 1 .. 7
accumulate D = V - I.  Written out from the schedule the kernel documents and
checked here:

  * the circle ordering turns one place per step, so pair j of step k + 1
    takes one element from pair j - 1 and one from pair j + 1 of step k (0 and 1
    for j = 0, 30 and 31 for j = 31), at every step, and each index the kernel
    keeps in a register follows it by one update (0 stays, 63 wraps to 1);
  * the slot map is a bijection of the 512 threads onto the 512 block slots,
    and threads 0 .. 31 hold exactly those 32 blocks;
  * the one-barrier order gives the same S and D, bit for bit, as steps that
    first compute all rotations, then apply them (two barriers);
  * within a step no entry of S or D is read by one thread and written by
    another, and none is written twice.

Plain Python floats on both sides, so "bit for bit" compares two orders of
the same arithmetic; the kernel's own roundings are checked on the GPU.
"""
import math

import numpy as np
import pytest

PW, NP, THREADS = 64, 32, 512


def circle_pair(n, k, j):
    f = lambda i: (i + k) % (n - 1) + 1
    return (0, f(0)) if j == 0 else (f(j), f(n - 1 - j))


def advance_circle(i, keep=PW - 1):
    """The kernel's index update from one step to the next: keep is 0 for the
    first index of pair 0 (which never moves), PW - 1 for every other."""
    x = i + 1
    return (x & keep) | (x >> 6)


def next_sources(j):
    """The two step-k pairs that pair j of step k + 1 draws from, in the order
    the kernel's slot gives them (rows, columns)."""
    if j == 0:
        return 0, 1
    if j == NP - 1:
        return NP - 2, NP - 1
    return j - 1, j + 1


def slot_pair(s):
    """Unordered pair {u, v} of slot s (None for the idle copy)."""
    u, dv = s >> 4, s & 15
    v = (u + 1 + dv) & 31
    return None if (dv == 15 and u >= 16) else (u, v)


def solve_slot(t):
    if t < NP:
        return 0 if t == 0 else 480 if t == NP - 1 else 16 * (t - 1) + 1
    if t == 480:
        return 31
    if (t & 15) == 1 and t <= 465:
        i = (t >> 4) - 2
        return i + 2 if i <= 14 else i + 3
    return t


def rotation(app, aqq, apq, thr):
    """Rutishauser's rotation zeroing apq: (t, s, tau), zeros below thr."""
    if abs(apq) <= thr:
        return 0.0, 0.0, 0.0
    theta = (aqq - app) / (2.0 * apq)
    if abs(theta) > 1e150:
        t = 0.5 / theta
    else:
        t = (1.0 if theta >= 0.0 else -1.0) / (abs(theta) + math.sqrt(theta * theta + 1.0))
    c = 1.0 / math.sqrt(t * t + 1.0)
    s = t * c
    return t, s, s / (1.0 + c)


def block(x, su, tu, sv, tv):
    x00, x01, x10, x11 = x
    y00, y10 = x00 - su * (x10 + tu * x00), x10 + su * (x00 - tu * x10)
    y01, y11 = x01 - su * (x11 + tu * x01), x11 + su * (x01 - tu * x11)
    return (y00 - sv * (y01 + tv * y00), y01 + sv * (y00 - tv * y01),
            y10 - sv * (y11 + tv * y10), y11 + sv * (y10 - tv * y11))


def d_update(D, r, a, b, s, tau):
    """Row r of D <- D J + (J - I): the rotation's products take V = I + D."""
    da, db = D[r][a], D[r][b]
    va, vb = da + (1.0 if r == a else 0.0), db + (1.0 if r == b else 0.0)
    return da - s * (vb + tau * va), db + s * (va - tau * vb)


def key(i, j):
    return (i, j) if i <= j else (j, i)


def two_barrier(S0, thr):
    """Reference order: all rotations of a step from S, then every update."""
    S = {key(i, j): float(S0[i, j]) for i in range(PW) for j in range(i, PW)}
    D = [[0.0] * PW for _ in range(PW)]
    for k in range(PW - 1):
        P = []
        for j in range(NP):
            a, b = circle_pair(PW, k, j)
            t, s, tau = rotation(S[(a, a)], S[(b, b)], S[key(a, b)], thr)
            P.append((a, b, t, s, tau, S[key(a, b)]))
        for sl in range(512):
            uv = slot_pair(sl)
            if uv is None:
                continue
            u, v = uv
            (au, bu, _, su, tu, _), (av, bv, _, sv, tv, _) = P[u], P[v]
            ks = [key(au, av), key(au, bv), key(bu, av), key(bu, bv)]
            for kk, z in zip(ks, block([S[q] for q in ks], su, tu, sv, tv)):
                S[kk] = z
        for a, b, t, s, tau, apq in P:
            if s != 0.0:
                S[(a, a)] -= t * apq
                S[(b, b)] += t * apq
                S[key(a, b)] = 0.0
        for r in range(PW):
            for a, b, t, s, tau, apq in P:
                D[r][a], D[r][b] = d_update(D, r, a, b, s, tau)
    return S, D


def one_barrier(S0, thr):
    """The kernel's order, thread by thread, with every access logged."""
    S = {key(i, j): float(S0[i, j]) for i in range(PW) for j in range(i, PW)}
    D = [[0.0] * PW for _ in range(PW)]
    par = [None] * NP                      # rotation j of the current step: (a, b, t, s, tau, apq)
    for j in range(NP):
        a, b = circle_pair(PW, 0, j)
        par[j] = (a, b) + rotation(S[(a, a)], S[(b, b)], S[key(a, b)], thr) + (S[key(a, b)],)
    for k in range(PW - 1):
        reads, writes, new_par = {}, {}, [None] * NP

        def rd(obj, kk, th):
            reads.setdefault((obj, kk), set()).add(th)
            return S[kk] if obj == "S" else D[kk[0]][kk[1]]

        def wr(obj, kk, v, th):
            assert (obj, kk) not in writes, ("written twice", obj, kk, k)
            writes[(obj, kk)] = (th, v)

        for th in range(THREADS):
            uv = slot_pair(solve_slot(th))
            if uv is not None:
                u, v = uv
                (au, bu, _, su, tu, _), (av, bv, _, sv, tv, _) = par[u], par[v]
                ks = [key(au, av), key(au, bv), key(bu, av), key(bu, bv)]
                z = block([rd("S", q, th) for q in ks], su, tu, sv, tv)
                for kk, val in zip(ks, z):
                    wr("S", kk, val, th)
            if th < NP:                        # next pivot th, from the block just updated
                a0, b0, _, s0, _, _ = par[th]
                if s0 != 0.0:
                    wr("S", key(a0, b0), 0.0, th)
                a2, b2 = circle_pair(PW, (k + 1) % (PW - 1), th)
                zmap = dict(zip([(au, av), (au, bv), (bu, av), (bu, bv)], z))
                apq2 = zmap[(a2, b2)] if (a2, b2) in zmap else zmap[(b2, a2)]
                diag = []
                for e in (a2, b2):
                    w = u if e in (au, bu) else v
                    a, b, t, s, tau, apq = par[w]
                    d = rd("S", (e, e), th)
                    if s != 0.0:
                        d = d - t * apq if e == a else d + t * apq
                    wr("S", (e, e), d, th)
                    diag.append(d)
                if k + 1 < PW - 1:
                    new_par[th] = (a2, b2) + rotation(diag[0], diag[1], apq2, thr) + (apq2,)
            elif th >= 64:                     # D on waves 1 .. 7
                for i in range(5):
                    q = (th - 64) + 448 * i
                    if q >= PW * NP:
                        break
                    w, r = q & (NP - 1), q >> 5
                    a, b, _, s, tau, _ = par[w]
                    rd("D", (r, a), th)
                    rd("D", (r, b), th)
                    na, nb = d_update(D, r, a, b, s, tau)
                    wr("D", (r, a), na, th)
                    wr("D", (r, b), nb, th)
        for (obj, kk), (th, _) in writes.items():
            others = reads.get((obj, kk), set()) - {th}
            assert not others, ("read and written by different threads", obj, kk, k)
        for (obj, kk), (_, v) in writes.items():
            if obj == "S":
                S[kk] = v
            else:
                D[kk[0]][kk[1]] = v
        if k + 1 < PW - 1:
            par = new_par
    return S, D


def test_next_pivots_come_from_neighbouring_pairs():
    for k in range(PW - 1):
        where = {}
        for j in range(NP):
            a, b = circle_pair(PW, k, j)
            where[a] = where[b] = j
        for j in range(NP):
            a2, b2 = circle_pair(PW, (k + 1) % (PW - 1), j)
            assert sorted((where[a2], where[b2])) == sorted(next_sources(j))


def test_indices_advance_with_the_circle():
    """The kernel keeps each pair's indices in registers and advances them; that
    gives circle_pair at every step, through the wrap from step 62 to step 0."""
    for k in range(PW - 1):
        for j in range(NP):
            a, b = circle_pair(PW, k, j)
            keep_a = 0 if j == 0 else PW - 1
            assert (advance_circle(a, keep_a), advance_circle(b)) == circle_pair(PW, (k + 1) % (PW - 1), j)


def test_slot_map_is_a_bijection_with_the_pivot_blocks_first():
    slots = [solve_slot(t) for t in range(THREADS)]
    assert sorted(slots) == list(range(512))
    for j in range(NP):
        assert slot_pair(slots[j]) == next_sources(j)
    pairs = {frozenset(p) for p in map(slot_pair, range(512)) if p is not None}
    assert len(pairs) == NP * (NP - 1) // 2


@pytest.mark.parametrize("case", ["random", "nearly_diagonal", "block_diagonal"])
def test_one_barrier_order_equals_two_barrier_steps(case):
    rng = np.random.default_rng(11)
    X = rng.standard_normal((PW, 3 * PW))
    S0 = X @ X.T
    if case == "nearly_diagonal":       # most pivots below the threshold
        S0 = np.diag(np.arange(1.0, PW + 1.0)) + 1e-9 * S0
    if case == "block_diagonal":        # the two halves already decoupled
        S0[:NP, NP:] = 0.0
        S0[NP:, :NP] = 0.0
    thr = 2.0 ** -48 * float(np.linalg.norm(S0))
    S_ref, D_ref = two_barrier(S0, thr)
    S_new, D_new = one_barrier(S0, thr)
    assert S_new == S_ref
    assert D_new == D_ref
    # and the sweep did its job: V = I + D orthogonal, V^T S0 V closer to diagonal
    V = np.eye(PW) + np.array(D_new)
    assert np.abs(V.T @ V - np.eye(PW)).max() < 1e-12
    off0 = np.linalg.norm(S0 - np.diag(np.diag(S0)))
    R = V.T @ S0 @ V
    assert np.linalg.norm(R - np.diag(np.diag(R))) <= off0


def test_packed_triangle_index():
    """The kernel's packed index of (i, j), min(i, j) (2 PW - 1 - min) / 2 + max,
    is row-major order over the upper triangle: a bijection onto 0 .. 2079,
    and its byte offset is eight times that."""
    def tri(i, j):
        a, b = min(i, j), max(i, j)
        assert a * (2 * PW - 1 - a) % 2 == 0
        return a * (2 * PW - 1 - a) // 2 + b
    order = [tri(i, j) for i in range(PW) for j in range(i, PW)]
    assert order == list(range(PW * (PW + 1) // 2))
    assert all(tri(i, j) == tri(j, i) for i in range(PW) for j in range(PW))
    # the byte offset the step loop uses: 4 a (2 PW - 1 - a) + 8 b
    for i in range(PW):
        for j in range(PW):
            a, b = min(i, j), max(i, j)
            assert 4 * a * (2 * PW - 1 - a) + 8 * b == 8 * tri(i, j)
