"""Optimal max-redundancy on tiny inputs, and bounds (test infrastructure only).

[MoonEP-fr] "La planification en ligne": exact optima from an offline
integer linear program are the yardstick the online planner is measured
against.  Here the same optimum is computed two independent ways:

* ``brute_force_opt`` -- enumerate, for a candidate M, every choice of M
  remote experts per rank and test feasibility of "every rank gets exactly
  S*K slots" with Gale's supply/demand condition (for every set Q of ranks,
  |Q|*S*K <= total count of experts some rank of Q may serve); the answer is
  the least feasible M;
* ``milp_opt`` -- the integer program solved by SciPy/HiGHS.

``per_rank_lower_bound`` and ``theorem2_bound`` are closed forms used as
further pins.  The deterministic planner is NOT expected to reach the
optimum; tests assert lower bound <= optimum <= plan <= E/R.
"""
import itertools
import math

import numpy as np


def redundancy(plan):
    """m_r = number of distinct remote experts rank r computes."""
    return np.asarray(plan.n_redundant, np.int64)


def theorem2_bound(E, R):
    """ceil(E(R-1)/R^2) ([K3-blog] "定理 2", [MoonEP-fr] Théorème 2)."""
    return -(-E * (R - 1) // (R * R))


def per_rank_lower_bound(counts, R, SK):
    """max over ranks of the fewest remote experts that can cover the deficit.

    An underloaded rank r must take SK - load_r remote slots; a remote expert
    gives at most T_e of them, so it needs at least as many remote experts
    as the shortest prefix of the descending remote counts reaching that
    deficit.  (The argument of Theorem 2, applied to any routing.)
    """
    T = np.asarray(counts, np.int64)
    E = T.size
    n = E // R
    lb = 0
    for r in range(R):
        deficit = SK - int(T[r * n:(r + 1) * n].sum())
        if deficit <= 0:
            continue
        remote = np.sort(np.concatenate([T[:r * n], T[(r + 1) * n:]]))[::-1]
        acc = np.cumsum(remote)
        k = int(np.searchsorted(acc, deficit, side="left")) + 1
        lb = max(lb, k)
    return lb


def _feasible(masks, supply_of_mask, R, SK):
    for q in range(1, 1 << R):
        nb = 0
        size = 0
        for r in range(R):
            if q >> r & 1:
                nb |= masks[r]
                size += 1
        if size * SK > supply_of_mask(nb):
            return False
    return True


def brute_force_opt(counts, R, SK, max_sets=2_000_000):
    """Least M such that some choice of <= M remote experts per rank is feasible."""
    T = np.asarray(counts, np.int64)
    E = T.size
    n = E // R
    if E > 20:
        raise ValueError("brute force is for tiny inputs only")
    cache = {}

    def supply(mask):
        v = cache.get(mask)
        if v is None:
            v = int(sum(T[e] for e in range(E) if mask >> e & 1))
            cache[mask] = v
        return v

    home = [sum(1 << e for e in range(r * n, (r + 1) * n)) for r in range(R)]
    remote = [[e for e in range(E) if e // n != r and T[e] > 0] for r in range(R)]
    for M in range(0, E - n + 1):
        choices = []
        for r in range(R):
            k = min(M, len(remote[r]))
            choices.append([home[r] | sum(1 << e for e in c)
                            for c in itertools.combinations(remote[r], k)])
        total = math.prod(len(c) for c in choices)
        if total > max_sets:
            raise ValueError("too many combinations (%d)" % total)
        for masks in itertools.product(*choices):
            if _feasible(masks, supply, R, SK):
                return M
    return E - n


def milp_opt(counts, R, SK):
    """The offline integer program of [MoonEP-fr] "La planification en ligne".

    Variables: x[e, r] >= 0 integer (slots of e computed on r); z[e, r] in
    {0, 1} for remote pairs (e not homed on r); M.  Constraints: every slot
    placed (sum_r x = T_e), every rank exactly S*K (sum_e x = S*K), x <= T_e z
    on remote pairs, sum_e z[e, r] <= M.  Minimise M.
    """
    from scipy.optimize import LinearConstraint, milp, Bounds

    T = np.asarray(counts, np.int64)
    E = T.size
    n = E // R
    remote = [(e, r) for e in range(E) for r in range(R) if e // n != r]
    nx = E * R
    nz = len(remote)
    nv = nx + nz + 1
    c = np.zeros(nv)
    c[-1] = 1.0
    rows, lo, hi = [], [], []

    def xi(e, r):
        return e * R + r

    for e in range(E):
        a = np.zeros(nv)
        for r in range(R):
            a[xi(e, r)] = 1
        rows.append(a); lo.append(T[e]); hi.append(T[e])
    for r in range(R):
        a = np.zeros(nv)
        for e in range(E):
            a[xi(e, r)] = 1
        rows.append(a); lo.append(SK); hi.append(SK)
    for k, (e, r) in enumerate(remote):
        a = np.zeros(nv)
        a[xi(e, r)] = 1
        a[nx + k] = -float(T[e])
        rows.append(a); lo.append(-np.inf); hi.append(0)
    for r in range(R):
        a = np.zeros(nv)
        for k, (e, rr) in enumerate(remote):
            if rr == r:
                a[nx + k] = 1
        a[-1] = -1
        rows.append(a); lo.append(-np.inf); hi.append(0)
    ub = np.concatenate([np.repeat(T, R).astype(float), np.ones(nz), [E]])
    res = milp(c, constraints=LinearConstraint(np.array(rows), lo, hi),
               integrality=np.ones(nv), bounds=Bounds(np.zeros(nv), ub))
    if not res.success:
        raise RuntimeError(res.message)
    return int(round(res.x[-1]))
