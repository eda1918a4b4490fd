"""Pins for oracle.plan / oracle.optimum / oracle.metrics (CPU only).

What fixes the expected values here is not the oracle itself:
* Theorem 1 and its lemma (every rank exactly S*K, one source rank per
  receiver, at most E/R redundant experts, at most R-1 fills);
* Theorem 2 (worst case needs ceil(E(R-1)/R^2)) and the pages' worked
  numbers in tests/golden/worked_examples.json;
* token conservation (route is a permutation of all slots);
* an independent slot-by-slot queue simulation of the same selection rules;
* brute-force and MILP optima on tiny inputs (optimum <= plan <= E/R);
* maxvio closed forms.
"""
import collections
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import metrics, optimum
from oracle.plan import POLICY_LARGEST, Cfg, make_plan, stable_rank, histogram

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def cfg_of(s):
    return Cfg(s.R, s.S, s.E, s.K, s.H, s.Hp, s.B, s.mode)


def check_invariants(ids, cfg, plan):
    R, E, SK, n, B = cfg.R, cfg.E, cfg.SK, cfg.n, cfg.B
    flat = ids.reshape(-1)
    # tokens conserved: route is a permutation of [0, R*S*K)
    assert np.array_equal(np.sort(plan.route), np.arange(R * SK))
    dst = plan.route // SK
    # exactly S*K per rank (Theorem 1)
    assert np.all(np.bincount(dst, minlength=R) == SK)
    # per expert, the slots over all ranks add to T_e
    assert np.array_equal(np.bincount(flat, minlength=E), plan.counts)
    # fills: at most R-1; each receiver filled once, from one source
    assert len(plan.fills) <= R - 1
    receivers = [f[0] for f in plan.fills]
    assert len(set(receivers)) == len(receivers)
    for r in range(R):
        remote = flat[(dst == r) & (flat // n != r)]
        srcs = set((remote // n).tolist())
        assert len(srcs) <= 1                                   # lemma
        assert len(set(remote.tolist())) == plan.n_redundant[r]
        assert plan.n_redundant[r] <= n                          # E/R bound
        if srcs:
            assert plan.src_rank[r] == srcs.pop()
        else:
            assert plan.src_rank[r] == -1
    # each destination row lies in the segment of its own expert
    off = plan.route % SK
    for i in range(0, flat.size, max(1, flat.size // 5000)):
        r, q, e = dst[i], off[i], flat[i]
        j = np.searchsorted(plan.cu_seqlens[r], q, side="right") - 1
        if j < E:
            assert j == e
        else:
            assert plan.slot_expert[r, j - E] == e
    # segments ordered by weight row, slots ascending (token, k) inside
    key = np.lexsort((np.arange(flat.size), plan.route))
    for r in range(R):
        sl = key[r * SK:(r + 1) * SK]
        j = np.searchsorted(plan.cu_seqlens[r], np.arange(SK), side="right") - 1
        for jj in np.unique(j):
            idx = sl[j == jj]
            assert np.all(np.diff(idx) > 0)
    assert np.all(plan.cu_seqlens[:, 0] == 0) and np.all(plan.cu_seqlens[:, -1] == SK)
    if cfg.mode == 0:
        assert B >= plan.n_redundant.max(initial=0)


def queue_simulation(ids, cfg, largest=False):
    """Slot-by-slot replay of the fill rules (independent formulation).

    Each rank keeps a queue of the slots of its home experts ordered by
    (expert, slot index).  A fill pops d slots from the front of the donor's
    queue -- or, with ``largest``, repeatedly pops the front slots of the
    donor's expert with the most slots left (ties: lowest id) until d slots
    moved.  Rank buffers are then ordered by (weight row, slot index).
    """
    R, E, SK, n, B = cfg.R, cfg.E, cfg.SK, cfg.n, cfg.B
    flat = ids.reshape(-1).tolist()
    queues = [collections.deque() for _ in range(R)]
    for i in sorted(range(len(flat)), key=lambda i: (flat[i], i)):
        queues[flat[i] // n].append(i)
    holder = [flat[i] // n for i in range(len(flat))]
    load = [len(q) for q in queues]
    fills = 0
    while any(l < SK for l in load):
        u = min(r for r in range(R) if load[r] < SK)
        o = max(range(R), key=lambda r: (load[r], -r))
        d = SK - load[u]
        if largest:
            left = collections.Counter(flat[i] for i in queues[o])
            moved = set()
            todo = d
            while todo:
                e = min(left, key=lambda x: (-left[x], x))
                k = min(todo, left[e])
                todo -= k
                left[e] -= k
                taken_e = [i for i in queues[o] if flat[i] == e][:k]
                moved.update(taken_e)
                for i in taken_e:
                    holder[i] = u
            queues[o] = collections.deque(i for i in queues[o] if i not in moved)
        else:
            for _ in range(d):
                holder[queues[o].popleft()] = u
        load[o] -= d
        load[u] = SK
        fills += 1
    route = [0] * len(flat)
    for r in range(R):
        mine = [i for i in range(len(flat)) if holder[i] == r]
        remote = sorted({flat[i] for i in mine if flat[i] // n != r})

        def row(i):
            e = flat[i]
            if e // n == r:
                return e
            b = remote.index(e)
            return E + b if b < B else e
        for pos, i in enumerate(sorted(mine, key=lambda i: (row(i), i))):
            route[i] = r * SK + pos
    return np.array(route), fills


def test_golden_worked_examples():
    g = json.load(open(GOLDEN))
    t2 = g["theorem2_demo"]
    assert optimum.theorem2_bound(t2["E"], t2["R"]) == t2["min_redundant_rank0"]
    shape = W.TINY.with_(E=t2["E"], R=t2["R"])
    ids = W.routing_theorem2(shape)
    plan = make_plan(ids, cfg_of(shape))
    assert plan.n_redundant[0] == t2["min_redundant_rank0"]
    assert plan.n_redundant.max() <= t2["upper_bound"]
    assert optimum.brute_force_opt(plan.counts, shape.R, shape.SK) == t2["min_redundant_rank0"]
    for R, slots in g["k3_slots_table"]["rows"]:
        assert g["k3_slots_table"]["E"] // R == slots
    q = g["large_e_quiz"]
    assert q["E"] // q["R"] == q["max_redundant"] == W.LARGE_E.n
    d = g["theorem1_demo"]
    shape = W.TINY.with_(S=3, K=2, E=8, R=4)          # S*K = 6, E/R = 2
    assert shape.SK == d["SK"] and shape.n == d["E_over_R"]
    for seed in range(300):
        ids, _ = W.routing_uniform(shape, salt=seed)
        plan = make_plan(ids, cfg_of(shape))
        check_invariants(ids, cfg_of(shape), plan)
        assert plan.n_redundant.max() <= d["E_over_R"]


def test_tiny_random_many_seeds_and_queue_replay():
    cfg = cfg_of(W.TINY)
    for seed in range(1000):
        ids, _ = W.routing_uniform(W.TINY, salt=seed)
        plan = make_plan(ids, cfg)
        check_invariants(ids, cfg, plan)
        if seed < 200:
            route, fills = queue_simulation(ids, cfg)
            assert np.array_equal(route, plan.route)
            assert fills == len(plan.fills)


@pytest.mark.parametrize("R,S,E,K,B,mode", [
    (4, 16, 8, 2, 2, 0), (3, 7, 9, 3, 3, 0), (5, 11, 10, 4, 2, 0),
    (5, 11, 10, 4, 1, 1), (6, 5, 12, 5, 0, 1), (2, 9, 8, 8, 4, 0),
    (1, 13, 4, 2, 4, 0), (4, 6, 4, 1, 1, 0), (8, 4, 16, 3, 2, 0)])
def test_queue_replay_shapes(R, S, E, K, B, mode):
    shape = W.TINY.with_(R=R, S=S, E=E, K=K, B=B, mode=mode)
    cfg = cfg_of(shape)
    for seed in range(40):
        if seed % 4 == 3:
            ids = W.routing_hot(shape)
        else:
            ids, _ = W.routing_uniform(shape, salt=seed)
        plan = make_plan(ids, cfg)
        check_invariants(ids, cfg, plan)
        route, fills = queue_simulation(ids, cfg)
        assert np.array_equal(route, plan.route)
        assert fills == len(plan.fills)


def test_theorem2_traces():
    # rank 0 needs exactly ceil(E(R-1)/R^2); deterministic plan hits it
    for shape, want_rank0 in [(W.TINY, 2), (W.ADVERSARIAL, 42)]:
        ids = W.routing_theorem2(shape)
        plan = make_plan(ids, cfg_of(shape))
        check_invariants(ids, cfg_of(shape), plan)
        assert want_rank0 == optimum.theorem2_bound(shape.E, shape.R)
        assert plan.n_redundant[0] == want_rank0
        assert optimum.per_rank_lower_bound(plan.counts, shape.R, shape.SK) == want_rank0
        assert plan.load0[0] == 0
    plan = make_plan(W.routing_theorem2(W.ADVERSARIAL), cfg_of(W.ADVERSARIAL))
    assert plan.n_redundant.tolist() == [42, 36, 30, 24, 18, 12, 6, 0]
    assert [f[:2] for f in plan.fills] == [(r, r + 1) for r in range(7)]


def test_theorem2_large_e_bound():
    shape = W.LARGE_E
    ids = W.routing_theorem2(shape)
    plan = make_plan(ids, cfg_of(shape))
    assert plan.n_redundant.max() == shape.n == optimum.theorem2_bound(shape.E, shape.R) == 14
    assert len(plan.fills) == shape.R - 1
    assert np.array_equal(np.bincount(plan.route // shape.SK, minlength=shape.R),
                          np.full(shape.R, shape.SK))


def test_optimum_brute_force_vs_milp_and_bounds():
    cfg = cfg_of(W.TINY)
    worse = 0
    for seed in range(20):
        ids, _ = W.routing_uniform(W.TINY, salt=1000 + seed)
        plan = make_plan(ids, cfg)
        lb = optimum.per_rank_lower_bound(plan.counts, cfg.R, cfg.SK)
        bf = optimum.brute_force_opt(plan.counts, cfg.R, cfg.SK)
        ilp = optimum.milp_opt(plan.counts, cfg.R, cfg.SK)
        assert bf == ilp
        assert lb <= bf <= plan.n_redundant.max() <= cfg.n
        worse += plan.n_redundant.max() > bf
    # skewed tiny instances where the optimum is above the counting bound
    shape = W.TINY.with_(R=3, S=4, E=6, K=2, B=2)
    for seed in range(10):
        ids, _ = W.routing_uniform(shape, salt=seed)
        plan = make_plan(ids, cfg_of(shape))
        bf = optimum.brute_force_opt(plan.counts, shape.R, shape.SK)
        assert bf == optimum.milp_opt(plan.counts, shape.R, shape.SK)
        assert bf <= plan.n_redundant.max() <= shape.n


def test_hot_and_degenerate():
    # every token on experts 0..K-1: rank 0 holds everything
    for shape in [W.SKEWED, W.TINY.with_(K=4, B=2)]:
        ids = W.routing_hot(shape)
        plan = make_plan(ids, cfg_of(shape))
        check_invariants(ids, cfg_of(shape), plan)
        assert metrics.maxvio(plan.counts, shape.R, shape.S, shape.K) == pytest.approx(
            shape.E / shape.K - 1)
    # R = 1: nothing moves
    shape = W.TINY.with_(R=1, B=8)
    ids, _ = W.routing_uniform(shape)
    plan = make_plan(ids, cfg_of(shape))
    assert len(plan.fills) == 0 and plan.moves.shape == (0, 4)
    # S = 0: empty plan
    shape = W.TINY.with_(S=0)
    plan = make_plan(np.zeros((0, shape.K), np.int32), cfg_of(shape))
    assert plan.route.size == 0 and np.all(plan.cu_seqlens == 0)
    # bad ids are rejected
    ids, _ = W.routing_uniform(W.TINY)
    ids = ids.copy()
    ids[3, 1] = W.TINY.E
    with pytest.raises(ValueError):
        make_plan(ids, cfg_of(W.TINY))


def test_perfectly_balanced_needs_no_fill():
    shape = W.TINY.with_(S=8, K=2, E=8, R=4)
    i = np.arange(shape.tokens * shape.K)
    ids = (i % shape.E).astype(np.int32).reshape(shape.tokens, shape.K)
    plan = make_plan(ids, cfg_of(shape))
    assert metrics.maxvio(plan.counts, shape.R, shape.S, shape.K) == 0.0
    assert len(plan.fills) == 0 and plan.n_redundant.max() == 0


def test_stable_rank_and_histogram_brute_force():
    g = np.random.default_rng(5)
    ids = g.integers(0, 7, size=300)
    p = stable_rank(ids, 7)
    for i in range(ids.size):
        assert p[i] == np.sum(ids[:i] == ids[i])
    T = histogram(ids, 7)
    assert [int(T[e]) for e in range(7)] == [int(np.sum(ids == e)) for e in range(7)]


def test_maxvio_sweep_generator_hits_targets():
    for target in W.MAXVIO_SWEEP["skewed"]:
        ids, gates, s, mv = W.routing_zipf(W.SKEWED, target)
        T = np.bincount(ids.reshape(-1), minlength=W.SKEWED.E)
        got = metrics.maxvio(T, W.SKEWED.R, W.SKEWED.S, W.SKEWED.K)
        assert abs(got - target) <= 0.02 * target
        assert np.allclose(gates.sum(axis=1), 1.0, atol=1e-6)
        assert all(len(set(r)) == W.SKEWED.K for r in ids[:2000].tolist())
        plan = make_plan(ids, cfg_of(W.SKEWED))
        check_invariants(ids, cfg_of(W.SKEWED), plan)


def test_bench_shape_sweep_invariants():
    shape = W.BENCH
    for target in W.MAXVIO_SWEEP["bench"]:
        ids, _, _, mv = W.routing_zipf(shape, target)
        assert abs(mv - target) <= 0.02 * target
        plan = make_plan(ids, cfg_of(shape))
        assert np.all(np.bincount(plan.route // shape.SK, minlength=shape.R) == shape.SK)
        assert np.array_equal(np.sort(plan.route), np.arange(shape.R * shape.SK))
        assert plan.n_redundant.max() <= shape.n
        assert len(plan.fills) <= shape.R - 1
        assert math.isclose(metrics.maxvio(plan.counts, shape.R, shape.S, shape.K), mv)


# ---------------------------------------------------------------------------
# The largest-remaining-first donor policy (the same theorem, another choice
# of the donor's experts): same invariants, an independent slot-level replay,
# and its redundancy against the offline integer program.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("R,S,E,K,B,mode", [
    (4, 16, 8, 2, 2, 0), (3, 7, 9, 3, 3, 0), (5, 11, 10, 4, 1, 1),
    (6, 5, 12, 5, 0, 1), (2, 9, 8, 8, 4, 0), (8, 4, 16, 3, 2, 0)])
def test_largest_policy_queue_replay(R, S, E, K, B, mode):
    shape = W.TINY.with_(R=R, S=S, E=E, K=K, B=B, mode=mode)
    cfg = cfg_of(shape)
    for seed in range(40):
        if seed % 4 == 3:
            ids = W.routing_hot(shape)
        else:
            ids, _ = W.routing_uniform(shape, salt=seed)
        plan = make_plan(ids, cfg, POLICY_LARGEST)
        check_invariants(ids, cfg, plan)
        route, fills = queue_simulation(ids, cfg, largest=True)
        assert np.array_equal(route, plan.route)
        assert fills == len(plan.fills)


def test_largest_policy_sweeps_and_milp():
    # same invariants on the skewed and bench sweeps and the Theorem-2 case;
    # on the skewed sweep the largest-first plan's worst rank needs exactly
    # what the integer program finds optimal, and never more than ascending
    for shape, targets in ((W.SKEWED, W.MAXVIO_SWEEP["skewed"]),
                           (W.BENCH, W.MAXVIO_SWEEP["bench"])):
        cfg = cfg_of(shape)
        for t in targets:
            ids, _, _, _ = W.routing_zipf(shape, t)
            big = make_plan(ids, cfg, POLICY_LARGEST)
            asc = make_plan(ids, cfg)
            check_invariants(ids, cfg, big)
            assert big.n_redundant.max() <= asc.n_redundant.max()
            assert len(big.moves) <= len(asc.moves)
            if shape is W.SKEWED:
                assert big.n_redundant.max() == optimum.milp_opt(big.counts, shape.R, shape.SK)
    shape = W.ADVERSARIAL
    ids = W.routing_theorem2(shape)
    big = make_plan(ids, cfg_of(shape), POLICY_LARGEST)
    check_invariants(ids, cfg_of(shape), big)
    assert big.n_redundant[0] == 42                   # the Theorem-2 worst case is tight
