"""Pins for oracle.dataflow (CPU only).

Expected values come from closed forms of special cases (W[e] = c_e * I with
distinct powers of two, gates 1/K), from plain triple loops on tiny shapes,
and from known constants for reduce_grad -- not from the oracle itself.
"""
import numpy as np
import pytest

import workloads as W
from oracle import bf16, dataflow
from oracle.plan import Cfg, make_plan


def cfg_of(s):
    return Cfg(s.R, s.S, s.E, s.K, s.H, s.Hp, s.B, s.mode)


def rand_bits(g, shape, scale=1.0):
    return bf16.f64_to_bits(g.standard_normal(shape) * scale)


def tiny_setup(shape, seed=0, hot=False):
    cfg = cfg_of(shape)
    if hot:
        ids = W.routing_hot(shape)
        gates = W.gates_uniform(shape)
    else:
        ids, gates = W.routing_uniform(shape, salt=seed)
    plan = make_plan(ids, cfg)
    return cfg, ids, gates, plan


@pytest.mark.parametrize("shape", [W.TINY, W.TINY.with_(B=1, mode=1),
                                   W.TINY.with_(R=2, E=8, K=3, S=10, B=4)])
def test_dispatch_and_prefetch_are_bit_copies(shape):
    g = np.random.default_rng(3)
    cfg, ids, _, plan = tiny_setup(shape, hot=False)
    x = rand_bits(g, (shape.tokens, shape.H))
    xp = dataflow.dispatch(x, plan, cfg)
    for i in range(ids.size):
        assert np.array_equal(xp[plan.route[i]], x[i // shape.K])
    w = rand_bits(g, (shape.E, shape.H, shape.Hp))
    wp = dataflow.prefetch(w, plan, cfg)
    for r in range(shape.R):
        for b in range(shape.B):
            e = plan.slot_expert[r, b]
            if e >= 0:
                assert np.array_equal(wp[r, b], w[e])
            else:
                assert not wp[r, b].any()


@pytest.mark.parametrize("mode,B", [(0, 2), (1, 1), (1, 0)])
def test_gemm_and_combine_closed_form_scaled_identity(mode, B):
    # W[e] = c_e * I with c_e = 2^(e - 3): y = c_e * x exactly; with gates
    # 1/K the combine is x * (sum_k c_{e_k}) / K, rounded once to bf16.
    shape = W.TINY.with_(H=64, Hp=64, mode=mode, B=B)
    cfg, ids, _, plan = tiny_setup(shape, seed=7)
    g = np.random.default_rng(11)
    x = rand_bits(g, (shape.tokens, shape.H))
    c = 2.0 ** (np.arange(shape.E) - 3)
    w = bf16.f64_to_bits(c[:, None, None] * np.eye(shape.H)[None])
    wp = dataflow.prefetch(w, plan, cfg)
    xp = dataflow.dispatch(x, plan, cfg)
    y = dataflow.grouped_gemm(xp, w, wp, plan, cfg)
    xf = bf16.bits_to_f64(x)
    yf = bf16.bits_to_f64(y)
    flat = ids.reshape(-1)
    for i in range(flat.size):
        assert np.array_equal(yf[plan.route[i]], c[flat[i]] * xf[i // shape.K])
    gates = W.gates_uniform(shape)
    out = dataflow.combine(y, gates, plan, cfg)
    want = xf * (c[ids].sum(axis=1) / shape.K)[:, None]
    assert np.array_equal(out, bf16.f64_to_bits(want))
    # sampled-rows form agrees with the full form
    rows = np.arange(0, shape.R * shape.SK, 3)
    assert np.array_equal(dataflow.gemm_rows(rows, x, w, wp, plan, cfg), y[rows])


def test_gemm_combine_triple_loops_tiny():
    shape = W.TINY.with_(H=8, Hp=4, S=4)
    cfg, ids, gates, plan = tiny_setup(shape, seed=2)
    g = np.random.default_rng(4)
    x = rand_bits(g, (shape.tokens, shape.H))
    w = rand_bits(g, (shape.E, shape.H, shape.Hp))
    wp = dataflow.prefetch(w, plan, cfg)
    xp = dataflow.dispatch(x, plan, cfg)
    y = dataflow.grouped_gemm(xp, w, wp, plan, cfg)
    xf, wf = bf16.bits_to_f64(x), bf16.bits_to_f64(w)
    flat = ids.reshape(-1)
    for i in range(flat.size):
        t, e = i // shape.K, flat[i]
        for col in range(shape.Hp):
            acc = 0.0
            for h in range(shape.H):
                acc += xf[t, h] * wf[e, h, col]
            assert y[plan.route[i], col] == bf16.f64_to_bits(np.float64(acc))
    out = dataflow.combine(y, gates, plan, cfg)
    yf = bf16.bits_to_f64(y)
    for t in range(shape.tokens):
        for col in range(shape.Hp):
            acc = 0.0
            for k in range(shape.K):
                acc += float(gates[t, k]) * yf[plan.route[t * shape.K + k], col]
            assert out[t, col] == bf16.f64_to_bits(np.float64(acc))


def test_wgrad_triple_loops_and_zero_home_rows():
    shape = W.TINY.with_(H=6, Hp=5, S=6)
    cfg, ids, _, plan = tiny_setup(shape, seed=9)
    g = np.random.default_rng(6)
    x = rand_bits(g, (shape.tokens, shape.H))
    xp = dataflow.dispatch(x, plan, cfg)
    dy = rand_bits(g, (shape.R * shape.SK, shape.Hp))
    gh, gp = dataflow.wgrad(xp, dy, plan, cfg)
    xf, dyf = bf16.bits_to_f64(x), bf16.bits_to_f64(dy)
    flat = ids.reshape(-1)
    want_h = np.zeros_like(gh)
    want_p = np.zeros_like(gp)
    for i in range(flat.size):
        e, q = flat[i], plan.route[i]
        r = q // shape.SK
        dst_home = (e // shape.n == r)
        for a in range(shape.H):
            for b in range(shape.Hp):
                v = xf[i // shape.K, a] * dyf[q, b]
                if dst_home:
                    want_h[e, a, b] += v
                else:
                    slot = list(plan.slot_expert[r]).index(e)
                    want_p[r, slot, a, b] += v
    assert np.allclose(gh, want_h, rtol=1e-12, atol=1e-12)
    assert np.allclose(gp, want_p, rtol=1e-12, atol=1e-12)
    # a full reduction recovers the per-expert gradient sum over all slots
    gh2, gp2 = dataflow.reduce_grad(gh, gp, plan, cfg)
    total = np.zeros_like(gh)
    for i in range(flat.size):
        total[flat[i]] += np.outer(xf[i // shape.K], dyf[plan.route[i]])
    assert np.allclose(gh2, total, rtol=1e-12, atol=1e-12)
    assert not gp2[plan.slot_expert >= 0].any()


def test_reduce_grad_known_constants():
    shape = W.ADVERSARIAL.with_(S=64, H=2, Hp=3)        # Theorem-2 routing
    cfg = cfg_of(shape)
    plan = make_plan(W.routing_theorem2(shape), cfg)
    gh = np.full((shape.E, 2, 3), 0.5)
    gp = np.zeros((shape.R, shape.B, 2, 3))
    for r in range(shape.R):
        for b in range(shape.B):
            gp[r, b] = (r + 1) * 1000 + b                  # every slot, used or not
    gh2, gp2 = dataflow.reduce_grad(gh, gp, plan, cfg)
    for e in range(shape.E):
        add = sum((r + 1) * 1000 + b for r in range(shape.R) for b in range(shape.B)
                  if plan.slot_expert[r, b] == e)
        assert np.all(gh2[e] == 0.5 + add)
    for r in range(shape.R):
        for b in range(shape.B):
            if plan.slot_expert[r, b] >= 0:
                assert not gp2[r, b].any()
            else:
                assert np.all(gp2[r, b] == (r + 1) * 1000 + b)   # untouched
    assert (plan.slot_expert >= 0).sum() == plan.n_redundant.sum()


# ---------------------------------------------------------------------------
# Backward of the data path.  Each backward map F^T is pinned to its forward
# map F (pinned above) by the adjoint identity <dout, F(x)> = <F^T(dout), x>,
# evaluated exactly: small-integer data and power-of-two gates keep every
# product and sum exact in bf16 and float64.
# ---------------------------------------------------------------------------
def int_bits(g, shape, lo=-2, hi=2):
    return bf16.f64_to_bits(g.integers(lo, hi + 1, size=shape).astype(np.float64))


def f64(bits):
    return bf16.bits_to_f64(bits)


@pytest.mark.parametrize("shape", [W.TINY, W.TINY.with_(B=1, mode=1),
                                   W.TINY.with_(R=2, E=8, K=3, S=10, B=4)])
def test_combine_backward_adjoint_and_gate_gradient(shape):
    g = np.random.default_rng(21)
    cfg, ids, _, plan = tiny_setup(shape, seed=5)
    nt, K = shape.tokens, shape.K
    gates = (2.0 ** g.integers(-2, 2, size=(nt, K))).astype(np.float32)
    y = int_bits(g, (shape.R * shape.SK, shape.Hp))
    dout = int_bits(g, (nt, shape.Hp))
    dy, dg = dataflow.combine_backward(dout, y, gates, plan, cfg)
    # <dout, combine(y)> = <dy, y>: combine is linear in y
    lhs = np.sum(f64(dout) * f64(dataflow.combine(y, gates, plan, cfg)))
    assert lhs == np.sum(f64(dy) * f64(y))
    # combine is linear in each gate: a unit step of g[t, k] changes
    # <dout, out> by exactly dgates[t, k]
    for t, k in [(0, 0), (1, K - 1), (nt - 1, 0), (nt // 2, K // 2)]:
        g2 = gates.copy()
        g2[t, k] += 1.0
        rhs = np.sum(f64(dout) * f64(dataflow.combine(y, g2, plan, cfg)))
        assert rhs - lhs == dg[t, k]


def test_combine_backward_rounds_the_exact_product_once():
    # gates with a full 24-bit significand: g * dout needs up to 32 bits, so
    # rounding through fp32 first would differ from one rounding of the exact
    # product for some entries (the test asserts it does here).  Every dy
    # value must be the bf16 nearest to the exact product, ties to even.
    from fractions import Fraction
    shape = W.TINY.with_(S=64)
    cfg, ids, _, plan = tiny_setup(shape, seed=2)
    g = np.random.default_rng(4)
    gates = g.random((shape.tokens, shape.K)).astype(np.float32)
    dout = rand_bits(g, (shape.tokens, shape.Hp))
    y = rand_bits(g, (shape.R * shape.SK, shape.Hp))
    # planted pairs (gate bits, dout value) whose fp32 product sits exactly
    # on a bf16 rounding midpoint while the exact product does not
    planted = [(1063494377, 0.171875), (1055868370, -0.171875),
               (1062663076, 2.265625), (1052535658, -2.234375)]
    for i, (gb, dv) in enumerate(planted):
        gates[5 + i, i % shape.K] = np.array(gb, np.uint32).view(np.float32)
        dout[5 + i, 3 * i] = bf16.f64_to_bits(np.array(dv))
    dy, _ = dataflow.combine_backward(dout, y, gates, plan, cfg)
    route = plan.route.reshape(-1, shape.K)

    def nearest_bf16(q):
        # candidates: the two bf16 values around q (8 significant bits)
        if q == 0:
            return Fraction(0)
        e = int(np.floor(np.log2(abs(float(q)))))
        step = Fraction(2) ** (e - 7)
        lo = (q // step) * step
        hi = lo + step
        if q - lo != hi - q:
            return lo if q - lo < hi - q else hi
        return lo if (lo / step) % 2 == 0 else hi

    via_fp32_differs = 0
    for t in range(shape.tokens):
        for k in range(shape.K):
            gk = Fraction(float(gates[t, k]))
            for h in range(shape.Hp):
                exact = gk * Fraction(float(f64(dout[t, h])))
                want = nearest_bf16(exact)
                assert Fraction(float(f64(dy[route[t, k], h]))) == want, (t, k, h)
                p32 = Fraction(float(np.float32(gates[t, k]) * np.float32(f64(dout[t, h]))))
                via_fp32_differs += nearest_bf16(p32) != want
    assert via_fp32_differs >= len(planted)


@pytest.mark.parametrize("mode,B", [(0, 2), (1, 1), (1, 0)])
def test_dgrad_adjoint_of_grouped_gemm(mode, B):
    shape = W.TINY.with_(H=32, Hp=16, mode=mode, B=B)
    cfg, ids, _, plan = tiny_setup(shape, seed=9)
    g = np.random.default_rng(13)
    xp = int_bits(g, (shape.R * shape.SK, shape.H), -1, 1)
    wh = int_bits(g, (shape.E, shape.H, shape.Hp), -1, 1)
    wp = dataflow.prefetch(wh, plan, cfg)
    dyb = int_bits(g, (shape.R * shape.SK, shape.Hp), -1, 1)
    y = dataflow.grouped_gemm(xp, wh, wp, plan, cfg)
    dx = dataflow.dgrad(dyb, wh, wp, plan, cfg)
    assert np.sum(f64(dyb) * f64(y)) == np.sum(f64(dx) * f64(xp))
    rows = np.arange(0, shape.R * shape.SK, 3)
    assert np.array_equal(dataflow.dgrad_rows(rows, dyb, wh, wp, plan, cfg), dx[rows])


def test_dgrad_closed_form_scaled_identity():
    # W[e] = c_e * I: dxperm rows of segment j are c_j * dy rows exactly.
    shape = W.TINY.with_(H=64, Hp=64)
    cfg, ids, _, plan = tiny_setup(shape, seed=3)
    g = np.random.default_rng(8)
    c = 2.0 ** (np.arange(shape.E) - 3)
    wh = bf16.f64_to_bits(c[:, None, None] * np.eye(64)[None])
    wp = dataflow.prefetch(wh, plan, cfg)
    dyb = rand_bits(g, (shape.R * shape.SK, shape.Hp))
    dx = dataflow.dgrad(dyb, wh, wp, plan, cfg)
    for r in range(shape.R):
        for j in range(shape.E + shape.B):
            lo, hi = plan.cu_seqlens[r, j], plan.cu_seqlens[r, j + 1]
            e = j if j < shape.E else plan.slot_expert[r, j - shape.E]
            rows = slice(r * shape.SK + lo, r * shape.SK + hi)
            assert np.array_equal(f64(dx[rows]), c[e] * f64(dyb[rows]))


@pytest.mark.parametrize("shape", [W.TINY, W.TINY.with_(B=1, mode=1),
                                   W.TINY.with_(R=2, E=8, K=3, S=10, B=4)])
def test_dispatch_backward_adjoint_and_round_trip(shape):
    g = np.random.default_rng(17)
    cfg, ids, _, plan = tiny_setup(shape, seed=1)
    x = int_bits(g, (shape.tokens, shape.H))
    dxp = int_bits(g, (shape.R * shape.SK, shape.H))
    dx = dataflow.dispatch_backward(dxp, plan, cfg)
    assert np.sum(f64(dxp) * f64(dataflow.dispatch(x, plan, cfg))) == np.sum(f64(dx) * f64(x))
    # every route is valid here, so the K copies of x sum back to K * x
    back = dataflow.dispatch_backward(dataflow.dispatch(x, plan, cfg), plan, cfg)
    assert np.array_equal(f64(back), shape.K * f64(x))


# ---------------------------------------------------------------------------
# Dedup encoding ([K3-blog] 在线规划、零拷贝、静态 shape).  Pinned against the
# plain route map and the pinned plain dispatch, not against itself.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape,kind", [(W.TINY, "uniform"), (W.TINY, "hot"),
                                        (W.TINY.with_(R=2, E=8, K=3, S=10, B=4), "uniform"),
                                        (W.SKEWED.with_(S=64, H=16, Hp=16), "theorem2")])
def test_route_encode_invariants_and_dedup_dispatch(shape, kind):
    cfg = cfg_of(shape)
    if kind == "hot":
        ids = W.routing_hot(shape)
    elif kind == "theorem2":
        ids = W.routing_theorem2(shape)
    else:
        ids, _ = W.routing_uniform(shape, salt=4)
    plan = make_plan(ids, cfg)
    enc = dataflow.route_encode(plan, cfg).reshape(-1, shape.K)
    route = plan.route.reshape(-1, shape.K)
    SK = shape.SK
    # decoding recovers the route; one non-negative entry per distinct
    # destination rank of the token, and it is the first one in k order
    dec = np.where(enc >= 0, enc, -enc.astype(np.int64) - 1)
    assert np.array_equal(dec, route)
    for t in range(route.shape[0]):
        ranks = route[t] // SK
        firsts = [k for k in range(shape.K) if ranks[k] not in ranks[:k]]
        assert sorted(np.nonzero(enc[t] >= 0)[0].tolist()) == firsts
    # the two-phase dispatch gives exactly the plain dispatch
    g = np.random.default_rng(6)
    x = rand_bits(g, (shape.tokens, shape.H))
    assert np.array_equal(dataflow.dispatch_dedup(x, enc, cfg), dataflow.dispatch(x, plan, cfg))


def test_route_encode_page_illustration():
    # [K3-blog]: a token whose six routes land on three ranks sends its row
    # three times; the repeats carry -(position) - 1.  Rows of rank d are
    # [d*S*K, (d+1)*S*K); the six routes hit ranks 0, 0, 1, 2, 2, 1.
    from types import SimpleNamespace
    shape = W.TINY.with_(R=4, E=8, K=6, S=2, B=2)
    cfg = cfg_of(shape)
    SK = shape.SK
    route = np.array([[0, 1, SK, 2 * SK, 2 * SK + 1, SK + 1],
                      [2, 3 * SK, 3 * SK + 1, 3 * SK + 2, 3, SK + 2]] * 4, np.int32).reshape(-1)
    enc = dataflow.route_encode(SimpleNamespace(route=route), cfg).reshape(-1, shape.K)
    assert enc[0].tolist() == [0, -2, SK, 2 * SK, -(2 * SK + 1) - 1, -(SK + 1) - 1]
    assert enc[1].tolist() == [2, 3 * SK, -(3 * SK + 1) - 1, -(3 * SK + 2) - 1, -4, SK + 2]
    assert int((enc[0] >= 0).sum()) == 3


# ---------------------------------------------------------------------------
# The tolerance scale of reduce_grad, on a hand-built slot map with values
# summed by hand (no call of the oracle's reduction).
# ---------------------------------------------------------------------------
class _SlotMap:
    def __init__(self, slot_expert):
        self.slot_expert = np.asarray(slot_expert, np.int64)


def test_reduce_terms_abs_hand_values():
    # R = 2 ranks, B = 2 slots, E = 4 experts; slot (1, 1) holds no expert.
    cfg = Cfg(R=2, S=1, E=4, K=1, H=1, Hp=2, B=2)
    plan = _SlotMap([[2, 3], [0, -1]])
    gh = np.array([1.0, -2.0, 3.0, -4.0])[:, None, None] * np.ones((4, 1, 2))
    gp = np.array([[-5.0, 6.0], [7.0, 8.0]])[:, :, None, None] * np.ones((2, 2, 1, 2))
    gp[0, 0, 0, 1] = 0.25                           # one element differs
    s = dataflow.reduce_terms_abs(gh, gp, plan, cfg)
    # e=0: |1| + |7|; e=1: |-2| only; e=2: |3| + |-5| (second column |3|+0.25);
    # e=3: |-4| + |6|; slot (1,1)'s 8 belongs to no expert
    want = np.array([[8.0, 8.0], [2.0, 2.0], [8.0, 3.25], [10.0, 10.0]])[:, None, :]
    assert np.array_equal(s, want)
    # sums of magnitudes, not magnitudes of sums: opposite signs do not cancel
    gh2 = np.full((4, 1, 2), -6.0)
    s2 = dataflow.reduce_terms_abs(gh2, np.abs(gp), plan, cfg)
    assert s2[2, 0, 0] == 11.0 and s2[1, 0, 0] == 6.0


# ---------------------------------------------------------------------------
# Sampled forms used at full sizes, each against its full form on small
# shapes (train and inference plans, uniform, hot and Theorem-2 routing).
# ---------------------------------------------------------------------------
SAMPLED_CASES = [
    (W.TINY, "uniform"), (W.TINY.with_(B=1, mode=1), "hot"),
    (W.TINY.with_(R=2, E=8, K=3, S=10, B=4), "uniform"),
    (W.ADVERSARIAL.with_(S=32, H=24, Hp=16), "theorem2"),
]


def _case(shape, kind, seed=0):
    cfg = cfg_of(shape)
    if kind == "hot":
        ids, gates = W.routing_hot(shape), W.gates_uniform(shape)
    elif kind == "theorem2":
        ids, gates = W.routing_theorem2(shape), W.gates_uniform(shape)
    else:
        ids, gates = W.routing_uniform(shape, salt=seed)
    return cfg, ids, gates, make_plan(ids, cfg)


@pytest.mark.parametrize("shape,kind", SAMPLED_CASES)
def test_sampled_forms_equal_full_forms(shape, kind):
    g = np.random.default_rng(41)
    cfg, ids, gates, plan = _case(shape, kind)
    x = rand_bits(g, (shape.tokens, shape.H))
    y = rand_bits(g, (shape.R * shape.SK, shape.Hp))
    dout = rand_bits(g, (shape.tokens, shape.Hp))
    dxp = rand_bits(g, (shape.R * shape.SK, shape.H))
    dy_in = rand_bits(g, (shape.R * shape.SK, shape.Hp))
    toks = np.unique(g.integers(0, shape.tokens, max(3, shape.tokens // 3)))
    rows = np.unique(g.integers(0, shape.R * shape.SK, max(3, shape.R * shape.SK // 3)))
    # dispatch
    xp = dataflow.dispatch(x, plan, cfg)
    assert np.array_equal(dataflow.dispatch_rows(rows, x, plan, cfg), xp[rows])
    # combine
    assert np.array_equal(dataflow.combine_tokens(toks, y, gates, plan, cfg),
                          dataflow.combine(y, gates, plan, cfg)[toks])
    # combine backward
    dy_full, dg_full = dataflow.combine_backward(dout, y, gates, plan, cfg)
    q, dy_s, dg_s = dataflow.combine_backward_tokens(toks, dout, y, gates, plan, cfg)
    assert np.array_equal(q, plan.route.reshape(-1, shape.K)[toks])
    for k in range(shape.K):
        assert np.array_equal(dy_s[:, k], dy_full[q[:, k]])
    assert np.array_equal(dg_s, dg_full[toks])
    # dispatch backward
    assert np.array_equal(dataflow.dispatch_backward_tokens(toks, dxp, plan, cfg),
                          dataflow.dispatch_backward(dxp, plan, cfg)[toks])
    # route encoding
    assert np.array_equal(dataflow.route_encode_tokens(toks, plan, cfg),
                          dataflow.route_encode(plan, cfg).reshape(-1, shape.K)[toks])
    # weight gradient, train mode only
    if cfg.mode == 0:
        gh, gp = dataflow.wgrad(xp, dy_in, plan, cfg)
        hs = np.unique(g.integers(0, shape.H, 5))
        for r in range(shape.R):
            for j in list(range(r * cfg.n, (r + 1) * cfg.n)) + list(range(cfg.E, cfg.E + cfg.B)):
                got = dataflow.wgrad_entries(r, j, hs, x, dy_in, plan, cfg)
                if j < cfg.E:
                    want = gh[j][hs]
                elif plan.slot_expert[r, j - cfg.E] >= 0:
                    want = gp[r, j - cfg.E][hs]
                else:
                    assert not got.any()
                    continue
                assert np.allclose(got, want, rtol=1e-13, atol=1e-13), (r, j)


def test_dispatch_rows_rejects_unnamed_rows():
    shape = W.TINY
    cfg, ids, _, plan = _case(shape, "uniform")
    bad = _bad_ids(shape)
    from oracle.plan import failed_plan
    fp = failed_plan(bad, cfg)
    x = np.zeros((shape.tokens, shape.H), np.uint16)
    with pytest.raises(ValueError):
        dataflow.dispatch_rows([0], x, fp, cfg)


# ---------------------------------------------------------------------------
# A failed plan (ids outside [0, E)): what every later step computes from its
# definition when there is no route and no segment.
# ---------------------------------------------------------------------------
def _bad_ids(shape, salt=3):
    ids, _ = W.routing_uniform(shape, salt=salt)
    ids = ids.copy()
    ids[1, 0] = shape.E + 2
    ids[shape.tokens - 1, shape.K - 1] = -1
    return ids


@pytest.mark.parametrize("shape", [W.TINY, W.TINY.with_(R=2, E=8, K=3, S=10, B=4)])
def test_failed_plan_and_the_steps_after_it(shape):
    from oracle.plan import STATUS_BAD_ID, STATUS_UNBALANCED, failed_plan
    cfg = cfg_of(shape)
    ids = _bad_ids(shape)
    with pytest.raises(ValueError):
        make_plan(ids, cfg)
    fp = failed_plan(ids, cfg)
    # counts over the valid ids only, by brute force
    for e in range(shape.E):
        assert fp.counts[e] == sum(1 for v in ids.reshape(-1) if v == e)
    assert fp.counts.sum() == ids.size - 2
    for r in range(shape.R):
        assert fp.load0[r] == sum(fp.counts[r * cfg.n:(r + 1) * cfg.n])
    assert fp.status == STATUS_BAD_ID | STATUS_UNBALANCED
    assert np.all(fp.route == -1) and not fp.cu_seqlens.any() and np.all(fp.slot_expert == -1)
    assert len(fp.fills) == 0 and fp.moves.shape == (0, 4)
    assert not fp.n_redundant.any() and np.all(fp.src_rank == -1)
    g = np.random.default_rng(5)
    x = rand_bits(g, (shape.tokens, shape.H))
    w = rand_bits(g, (shape.E, shape.H, shape.Hp))
    y = rand_bits(g, (shape.R * shape.SK, shape.Hp))
    gates = g.random((shape.tokens, shape.K)).astype(np.float32)
    # nothing is placed, so nothing is written
    assert not dataflow.dispatch(x, fp, cfg).any()
    assert not dataflow.prefetch(w, fp, cfg).any()
    assert not dataflow.grouped_gemm(dataflow.dispatch(x, fp, cfg), w,
                                     np.zeros((shape.R, shape.B, shape.H, shape.Hp), np.uint16),
                                     fp, cfg).any()
    # sums over no routes are zero
    assert not dataflow.combine(y, gates, fp, cfg).any()
    assert not dataflow.dispatch_backward(rand_bits(g, (shape.R * shape.SK, shape.H)), fp,
                                          cfg).any()
    dy, dg = dataflow.combine_backward(rand_bits(g, (shape.tokens, shape.Hp)), y, gates, fp, cfg)
    assert not dy.any() and not dg.any()
    # every home segment is empty: zero gradients; no slot holds an expert
    gh, gp = dataflow.wgrad(rand_bits(g, (shape.R * shape.SK, shape.H)), y, fp, cfg)
    assert not gh.any() and not gp.any()
    h0 = g.standard_normal((shape.E, 2, 3))
    p0 = g.standard_normal((shape.R, shape.B, 2, 3))
    h1, p1 = dataflow.reduce_grad(h0, p0, fp, cfg)
    assert np.array_equal(h1, h0) and np.array_equal(p1, p0)
    assert np.all(dataflow.route_encode(fp, cfg) == dataflow.NO_DEST)
    toks = np.arange(shape.tokens)
    assert not dataflow.combine_tokens(toks, y, gates, fp, cfg).any()
    assert np.all(dataflow.route_encode_tokens(toks, fp, cfg) == dataflow.NO_DEST)
