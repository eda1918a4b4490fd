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
