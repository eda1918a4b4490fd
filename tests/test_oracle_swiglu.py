"""Pins for oracle.swiglu (CPU only).

Expected values come from SciPy's logistic function (scipy.special.expit)
and the tanh form of it, from
closed forms with W13[e] = [c_e I | d_e I] (powers of two, so gate and up are
exact multiples of x), from a brute-force loop on small-integer data (exact
sums), and from central finite differences of the forward map -- not from
the oracle's own formulas.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import workloads as W
from oracle import bf16, dataflow, swiglu
from oracle.plan import Cfg, make_plan


def silu_ref(z):
    return np.asarray(z, np.float64) * expit(np.asarray(z, np.float64))


def silu_tanh(z):
    # logistic(z) = (1 + tanh(z / 2)) / 2; loses relative accuracy for z << 0
    return z * (1.0 + np.tanh(np.asarray(z, np.float64) / 2.0)) / 2.0


def setup(shape, seed=0):
    cfg = Cfg(shape.R, shape.S, shape.E, shape.K, shape.H, shape.Hp, shape.B, shape.mode)
    ids, gates = W.routing_uniform(shape, salt=seed)
    return cfg, ids, make_plan(ids, cfg)


def test_silu_against_library_logistic_and_limits():
    z = np.concatenate([np.linspace(-60, 60, 4001), [-1e-8, 1e-8, 0.5, -0.5]])
    np.testing.assert_allclose(swiglu.silu(z), silu_ref(z), rtol=1e-14, atol=1e-300)
    pos = z[z >= -2]
    np.testing.assert_allclose(swiglu.silu(pos), silu_tanh(pos), rtol=1e-13, atol=1e-300)
    # silu(-z) = silu(z) - z
    np.testing.assert_allclose(swiglu.silu(-z), swiglu.silu(z) - z, rtol=1e-12, atol=1e-12)
    assert swiglu.silu(0.0) == 0.0
    assert swiglu.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert swiglu.silu(60.0) == pytest.approx(60.0, rel=1e-15)
    assert swiglu.silu(-800.0) == 0.0          # sigmoid underflows to zero


@pytest.mark.parametrize("mode,B", [(0, 2), (1, 1)])
def test_swiglu_gemm_closed_form_scaled_identity(mode, B):
    # W13[e] = [c_e I | d_e I]: gate = c_e x and up = d_e x exactly, so
    # act = bf16(silu(c_e x) * d_e x) and h13 = [c_e x | d_e x] bit for bit.
    shape = W.TINY.with_(H=32, Hp=32, mode=mode, B=B)
    cfg, ids, plan = setup(shape, seed=5)
    g = np.random.default_rng(21)
    x = bf16.f64_to_bits(g.standard_normal((shape.tokens, shape.H)))
    c = 2.0 ** (np.arange(shape.E) - 3)
    d = 2.0 ** (2 - np.arange(shape.E))
    eye = np.eye(shape.H)
    w13 = bf16.f64_to_bits(np.stack([np.concatenate([c[e] * eye, d[e] * eye], axis=1)
                                     for e in range(shape.E)]))
    xp = dataflow.dispatch(x, plan, cfg)
    wp = dataflow.prefetch(w13, plan, cfg)
    act, h13 = swiglu.swiglu_gemm(xp, w13, wp, plan, cfg)
    xv = bf16.bits_to_f64(x)
    for i in range(ids.size):
        q, t, e = plan.route[i], i // shape.K, ids.reshape(-1)[i]
        gate, up = c[e] * xv[t], d[e] * xv[t]
        assert np.array_equal(act[q], bf16.f64_to_bits(silu_ref(gate) * up)), i
        assert np.array_equal(h13[q], bf16.f64_to_bits(np.concatenate([gate, up]))), i
    rows = np.arange(0, shape.R * cfg.SK, 3)
    ar, hr = swiglu.swiglu_gemm_rows(rows, x, w13, wp, plan, cfg)
    assert np.array_equal(ar, act[rows]) and np.array_equal(hr, h13[rows])


def test_swiglu_gemm_brute_force_small_integers():
    # Small-integer x and W13 in eighths: every dot product is exact, so the
    # loop below and the oracle see the same gate and up.
    shape = W.TINY.with_(H=8, Hp=4, S=6)
    cfg, ids, plan = setup(shape, seed=2)
    g = np.random.default_rng(8)
    x = bf16.f64_to_bits(g.integers(-4, 5, (shape.tokens, shape.H)).astype(np.float64))
    w13 = bf16.f64_to_bits(g.integers(-8, 9, (shape.E, shape.H, 2 * shape.Hp)) / 8.0)
    xp = dataflow.dispatch(x, plan, cfg)
    wp = dataflow.prefetch(w13, plan, cfg)
    act, h13 = swiglu.swiglu_gemm(xp, w13, wp, plan, cfg)
    xv, wv = bf16.bits_to_f64(x), bf16.bits_to_f64(w13)
    for i in range(ids.size):
        q, t, e = plan.route[i], i // shape.K, ids.reshape(-1)[i]
        h = [sum(xv[t, k] * wv[e, k, col] for k in range(shape.H)) for col in range(2 * shape.Hp)]
        for col in range(shape.Hp):
            gate, up = h[col], h[shape.Hp + col]
            want = bf16.f64_to_bits(gate * float(expit(gate)) * up)
            assert act[q, col] == want, (i, col)
        assert np.array_equal(h13[q], bf16.f64_to_bits(np.array(h))), i


def test_swiglu_backward_finite_differences():
    g = np.random.default_rng(4)
    gate = g.standard_normal(4000) * 3.0
    up = g.standard_normal(4000)
    dact = g.standard_normal(4000)
    dgate, dup = swiglu.swiglu_backward_f64(gate, up, dact)
    eps = 1e-5 * np.maximum(1.0, np.abs(gate))
    f = lambda a, b: silu_ref(a) * b
    num_g = dact * (f(gate + eps, up) - f(gate - eps, up)) / (2 * eps)
    num_u = dact * (f(gate, up + 0.5) - f(gate, up - 0.5))     # linear in up
    np.testing.assert_allclose(dgate, num_g, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(dup, num_u, rtol=1e-12, atol=1e-12)


def test_swiglu_backward_bits_layout_special_cases():
    # gate = 0: sigmoid = 1/2, so d gate = d act * up / 2 and d up = 0.
    # gate = 100: sigmoid = 1 in float64, so d gate = d act * up, d up = d act * gate.
    g = np.random.default_rng(6)
    H = 24
    up = bf16.f64_to_bits(g.standard_normal((5, H)))
    dact = bf16.f64_to_bits(g.standard_normal((5, H)))
    upv, dv = bf16.bits_to_f64(up), bf16.bits_to_f64(dact)
    zero = np.zeros((5, H), np.uint16)
    out = swiglu.swiglu_backward(np.concatenate([zero, up], axis=1), dact)
    assert np.array_equal(out[:, :H], bf16.f64_to_bits(dv * upv / 2))
    assert not (out[:, H:] & 0x7FFF).any()
    big = bf16.f64_to_bits(np.full((5, H), 100.0))
    out = swiglu.swiglu_backward(np.concatenate([big, up], axis=1), dact)
    assert np.array_equal(out[:, :H], bf16.f64_to_bits(dv * upv))
    assert np.array_equal(out[:, H:], bf16.f64_to_bits(dv * 100.0))
