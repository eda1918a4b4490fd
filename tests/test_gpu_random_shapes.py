"""Randomised sweep of small configurations through the whole path.

Forty-eight seeded configurations drawn across the ranges the header allows
at small sizes: R in {1, 2, 3, 4, 8}, E/R in {1, 2, 3, 5, 8}, K from 1 to
min(E, 8), S from 1 to 150 tokens per rank (every fourth up to 600, so
segments span several 256-row tiles), H and H' any multiple of 8 up to 320
(every fourth up to 640), ragged against every tile size, train mode (B = E/R) or inference
with 0..E/R slots, and Zipf-biased routing of random strength.  Each runs
plan, prefetch, dispatch, grouped GEMM, combine, weight gradient and
reduce_grad (train), combine backward, data gradient, dispatch backward,
the SwiGLU first projection and backward, and the dedup encoding and
dispatch, against the oracle: bit-exact for plan, dispatch, prefetch, dy of
combine backward, route encoding and dedup dispatch; within 2e-2 per row
for the products; reduce_grad within 1e-5 of the sum of |terms|.
"""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import REDUCE_TOL, announce, assert_plan_equal, bits, cfgs, free, rows_close
from oracle import bf16, dataflow, swiglu
from oracle.plan import make_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


def draw(seed):
    g = np.random.default_rng(1000 + seed)
    R = int(g.choice([1, 2, 3, 4, 8]))
    n = int(g.choice([1, 2, 3, 5, 8]))
    E = R * n
    K = int(g.integers(1, min(E, 8) + 1))
    big = seed % 4 == 3
    S = int(g.integers(1, 601 if big else 151))
    H = 8 * int(g.integers(1, 81 if big else 41))
    Hp = 8 * int(g.integers(1, 81 if big else 41))
    train = bool(g.integers(0, 2))
    B = n if train else int(g.integers(0, n + 1))
    shape = W.TINY.with_(name="rand%d" % seed, R=R, S=S, E=E, K=K, H=H, Hp=Hp, B=B,
                         mode=0 if train else 1, cfg_id=100 + seed)
    strength = float(g.uniform(0.0, 3.0))
    return shape, strength


def dev_bf16(shape_tuple, seed):
    return W.randn_bf16(shape_tuple, seed, "cuda")


@pytest.mark.parametrize("seed", range(48))
def test_random_configuration(seed):
    shape, strength = draw(seed)
    s = shape
    announce("random shape", s, "zipf strength %.2f" % strength)
    c, oc = cfgs(s)
    ids, vals = W.ZipfRouter(s).route(strength)
    gates = W._softmax_rows(vals)
    ref = make_plan(ids, oc)
    ids_t = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    plan = mx.Plan(c)
    mx.moe_plan_run(c, ids_t, plan)
    torch.cuda.synchronize()
    assert_plan_equal({k: v.cpu().numpy() for k, v in plan.views().items()}, ref, s)

    rows, T = s.R * s.SK, s.tokens
    bf = dict(dtype=torch.bfloat16, device="cuda")
    x = dev_bf16((T, s.H), 11 * seed + 1)
    w = dev_bf16((s.E, s.H, s.Hp), 11 * seed + 2)
    dout = dev_bf16((T, s.Hp), 11 * seed + 3)
    gates_t = torch.from_numpy(gates).cuda()
    wp = torch.zeros((max(1, s.R * s.B), s.H, s.Hp), **bf)
    xp = torch.zeros((rows, s.H), **bf)
    y = torch.zeros((rows, s.Hp), **bf)
    out = torch.zeros((T, s.Hp), **bf)
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w, wp)
    mx.moe_dispatch(c, plan, x, xp)
    mx.moe_grouped_gemm(c, xp, w, wp, plan.cu_seqlens, y, 0, s.R, ws)
    mx.moe_combine(c, plan, y, gates_t, out)
    torch.cuda.synchronize()
    xb, wb, db = bits(x), bits(w), bits(dout)
    rxp = dataflow.dispatch(xb, ref, oc)
    rpref = dataflow.prefetch(wb, ref, oc)
    assert np.array_equal(bits(xp), rxp)
    if s.B:
        got_p = bits(wp)[:s.R * s.B].reshape(s.R, s.B, s.H, s.Hp)
        used = ref.slot_expert >= 0
        assert np.array_equal(got_p[used], rpref[used])
    ry = dataflow.grouped_gemm(rxp, wb, rpref, ref, oc)
    rows_close(bits(y), ry)
    rows_close(bits(out), dataflow.combine(ry, gates, ref, oc))

    # data backward from the oracle's y
    y.copy_(W.from_bits(ry, "cuda"))
    dy = torch.zeros((rows, s.Hp), **bf)
    dg = torch.zeros((T, s.K), dtype=torch.float32, device="cuda")
    dxp = torch.zeros((rows, s.H), **bf)
    dx = torch.zeros((T, s.H), **bf)
    mx.moe_combine_backward(c, plan, dout, y, gates_t, dy, dg)
    torch.cuda.synchronize()
    rdy, _ = dataflow.combine_backward(db, ry, gates, ref, oc)
    assert np.array_equal(bits(dy), rdy)
    mx.moe_grouped_gemm_dgrad(c, W.from_bits(rdy, "cuda"), w, wp, plan.cu_seqlens, dxp, 0, s.R,
                              ws)
    torch.cuda.synchronize()
    rdxp = dataflow.dgrad(rdy, wb, rpref, ref, oc)
    rows_close(bits(dxp), rdxp)
    mx.moe_dispatch_backward(c, plan, W.from_bits(rdxp, "cuda"), dx)
    torch.cuda.synchronize()
    rows_close(bits(dx), dataflow.dispatch_backward(rdxp, ref, oc), tol=1e-2)

    if s.mode == 0:
        gh = torch.full((s.E, s.H, s.Hp), 5.0, dtype=torch.float32, device="cuda")
        gp = torch.full((max(1, s.R * s.B), s.H, s.Hp), -2.0, dtype=torch.float32,
                        device="cuda")
        mx.moe_grouped_gemm_wgrad(c, plan, W.from_bits(rxp, "cuda"), W.from_bits(rdy, "cuda"),
                                  gh, gp, ws)
        torch.cuda.synchronize()
        rh, rp = dataflow.wgrad(rxp, rdy, ref, oc)
        ghn = gh.cpu().numpy()
        for e in range(s.E):
            if rh[e].any():
                rows_close(ghn[e], rh[e])
            else:
                assert not ghn[e].any(), e
        gpn = gp.cpu().numpy()[:s.R * s.B].reshape(s.R, s.B, s.H, s.Hp)
        for r in range(s.R):
            for b in range(s.B):
                if ref.slot_expert[r, b] >= 0:
                    rows_close(gpn[r, b], rp[r, b])
        # reduce_grad on seeded inputs
        gen = torch.Generator(device="cuda").manual_seed(seed)
        h0 = torch.randn(gh.shape, generator=gen, device="cuda")
        p0 = torch.randn(gp.shape, generator=gen, device="cuda")
        h0n = h0.cpu().numpy()
        p0n = p0.cpu().numpy()[:s.R * s.B].reshape(s.R, s.B, s.H, s.Hp)
        mx.moe_reduce_grad(c, plan, h0, p0)
        torch.cuda.synchronize()
        eh, ep = dataflow.reduce_grad(h0n, p0n, ref, oc)
        terms = dataflow.reduce_terms_abs(h0n, p0n, ref, oc)
        assert np.all(np.abs(h0.cpu().numpy() - eh) <= REDUCE_TOL * terms + 1e-30)
        got_p = p0.cpu().numpy()[:s.R * s.B].reshape(s.R, s.B, s.H, s.Hp)
        assert np.array_equal(got_p, ep.astype(np.float32))

    # SwiGLU first projection with H' = this shape's Hp, and its backward
    c13, oc13 = cfgs(s.with_(Hp=2 * s.Hp))
    w13 = dev_bf16((s.E, s.H, 2 * s.Hp), 11 * seed + 4)
    w13p = torch.zeros((max(1, s.R * s.B), s.H, 2 * s.Hp), **bf)
    act = torch.zeros((rows, s.Hp), **bf)
    h13 = torch.zeros((rows, 2 * s.Hp), **bf)
    mx.moe_prefetch_weight(c13, plan, w13, w13p)
    mx.moe_grouped_gemm_swiglu(c, W.from_bits(rxp, "cuda"), w13, w13p, plan.cu_seqlens, act,
                               h13, 0, s.R, ws)
    torch.cuda.synchronize()
    w13b = bits(w13)
    ract, rh13 = swiglu.swiglu_gemm(rxp, w13b, dataflow.prefetch(w13b, ref, oc13), ref, oc)
    rows_close(bits(act), ract)
    rows_close(bits(h13), rh13)
    dact = dev_bf16((rows, s.Hp), 11 * seed + 5)
    dh13 = torch.zeros_like(h13)
    mx.moe_swiglu_backward(c, W.from_bits(rh13, "cuda"), dact, dh13)
    torch.cuda.synchronize()
    g64 = bf16.bits_to_f64(bits(dh13))
    r64 = bf16.bits_to_f64(swiglu.swiglu_backward(rh13, bits(dact)))
    scale = np.abs(r64).max(axis=1, keepdims=True) + 1e-30
    assert np.all(np.abs(g64 - r64) <= 2.0 ** -7 * np.abs(r64) + 1e-4 * scale)

    # dedup encoding and two-phase dispatch
    enc = torch.zeros(T * s.K, dtype=torch.int32, device="cuda")
    xp2 = torch.zeros((rows, s.H), **bf)
    mx.moe_route_encode(c, plan, enc)
    mx.moe_dispatch_dedup(c, enc, x, xp2)
    torch.cuda.synchronize()
    assert np.array_equal(enc.cpu().numpy(), dataflow.route_encode(ref, oc))
    assert np.array_equal(bits(xp2), rxp)
