"""GPU parity of the two-projection SwiGLU expert against the oracle.

* moe_grouped_gemm_swiglu: act and h13 rows within 2e-2 (max-norm relative
  per row) of oracle.swiglu.swiglu_gemm on small shapes (ragged H and H',
  several column tiles, inference with few or no prefetch slots); act is the
  same bit for bit with and without h13, and h13 equals the plain grouped
  GEMM over [E+B, H, 2H'] bit for bit (same products, same order).
* moe_swiglu_backward: every element within one bf16 rounding of the
  oracle, |gpu - ref| <= 2^-7 |ref| + 2^-18 |d act * up| (1 + |gate|)
  + 1e-30 (the second term covers the fp32 cancellation in
  1 + gate (1 - s) near its root), in place and out of place.
* A whole expert (first projection + activation, second projection,
  combine, and the backward through both projections) on small shapes,
  against the oracle's chain from the same inputs.
* Bench shape (R=8, S=8192, E=384, K=8, H=7168, H'=2048), maxvio 1, in the
  launch configuration the bench times: sampled rows.
"""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import (DeviceRows, OraclePref, announce, assert_plan_equal, bits, cfgs, free,
                         gpu_plan, rows_close, sample_rows, sample_segments)
from oracle import bf16, dataflow, swiglu
from oracle.plan import make_plan

pytestmark = pytest.mark.gpu

SENT = 0x7E57


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


def shapes():
    yield W.TINY, "uniform", 0
    yield W.TINY.with_(B=1, mode=1), "uniform", 1
    yield W.TINY.with_(B=0, mode=1), "uniform", 2
    yield W.TINY.with_(H=72, Hp=40, S=37), "uniform", 3          # ragged H, H'
    yield W.TINY.with_(R=2, E=4, S=300, K=2, B=2, H=264, Hp=136), "hot", 0   # 2 column tiles
    yield W.SKEWED, "zipf", 10.0
    yield W.SKEWED.with_(name="skewed_adv", Hp=256), "theorem2", 0


def routing(shape, kind, arg):
    if kind == "uniform":
        return W.routing_uniform(shape, salt=arg)
    if kind == "zipf":
        ids, gates, _, _ = W.routing_zipf(shape, arg)
        return ids, gates
    if kind == "hot":
        return W.routing_hot(shape), W.gates_uniform(shape)
    return W.routing_theorem2(shape), W.gates_uniform(shape)


def proj_cfgs(shape, H_in, H_out):
    """moe_cfg and oracle Cfg of one projection [E+B, H_in, H_out]."""
    return cfgs(shape.with_(H=H_in, Hp=H_out))


def sentinel(rows, cols):
    return torch.full((rows, cols), 0, dtype=torch.int16, device="cuda").fill_(SENT).view(
        torch.bfloat16)


@pytest.mark.parametrize("shape,kind,arg", list(shapes()),
                         ids=lambda v: str(getattr(v, "name", v)))
def test_swiglu_gemm(shape, kind, arg):
    announce("swiglu gemm", shape, kind, arg)
    c, oc = cfgs(shape)                                  # Hp = H'
    c13, _ = proj_cfgs(shape, shape.H, 2 * shape.Hp)
    ids, _ = routing(shape, kind, arg)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    seed = 500 + shape.cfg_id * 10 + int(arg)
    x = W.randn_bf16((shape.tokens, shape.H), seed, "cuda")
    w13 = W.randn_bf16((shape.E, shape.H, 2 * shape.Hp), seed + 1, "cuda")
    w13p = torch.zeros((max(1, shape.R * shape.B), shape.H, 2 * shape.Hp), dtype=torch.bfloat16,
                       device="cuda")
    rows = shape.R * shape.SK
    xp = torch.empty((rows, shape.H), dtype=torch.bfloat16, device="cuda")
    act, h13 = sentinel(rows, shape.Hp), sentinel(rows, 2 * shape.Hp)
    ws = torch.empty(mx.moe_gemm_workspace_size(c13), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c13, plan, w13, w13p)
    mx.moe_dispatch(c, plan, x, xp)
    mx.moe_grouped_gemm_swiglu(c, xp, w13, w13p, plan.cu_seqlens, act, h13, 0, shape.R, ws)
    torch.cuda.synchronize()

    xb, wb = bits(x), bits(w13)
    ref_xp = dataflow.dispatch(xb, ref, oc)
    ref_act, ref_h13 = swiglu.swiglu_gemm(ref_xp, wb, dataflow.prefetch(wb, ref, oc), ref, oc)
    worst = rows_close(bits(act), ref_act)
    rows_close(bits(h13), ref_h13)
    announce("act worst rel err", worst)
    # act alone (no h13) is the same computation
    act2 = sentinel(rows, shape.Hp)
    mx.moe_grouped_gemm_swiglu(c, xp, w13, w13p, plan.cu_seqlens, act2, None, 0, shape.R, ws)
    # h13 is the plain grouped GEMM over [E+B, H, 2H']
    y13 = sentinel(rows, 2 * shape.Hp)
    mx.moe_grouped_gemm(c13, xp, w13, w13p, plan.cu_seqlens, y13, 0, shape.R, ws)
    torch.cuda.synchronize()
    assert torch.equal(act.view(torch.int16), act2.view(torch.int16))
    assert torch.equal(h13.view(torch.int16), y13.view(torch.int16))


def swiglu_bwd_close(got_bits, ref_bits, h13_bits, dact_bits):
    Hp = dact_bits.shape[-1]
    g = bf16.bits_to_f64(got_bits)
    r = bf16.bits_to_f64(ref_bits)
    h = bf16.bits_to_f64(h13_bits)
    d = bf16.bits_to_f64(dact_bits)
    gate, up = h[:, :Hp], h[:, Hp:]
    slack = np.concatenate([np.abs(d * up) * (1 + np.abs(gate)),
                            np.abs(d * gate)], axis=1) * 2.0 ** -18
    err = np.abs(g - r)
    bound = 2.0 ** -7 * np.abs(r) + slack + 1e-30
    bad = ~(err <= bound)
    assert not bad.any(), (np.argwhere(bad)[:6], g[bad][:6], r[bad][:6])


@pytest.mark.parametrize("R,S,K,Hp", [(4, 16, 2, 64), (2, 37, 3, 40), (8, 512, 4, 512)])
def test_swiglu_backward(R, S, K, Hp):
    announce("swiglu backward", R, S, K, Hp)
    shape = W.TINY.with_(R=R, S=S, K=K, E=8 if R <= 4 else 64, B=8 // R if R <= 4 else 8, Hp=Hp)
    c, _ = cfgs(shape)
    rows = R * S * K
    rng = np.random.default_rng(R * 1000 + S)
    gate = rng.standard_normal((rows, Hp)) * 3.0
    # planted special gates: zero, tiny, near the root of 1 + g(1 - s),
    # large of both signs, past the fp32 exp range
    special = np.array([0.0, 1e-3, -1e-3, -1.2785, 20.0, -20.0, 87.0, -87.0, 100.0, -100.0])
    gate.reshape(-1)[:special.size] = special
    h13b = bf16.f64_to_bits(np.concatenate([gate, rng.standard_normal((rows, Hp))], axis=1))
    dactb = bf16.f64_to_bits(rng.standard_normal((rows, Hp)))
    ref = swiglu.swiglu_backward(h13b, dactb)
    h13 = W.from_bits(h13b, "cuda")
    dact = W.from_bits(dactb, "cuda")
    out = sentinel(rows, 2 * Hp)
    mx.moe_swiglu_backward(c, h13, dact, out)
    torch.cuda.synchronize()
    swiglu_bwd_close(bits(out), ref, h13b, dactb)
    mx.moe_swiglu_backward(c, h13, dact, h13)            # in place
    torch.cuda.synchronize()
    assert torch.equal(h13.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("shape,kind,arg", [(W.TINY, "uniform", 0),
                                            (W.TINY.with_(H=72, Hp=40, S=37), "uniform", 3),
                                            (W.SKEWED.with_(H=256, Hp=128), "zipf", 10.0)],
                         ids=lambda v: str(getattr(v, "name", v)))
def test_swiglu_expert_forward_backward(shape, kind, arg):
    """x -> [W13, SwiGLU] -> act -> [W2] -> y -> combine -> out, and back."""
    announce("swiglu expert", shape, kind, arg)
    H, Hi = shape.H, shape.Hp                            # model width, intermediate size
    c, oc = cfgs(shape)
    c13, oc13 = proj_cfgs(shape, H, 2 * Hi)
    c2, oc2 = proj_cfgs(shape, Hi, H)
    ids, gates = routing(shape, kind, arg)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    seed = 700 + shape.cfg_id
    rows, R, B, E = shape.R * shape.SK, shape.R, shape.B, shape.E
    x = W.randn_bf16((shape.tokens, H), seed, "cuda")
    w13 = W.randn_bf16((E, H, 2 * Hi), seed + 1, "cuda")
    w2 = W.randn_bf16((E, Hi, H), seed + 2, "cuda")
    dout = W.randn_bf16((shape.tokens, H), seed + 3, "cuda")
    gates_t = torch.from_numpy(gates).cuda()
    dev = dict(dtype=torch.bfloat16, device="cuda")
    w13p = torch.zeros((R * B, H, 2 * Hi), **dev)
    w2p = torch.zeros((R * B, Hi, H), **dev)
    xp, act, h13 = (torch.empty((rows, H), **dev), torch.empty((rows, Hi), **dev),
                    torch.empty((rows, 2 * Hi), **dev))
    y, out = torch.empty((rows, H), **dev), torch.empty((shape.tokens, H), **dev)
    dy, dact = torch.empty((rows, H), **dev), torch.empty((rows, Hi), **dev)
    dxp, dx = torch.empty((rows, H), **dev), torch.empty((shape.tokens, H), **dev)
    dg = torch.empty((shape.tokens, shape.K), device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    g13h, g13p = torch.zeros((E, H, 2 * Hi), **f32), torch.zeros((R * B, H, 2 * Hi), **f32)
    g2h, g2p = torch.zeros((E, Hi, H), **f32), torch.zeros((R * B, Hi, H), **f32)
    ws = torch.empty(max(mx.moe_gemm_workspace_size(cc) for cc in (c13, c2)), dtype=torch.uint8,
                     device="cuda")
    # forward
    mx.moe_prefetch_weight(c13, plan, w13, w13p)
    mx.moe_prefetch_weight(c2, plan, w2, w2p)
    mx.moe_dispatch(c, plan, x, xp)
    mx.moe_grouped_gemm_swiglu(c, xp, w13, w13p, plan.cu_seqlens, act, h13, 0, R, ws)
    mx.moe_grouped_gemm(c2, act, w2, w2p, plan.cu_seqlens, y, 0, R, ws)
    mx.moe_combine(c2, plan, y, gates_t, out)
    # backward
    mx.moe_combine_backward(c2, plan, dout, y, gates_t, dy, dg)
    mx.moe_grouped_gemm_dgrad(c2, dy, w2, w2p, plan.cu_seqlens, dact, 0, R, ws)
    mx.moe_grouped_gemm_wgrad(c2, plan, act, dy, g2h, g2p, ws)
    mx.moe_swiglu_backward(c, h13, dact, h13)            # h13 now holds d h13
    mx.moe_grouped_gemm_wgrad(c13, plan, xp, h13, g13h, g13p, ws)
    mx.moe_grouped_gemm_dgrad(c13, h13, w13, w13p, plan.cu_seqlens, dxp, 0, R, ws)
    mx.moe_dispatch_backward(c, plan, dxp, dx)
    mx.moe_reduce_grad(c13, plan, g13h, g13p)
    mx.moe_reduce_grad(c2, plan, g2h, g2p)
    torch.cuda.synchronize()

    # the oracle's chain from the same inputs
    xb, w13b, w2b, doutb = bits(x), bits(w13), bits(w2), bits(dout)
    o_xp = dataflow.dispatch(xb, ref, oc)
    o_act, o_h13 = swiglu.swiglu_gemm(o_xp, w13b, dataflow.prefetch(w13b, ref, oc13), ref, oc)
    w2pb = dataflow.prefetch(w2b, ref, oc2)
    o_y = dataflow.grouped_gemm(o_act, w2b, w2pb, ref, oc2)
    o_out = dataflow.combine(o_y, gates, ref, oc2)
    o_dy, _ = dataflow.combine_backward(doutb, o_y, gates, ref, oc2)
    o_dact = dataflow.dgrad(o_dy, w2b, w2pb, ref, oc2)
    o_g2h, o_g2p = dataflow.wgrad(o_act, o_dy, ref, oc2)
    o_dh13 = swiglu.swiglu_backward(o_h13, o_dact)
    o_g13h, o_g13p = dataflow.wgrad(o_xp, o_dh13, ref, oc13)
    o_dxp = dataflow.dgrad(o_dh13, w13b, dataflow.prefetch(w13b, ref, oc13), ref, oc13)
    o_dx = dataflow.dispatch_backward(o_dxp, ref, oc)
    o_g13h, _ = dataflow.reduce_grad(o_g13h, o_g13p, ref, oc13)
    o_g2h, _ = dataflow.reduce_grad(o_g2h, o_g2p, ref, oc2)

    rows_close(bits(act), o_act)
    rows_close(bits(out), o_out)
    rows_close(bits(dact), o_dact)
    rows_close(bits(dx), o_dx)
    rows_close(g2h.cpu().numpy().reshape(-1, H), o_g2h.reshape(-1, H))
    rows_close(g13h.cpu().numpy().reshape(-1, 2 * Hi), o_g13h.reshape(-1, 2 * Hi))


def test_bench_shape_swiglu():
    shape = W.BENCH
    c, oc = cfgs(shape)
    c13, _ = proj_cfgs(shape, shape.H, 2 * shape.Hp)
    ids, _, _, mv = W.routing_zipf(shape, 1.0)
    announce("bench swiglu maxvio", mv)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    rows_n = shape.R * shape.SK
    x = W.randn_bf16((shape.tokens, shape.H), 81, "cuda")
    w13 = W.randn_bf16((shape.E, shape.H, 2 * shape.Hp), 82, "cuda", chunk_rows=1)
    w13p = torch.empty((shape.R * shape.B, shape.H, 2 * shape.Hp), dtype=torch.bfloat16,
                       device="cuda")
    xp = torch.empty((rows_n, shape.H), dtype=torch.bfloat16, device="cuda")
    act = torch.empty((rows_n, shape.Hp), dtype=torch.bfloat16, device="cuda")
    h13 = torch.empty((rows_n, 2 * shape.Hp), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c13), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c13, plan, w13, w13p)
    mx.moe_dispatch(c, plan, x, xp)
    mx.moe_grouped_gemm_swiglu(c, xp, w13, w13p, plan.cu_seqlens, act, h13, 0, shape.R, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    segs = sample_segments(ref, shape, rng, per_rank=6)
    rows = sample_rows(ref, shape, segs, rng, total=2048)
    wr = DeviceRows(w13)
    ref_act, ref_h13 = swiglu.swiglu_gemm_rows(rows, DeviceRows(x), wr, OraclePref(wr, ref),
                                               ref, oc)
    idx = torch.as_tensor(rows, device="cuda")
    worst = rows_close(bits(act.index_select(0, idx)), ref_act)
    rows_close(bits(h13.index_select(0, idx)), ref_h13)
    announce("bench swiglu rows", rows.size, "worst rel err", worst)
    # activation backward over all rows (generated h13 and d act), checked
    # on the sampled ones
    del act, xp
    h13.copy_(W.randn_bf16((rows_n, 2 * shape.Hp), 84, "cuda"))
    dact = W.randn_bf16((rows_n, shape.Hp), 83, "cuda")
    dh13 = torch.empty_like(h13)
    mx.moe_swiglu_backward(c, h13, dact, dh13)
    torch.cuda.synchronize()
    hb, db = bits(h13.index_select(0, idx)), bits(dact.index_select(0, idx))
    swiglu_bwd_close(bits(dh13.index_select(0, idx)), swiglu.swiglu_backward(hb, db), hb, db)


def test_swiglu_gemm_rank_range_leaves_other_ranks():
    shape = W.SKEWED.with_(H=256, Hp=128)
    c, oc = cfgs(shape)
    c13, _ = proj_cfgs(shape, shape.H, 2 * shape.Hp)
    ids, _, _, _ = W.routing_zipf(shape, 10.0)
    ref = make_plan(ids, oc)
    plan, _ = gpu_plan(shape, ids)
    announce("swiglu rank range 2..6")
    x = W.randn_bf16((shape.tokens, shape.H), 91, "cuda")
    w13 = W.randn_bf16((shape.E, shape.H, 2 * shape.Hp), 92, "cuda")
    w13p = torch.zeros((shape.R * shape.B, shape.H, 2 * shape.Hp), dtype=torch.bfloat16,
                       device="cuda")
    rows = shape.R * shape.SK
    xp = torch.empty((rows, shape.H), dtype=torch.bfloat16, device="cuda")
    act, h13 = sentinel(rows, shape.Hp), sentinel(rows, 2 * shape.Hp)
    ws = torch.empty(mx.moe_gemm_workspace_size(c13), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c13, plan, w13, w13p)
    mx.moe_dispatch(c, plan, x, xp)
    mx.moe_grouped_gemm_swiglu(c, xp, w13, w13p, plan.cu_seqlens, act, h13, 2, 6, ws)
    torch.cuda.synchronize()
    wb = bits(w13)
    ref_act, ref_h13 = swiglu.swiglu_gemm(dataflow.dispatch(bits(x), ref, oc), wb,
                                          dataflow.prefetch(wb, ref, oc), ref, oc,
                                          ranks=[2, 3, 4, 5])
    SK = shape.SK
    ga, gh = bits(act), bits(h13)
    rows_close(ga[2 * SK:6 * SK], ref_act[2 * SK:6 * SK])
    rows_close(gh[2 * SK:6 * SK], ref_h13[2 * SK:6 * SK])
    for g in (ga, gh):
        assert np.all(g[:2 * SK] == SENT) and np.all(g[6 * SK:] == SENT)
    with pytest.raises(mx.MoeError):
        mx.moe_grouped_gemm_swiglu(c, xp, w13, w13p, plan.cu_seqlens, act, h13, 6, 2, ws)
