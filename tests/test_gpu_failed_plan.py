"""A failed plan (router ids outside [0, E)) and every step after it.

The planner reports bad ids in plan->status and leaves an empty plan: every
route -1, cu_seqlens all zero, no prefetch slot in use.  Each later step is
then run on outputs pre-filled with a sentinel and compared with the
oracle's steps on the oracle's failed plan (``oracle.plan.failed_plan``):
what a route, segment or slot addresses must keep the sentinel; sums over a
token's (absent) routes are zero; home-row weight gradients are zero.
"""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import announce, bits, cfgs, free, gpu_plan
from oracle import dataflow
from oracle.plan import failed_plan

pytestmark = pytest.mark.gpu

SENT = 0x7E57                  # a bf16 bit pattern no step writes by itself
FSENT = -7.25                  # an fp32 sentinel


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


def sentinel_bf16(*shape):
    return torch.full(shape, SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def bad_ids(shape, salt=3):
    ids, gates = W.routing_uniform(shape, salt=salt)
    ids = ids.copy()
    ids[1, 0] = shape.E + 2
    ids[shape.tokens - 1, shape.K - 1] = -1
    return ids, gates


@pytest.mark.parametrize("shape", [W.TINY, W.TINY.with_(R=2, E=8, K=3, S=10, B=4),
                                   W.SKEWED.with_(H=72, Hp=40)],
                         ids=["tiny", "r2", "skewed"])
def test_every_step_after_a_failed_plan(shape):
    c, oc = cfgs(shape)
    ids, gates = bad_ids(shape)
    ref = failed_plan(ids, oc)
    announce("failed plan", shape.name, shape.R, shape.E, shape.K)
    plan, g = gpu_plan(shape, ids)
    st = int(g["status"][2])
    assert st == ref.status, st
    assert int(g["status"][0]) == 0 and int(g["status"][1]) == 0
    assert np.array_equal(g["counts"], ref.counts)
    assert np.array_equal(g["load0"], ref.load0)
    assert np.array_equal(g["route"], ref.route)
    assert np.array_equal(g["cu_seqlens"], ref.cu_seqlens)
    assert np.array_equal(g["slot_expert"], ref.slot_expert)
    assert np.array_equal(g["n_redundant"], ref.n_redundant)
    assert np.array_equal(g["src_rank"], ref.src_rank)

    rows = shape.R * shape.SK
    x = W.randn_bf16((shape.tokens, shape.H), 81, "cuda")
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), 82, "cuda")
    y_in = W.randn_bf16((rows, shape.Hp), 83, "cuda")
    dout = W.randn_bf16((shape.tokens, shape.Hp), 84, "cuda")
    dxp_in = W.randn_bf16((rows, shape.H), 85, "cuda")
    dy_in = W.randn_bf16((rows, shape.Hp), 86, "cuda")
    gates_t = torch.from_numpy(gates).cuda()
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")

    w_pref = sentinel_bf16(max(1, shape.R * shape.B), shape.H, shape.Hp)
    xperm = sentinel_bf16(rows, shape.H)
    y = sentinel_bf16(rows, shape.Hp)
    out = sentinel_bf16(shape.tokens, shape.Hp)
    gh = torch.full((shape.E, shape.H, shape.Hp), FSENT, device="cuda")
    gp = torch.full((max(1, shape.R * shape.B), shape.H, shape.Hp), FSENT, device="cuda")
    dy = sentinel_bf16(rows, shape.Hp)
    dg = torch.full((shape.tokens, shape.K), FSENT, device="cuda")
    dxp = sentinel_bf16(rows, shape.H)
    dx = sentinel_bf16(shape.tokens, shape.H)
    enc = torch.zeros(shape.tokens * shape.K, dtype=torch.int32, device="cuda")
    xperm2 = sentinel_bf16(rows, shape.H)

    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, 0, shape.R, ws)
    mx.moe_combine(c, plan, y_in, gates_t, out)
    mx.moe_combine_backward(c, plan, dout, y_in, gates_t, dy, dg)
    mx.moe_grouped_gemm_dgrad(c, dy_in, w_home, w_pref, plan.cu_seqlens, dxp, 0, shape.R, ws)
    mx.moe_dispatch_backward(c, plan, dxp_in, dx)
    mx.moe_route_encode(c, plan, enc)
    mx.moe_dispatch_dedup(c, enc, x, xperm2)
    if shape.mode == mx.MODE_TRAIN:
        mx.moe_grouped_gemm_wgrad(c, plan, dxp_in, dy_in, gh, gp, ws)
    torch.cuda.synchronize()

    # the oracle's steps on its failed plan
    xb, yb = bits(x), bits(y_in)
    ref_xp = dataflow.dispatch(xb, ref, oc)             # nothing placed: all zero
    assert not ref_xp.any()
    assert np.all(bits(xperm) == SENT) and np.all(bits(xperm2) == SENT)
    assert np.all(bits(w_pref) == SENT)
    assert np.all(bits(y) == SENT) and np.all(bits(dxp) == SENT) and np.all(bits(dy) == SENT)
    assert np.array_equal(bits(out), dataflow.combine(yb, gates, ref, oc))
    _, ref_dg = dataflow.combine_backward(bits(dout), yb, gates, ref, oc)
    assert np.array_equal(dg.cpu().numpy().astype(np.float64), ref_dg)
    assert np.array_equal(bits(dx), dataflow.dispatch_backward(bits(dxp_in), ref, oc))
    assert np.array_equal(enc.cpu().numpy(), dataflow.route_encode(ref, oc))
    if shape.mode == mx.MODE_TRAIN:
        ref_gh, _ = dataflow.wgrad(bits(dxp_in), bits(dy_in), ref, oc)
        assert np.array_equal(gh.cpu().numpy().astype(np.float64), ref_gh)
        assert torch.all(gp == FSENT)
        # reduce_grad consumes no slot: both buffers unchanged
        gh.fill_(1.5)
        mx.moe_reduce_grad(c, plan, gh, gp)
        torch.cuda.synchronize()
        assert torch.all(gh == 1.5) and torch.all(gp == FSENT)
