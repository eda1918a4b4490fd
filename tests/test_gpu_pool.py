"""GPU test of the multi-layer prefetch pool.

[MoonEP-news] 核心思想: the prefetch slots come from one rank-global pool
shared by all layers, so the extra memory is B expert weights per
projection in total, not per layer.  Here every layer of a projection uses
one slot buffer w_pool [R][B][H][H'] and one reduce buffer g_pool
[R][B][H][H'] (fp32); the ordering rules that make this safe:

* forward: a layer's prefetch overwrites the slots after the previous
  layer's grouped GEMM has read them (same stream);
* backward (last layer first): the pool holds the next layer's slots, so
  each layer re-prefetches its own before its data-gradient GEMM; that copy
  runs on a second stream which waits for the previous user's last read (its
  data-gradient GEMM) and overlaps that layer's weight gradient, reduce_grad
  and dispatch backward;
* a layer's weight gradient writes g_pool only after the previous layer's
  reduce_grad has consumed it (same stream).

Checks: three layers with different routings (zipf maxvio 1 and 10, the
Theorem-2 case) and weights; every layer's y, out, dy, dxperm, dx and
reduced grad_home equal, bit for bit, those of the same layers run with
private slot and reduce buffers on one stream (the pool changes no
arithmetic); and each layer's y and reduced grad_home are within 2e-2 per
row of the oracle.
"""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import announce, bits, cfgs, free, rows_close
from oracle import dataflow
from oracle.plan import POLICY_LARGEST, make_plan

pytestmark = pytest.mark.gpu

SHAPE = W.SKEWED.with_(H=256, Hp=128)


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


def routing(k):
    if k == 0:
        ids, gates, _, _ = W.routing_zipf(SHAPE, 1.0)
    elif k == 1:
        ids, gates, _, _ = W.routing_zipf(SHAPE, 10.0)
    else:
        ids, gates = W.routing_theorem2(SHAPE), W.gates_uniform(SHAPE)
    return ids, gates


class Layer:
    def __init__(self, k, c):
        s = SHAPE
        dev = "cuda"
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.ids_np, self.gates_np = routing(k)
        self.ids = torch.from_numpy(np.ascontiguousarray(self.ids_np, np.int32)).to(dev)
        self.gates = torch.from_numpy(self.gates_np).to(dev)
        self.x = W.randn_bf16((s.tokens, s.H), 900 + 10 * k, dev)
        self.w = W.randn_bf16((s.E, s.H, s.Hp), 901 + 10 * k, dev)
        self.dout = W.randn_bf16((s.tokens, s.Hp), 902 + 10 * k, dev)
        self.plan = mx.Plan(c, dev)
        rows = s.R * s.SK
        self.xperm, self.y = torch.empty((rows, s.H), **bf), torch.empty((rows, s.Hp), **bf)
        self.out = torch.empty((s.tokens, s.Hp), **bf)
        self.dy, self.dxp = torch.empty((rows, s.Hp), **bf), torch.empty((rows, s.H), **bf)
        self.dx = torch.empty((s.tokens, s.H), **bf)
        self.dg = torch.empty((s.tokens, s.K), dtype=torch.float32, device=dev)
        self.gh = torch.zeros((s.E, s.H, s.Hp), dtype=torch.float32, device=dev)

    def outputs(self):
        return [self.y, self.out, self.dy, self.dxp, self.dx, self.gh]


def forward(c, L, w_slots, ws):
    mx.moe_plan_run_policy(c, L.ids, L.plan, mx.PLAN_LARGEST_FIRST)
    mx.moe_prefetch_weight(c, L.plan, L.w, w_slots)
    mx.moe_dispatch(c, L.plan, L.x, L.xperm)
    mx.moe_grouped_gemm(c, L.xperm, L.w, w_slots, L.plan.cu_seqlens, L.y, 0, SHAPE.R, ws)
    mx.moe_combine(c, L.plan, L.y, L.gates, L.out)


def backward_tail(c, L, g_slots, ws):
    mx.moe_grouped_gemm_wgrad(c, L.plan, L.xperm, L.dy, L.gh, g_slots, ws)
    mx.moe_reduce_grad(c, L.plan, L.gh, g_slots)
    mx.moe_dispatch_backward(c, L.plan, L.dxp, L.dx)


def test_shared_prefetch_pool_three_layers():
    s = SHAPE
    c, oc = cfgs(s)
    nl = 3
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    # private slot and reduce buffers, one stream
    announce("pool: private buffers")
    priv = [Layer(k, c) for k in range(nl)]
    for L in priv:
        wp = torch.zeros((s.R * s.B, s.H, s.Hp), dtype=torch.bfloat16, device="cuda")
        gp = torch.zeros((s.R * s.B, s.H, s.Hp), dtype=torch.float32, device="cuda")
        L.wp, L.gp = wp, gp
        forward(c, L, wp, ws)
    for L in reversed(priv):
        mx.moe_combine_backward(c, L.plan, L.dout, L.y, L.gates, L.dy, L.dg)
        mx.moe_grouped_gemm_dgrad(c, L.dy, L.w, L.wp, L.plan.cu_seqlens, L.dxp, 0, s.R, ws)
        backward_tail(c, L, L.gp, ws)
    torch.cuda.synchronize()

    # one pool for every layer; backward re-prefetch on a second stream
    announce("pool: shared buffers, two streams")
    pooled = [Layer(k, c) for k in range(nl)]
    w_pool = torch.zeros((s.R * s.B, s.H, s.Hp), dtype=torch.bfloat16, device="cuda")
    g_pool = torch.zeros((s.R * s.B, s.H, s.Hp), dtype=torch.float32, device="cuda")
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()                       # default priority
    for L in pooled:
        forward(c, L, w_pool, ws)
    filled = [torch.cuda.Event() for _ in range(nl)]
    released = [torch.cuda.Event() for _ in range(nl)]
    for i in reversed(range(nl)):
        L = pooled[i]
        if i != nl - 1:
            compute.wait_event(filled[i])            # this layer's slots are back
        mx.moe_combine_backward(c, L.plan, L.dout, L.y, L.gates, L.dy, L.dg)
        mx.moe_grouped_gemm_dgrad(c, L.dy, L.w, w_pool, L.plan.cu_seqlens, L.dxp, 0, s.R, ws)
        released[i].record(compute)                  # last read of the slots
        if i > 0:
            prev = pooled[i - 1]
            copy.wait_event(released[i])
            with torch.cuda.stream(copy):
                mx.moe_prefetch_weight(c, prev.plan, prev.w, w_pool, stream=copy)
            filled[i - 1].record(copy)
        backward_tail(c, L, g_pool, ws)
    torch.cuda.synchronize()

    for k in range(nl):
        announce("pool: layer", k)
        for a, b in zip(priv[k].outputs(), pooled[k].outputs()):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), k
        # against the oracle, layer by layer
        Lp = pooled[k]
        ref = make_plan(Lp.ids_np, oc, policy=POLICY_LARGEST)
        xb, wb = bits(Lp.x), bits(Lp.w)
        pref = dataflow.prefetch(wb, ref, oc)
        xp = dataflow.dispatch(xb, ref, oc)
        ry = dataflow.grouped_gemm(xp, wb, pref, ref, oc)
        rows_close(bits(Lp.y), ry)
        rdy, _ = dataflow.combine_backward(bits(Lp.dout), ry, Lp.gates_np, ref, oc)
        gh, gp = dataflow.wgrad(xp, rdy, ref, oc)
        eh, _ = dataflow.reduce_grad(gh, gp, ref, oc)
        rows_close(Lp.gh.cpu().numpy().reshape(-1, s.Hp), eh.reshape(-1, s.Hp))
