"""GPU parity of the data backward -- combine backward, the data-gradient
grouped GEMM and dispatch backward -- against the oracle.

* Small shapes (full outputs): dy of combine backward bit-exact (the exact
  product g * dout rounded once); dgates within 1e-5 * sum |dout * y|;
  dxperm rows within 2e-2 (max-norm relative per row); dx rows within 1e-2
  given the oracle's dxperm, 2e-2 end to end.
* Bench shape (R=8, S=8192, E=384, K=8, H=7168, H'=2048), maxvio 1, in the
  launch configuration the bench times: sampled tokens and rows.
"""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import (DeviceRows, OraclePref, announce, assert_plan_equal, bits, cfgs, free,
                         gpu_plan, rows_close, sample_rows, sample_segments)
from oracle import bf16, dataflow
from oracle.plan import make_plan

pytestmark = pytest.mark.gpu

SENT = 0x7E57
DGATE_TOL = 1e-5      # per entry: |gpu - ref| <= tol * sum_h |dout * y|


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
    yield W.TINY.with_(H=72, Hp=40, S=37), "uniform", 3          # ragged H, Hp
    yield W.TINY.with_(R=2, E=4, S=300, K=2, B=2, H=264, Hp=136), "hot", 0   # long segments
    # rows of more than 1,024 16-byte vectors (dispatch backward walks them in two passes)
    yield W.TINY.with_(name="wide_rows", H=9160, Hp=40, S=20), "uniform", 4
    # more routes per token than one batch of loads in flight (K = 12 > 8)
    yield W.TINY.with_(name="many_routes", R=2, E=16, K=12, S=24, B=8, H=264, Hp=72), "uniform", 5
    yield W.SKEWED, "zipf", 1.0
    yield W.SKEWED, "zipf", 15.0
    yield W.SKEWED.with_(name="skewed_adv"), "theorem2", 0


def routing(shape, kind, arg):
    if kind == "uniform":
        return W.routing_uniform(shape, salt=arg)
    if kind == "zipf":
        ids, gates, _, _ = W.routing_zipf(shape, arg)
        return ids, gates
    if kind == "hot":
        return W.routing_hot(shape), W.gates_uniform(shape)
    return W.routing_theorem2(shape), W.gates_uniform(shape)


def dgates_close(got, ref, dout_bits, y_bits, plan, K):
    route = plan.route.reshape(-1, K)
    d = bf16.bits_to_f64(dout_bits)
    y = bf16.bits_to_f64(y_bits)
    for k in range(K):
        terms = np.sum(np.abs(d * y[route[:, k]]), axis=1)
        err = np.abs(got[:, k].astype(np.float64) - ref[:, k])
        assert np.all(err <= DGATE_TOL * terms + 1e-30), (k, err.max(), terms.max())


@pytest.mark.parametrize("shape,kind,arg", list(shapes()),
                         ids=lambda v: str(getattr(v, "name", v)))
def test_data_backward_path(shape, kind, arg):
    announce("data backward", shape, kind, arg)
    c, oc = cfgs(shape)
    ids, gates = routing(shape, kind, arg)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    seed = 300 + shape.cfg_id * 10 + int(arg)
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), seed, "cuda")
    w_pref = torch.zeros((max(1, shape.R * shape.B), shape.H, shape.Hp), dtype=torch.bfloat16,
                         device="cuda")
    y = W.randn_bf16((shape.R * shape.SK, shape.Hp), seed + 1, "cuda")     # forward output
    dout = W.randn_bf16((shape.tokens, shape.Hp), seed + 2, "cuda")
    gates_t = torch.from_numpy(gates).cuda()
    dy = torch.full((shape.R * shape.SK, shape.Hp), 0, dtype=torch.int16,
                    device="cuda").fill_(SENT).view(torch.bfloat16)
    dg = torch.full((shape.tokens, shape.K), -7.0, device="cuda")
    dxp = torch.full((shape.R * shape.SK, shape.H), 0, dtype=torch.int16,
                     device="cuda").fill_(SENT).view(torch.bfloat16)
    dx = torch.zeros((shape.tokens, shape.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")

    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_combine_backward(c, plan, dout, y, gates_t, dy, dg)
    mx.moe_grouped_gemm_dgrad(c, dy, w_home, w_pref, plan.cu_seqlens, dxp, 0, shape.R, ws)
    mx.moe_dispatch_backward(c, plan, dxp, dx)
    torch.cuda.synchronize()

    wb, yb, db = bits(w_home), bits(y), bits(dout)
    ref_pref = dataflow.prefetch(wb, ref, oc)
    ref_dy, ref_dg = dataflow.combine_backward(db, yb, gates, ref, oc)
    # dy: every row is some slot's destination; bit-exact
    assert np.array_equal(bits(dy), ref_dy)
    dgates_close(dg.cpu().numpy(), ref_dg, db, yb, ref, shape.K)
    # data-gradient GEMM on the oracle's dy
    ref_dxp = dataflow.dgrad(ref_dy, wb, ref_pref, ref, oc)
    rows_close(bits(dxp), ref_dxp)
    # dispatch backward end to end, and on the oracle's dxperm
    ref_dx = dataflow.dispatch_backward(ref_dxp, ref, oc)
    rows_close(bits(dx), ref_dx)
    dx2 = torch.zeros_like(dx)
    mx.moe_dispatch_backward(c, plan, W.from_bits(ref_dxp, "cuda"), dx2)
    torch.cuda.synchronize()
    rows_close(bits(dx2), ref_dx, tol=1e-2)
    # determinism of the data-gradient GEMM
    dxp2 = torch.zeros_like(dxp)
    mx.moe_grouped_gemm_dgrad(c, dy, w_home, w_pref, plan.cu_seqlens, dxp2, 0, shape.R, ws)
    torch.cuda.synchronize()
    assert torch.equal(dxp.view(torch.int16), dxp2.view(torch.int16))


def test_dgrad_rank_range_leaves_other_ranks():
    shape = W.SKEWED
    c, oc = cfgs(shape)
    ids, _, _, _ = W.routing_zipf(shape, 10.0)
    ref = make_plan(ids, oc)
    plan, _ = gpu_plan(shape, ids)
    announce("dgrad rank range 2..6")
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), 61, "cuda")
    w_pref = torch.zeros((shape.R * shape.B, shape.H, shape.Hp), dtype=torch.bfloat16, device="cuda")
    dy = W.randn_bf16((shape.R * shape.SK, shape.Hp), 62, "cuda")
    dxp = torch.full((shape.R * shape.SK, shape.H), 0, dtype=torch.int16,
                     device="cuda").fill_(SENT).view(torch.bfloat16)
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_grouped_gemm_dgrad(c, dy, w_home, w_pref, plan.cu_seqlens, dxp, 2, 6, ws)
    torch.cuda.synchronize()
    wb = bits(w_home)
    ref_dxp = dataflow.dgrad(bits(dy), wb, dataflow.prefetch(wb, ref, oc), ref, oc,
                             ranks=[2, 3, 4, 5])
    got = bits(dxp)
    SK = shape.SK
    rows_close(got[2 * SK:6 * SK], ref_dxp[2 * SK:6 * SK])
    assert np.all(got[:2 * SK] == SENT) and np.all(got[6 * SK:] == SENT)
    with pytest.raises(mx.MoeError):
        mx.moe_grouped_gemm_dgrad(c, dy, w_home, w_pref, plan.cu_seqlens, dxp, 6, 2, ws)


def test_bench_shape_data_backward():
    """The data backward at the bench shape in the bench's launch
    configuration.  Each kernel runs on generated inputs (never on another
    kernel's output), so every oracle input is independent of the HIP path:
    combine backward on a generated y and dout, the data-gradient GEMM on a
    generated dy, dispatch backward on a generated dxperm."""
    shape = W.BENCH
    c, oc = cfgs(shape)
    ids, gates, _, mv = W.routing_zipf(shape, 1.0)
    announce("bench data backward maxvio", mv)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), 71, "cuda", chunk_rows=1)
    w_pref = torch.empty((shape.R * shape.B, shape.H, shape.Hp), dtype=torch.bfloat16,
                         device="cuda")
    y = W.randn_bf16((shape.R * shape.SK, shape.Hp), 72, "cuda")
    dout = W.randn_bf16((shape.tokens, shape.Hp), 73, "cuda")
    dy_in = W.randn_bf16((shape.R * shape.SK, shape.Hp), 74, "cuda")
    dxp_in = W.randn_bf16((shape.R * shape.SK, shape.H), 75, "cuda")
    gates_t = torch.from_numpy(gates).cuda()
    dy = torch.empty((shape.R * shape.SK, shape.Hp), dtype=torch.bfloat16, device="cuda")
    dg = torch.empty((shape.tokens, shape.K), device="cuda")
    dxp = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((shape.tokens, shape.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_combine_backward(c, plan, dout, y, gates_t, dy, dg)
    mx.moe_grouped_gemm_dgrad(c, dy_in, w_home, w_pref, plan.cu_seqlens, dxp, 0, shape.R, ws)
    mx.moe_dispatch_backward(c, plan, dxp_in, dx)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    # combine backward on sampled tokens: dy rows bit-exact, dgates
    toks = np.unique(rng.integers(0, shape.tokens, 256))
    q, want_dy, want_dg = dataflow.combine_backward_tokens(toks, DeviceRows(dout), DeviceRows(y),
                                                           gates, ref, oc)
    assert (q >= 0).all()
    for k in range(shape.K):
        got = bits(dy.index_select(0, torch.as_tensor(q[:, k], device="cuda")))
        assert np.array_equal(got, want_dy[:, k]), k
    d64 = bf16.bits_to_f64(DeviceRows(dout)[toks])
    yk = bf16.bits_to_f64(DeviceRows(y)[q.reshape(-1)]).reshape(toks.size, shape.K, -1)
    terms = np.abs(d64[:, None, :] * yk).sum(axis=2)
    got_dg = dg.index_select(0, torch.as_tensor(toks, device="cuda")).cpu().numpy()
    assert np.all(np.abs(got_dg.astype(np.float64) - want_dg) <= DGATE_TOL * terms + 1e-30)
    # data-gradient GEMM on 4096 sampled rows
    segs = sample_segments(ref, shape, rng, per_rank=6)
    rows = sample_rows(ref, shape, segs, rng, total=4096)
    wr = DeviceRows(w_home)
    ref_rows = dataflow.dgrad_rows(rows, DeviceRows(dy_in), wr, OraclePref(wr, ref), ref, oc)
    worst = rows_close(bits(dxp.index_select(0, torch.as_tensor(rows, device="cuda"))), ref_rows)
    announce("bench dgrad rows", rows.size, "worst rel err", worst)
    # dispatch backward on sampled tokens
    toks = np.unique(rng.integers(0, shape.tokens, 512))
    rows_close(bits(dx.index_select(0, torch.as_tensor(toks, device="cuda"))),
               dataflow.dispatch_backward_tokens(toks, DeviceRows(dxp_in), ref, oc), tol=1e-2)
