"""GPU parity of prefetch, dispatch, grouped GEMM, combine, wgrad and
reduce_grad against the oracle, on shapes the oracle finishes in seconds
(full outputs compared; several tiles and ragged tails).

Bit-exact: prefetch and dispatch.  Within 2e-2 per row (max-norm relative):
grouped GEMM, combine, weight gradients.  reduce_grad: |gpu - ref| <= 1e-5 *
sum |terms| per element, consumed slots exactly zero, others untouched.
"""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import (REDUCE_TOL, announce, assert_plan_equal, bits, cfgs, free, gpu_plan,
                         rows_close)
from oracle import bf16, dataflow
from oracle.plan import make_plan

pytestmark = pytest.mark.gpu

SENT = 0x7E57  # bf16 bit pattern used to detect writes into rows that must stay untouched


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    free()


def shapes():
    yield W.TINY, "uniform", 0
    yield W.TINY.with_(B=1, mode=1), "uniform", 1
    yield W.TINY.with_(B=0, mode=1), "uniform", 2
    yield W.TINY.with_(H=72, Hp=40, S=37), "uniform", 3          # ragged H, Hp
    yield W.TINY.with_(R=2, E=4, S=300, K=2, B=2, H=192, Hp=264), "hot", 0   # long segments
    # rows of more than 1,024 16-byte vectors; more routes per token than one batch (K = 12)
    yield W.TINY.with_(name="wide_rows", H=9160, Hp=40, S=20), "uniform", 4
    yield W.TINY.with_(name="many_routes", R=2, E=16, K=12, S=24, B=8, H=264, Hp=72), "uniform", 5
    for t in W.MAXVIO_SWEEP["skewed"]:
        yield W.SKEWED, "zipf", t
    yield W.SKEWED.with_(name="skewed_adv"), "theorem2", 0
    # an expert named twice in one token's row: every slot is routed on its own
    yield W.TINY.with_(name="repeated_ids", K=3), "repeat", 6


def routing(shape, kind, arg):
    if kind == "uniform":
        return W.routing_uniform(shape, salt=arg)
    if kind == "repeat":
        ids, gates = W.routing_uniform(shape, salt=arg)
        ids = ids.copy()
        ids[::3, 1] = ids[::3, 0]                   # every third token repeats its first expert
        return ids, gates
    if kind == "zipf":
        ids, gates, _, _ = W.routing_zipf(shape, arg)
        return ids, gates
    if kind == "hot":
        return W.routing_hot(shape), W.gates_uniform(shape)
    return W.routing_theorem2(shape), W.gates_uniform(shape)


@pytest.mark.parametrize("shape,kind,arg", list(shapes()),
                         ids=lambda v: str(getattr(v, "name", v)))
def test_forward_path(shape, kind, arg):
    announce("forward", shape, kind, arg)
    c, oc = cfgs(shape)
    ids, gates = routing(shape, kind, arg)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    seed = shape.cfg_id * 100 + int(arg * 10)
    x = W.randn_bf16((shape.tokens, shape.H), seed, "cuda")
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), seed + 1, "cuda")
    w_pref = torch.full((max(1, shape.R * shape.B), shape.H, shape.Hp), 0, dtype=torch.int16,
                        device="cuda").fill_(SENT).view(torch.bfloat16)
    xperm = torch.zeros((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((shape.R * shape.SK, shape.Hp), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((shape.tokens, shape.Hp), dtype=torch.bfloat16, device="cuda")
    gates_t = torch.from_numpy(gates).cuda()
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")

    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, 0, shape.R, ws)
    mx.moe_combine(c, plan, y, gates_t, out)
    torch.cuda.synchronize()

    xb, wb = bits(x), bits(w_home)
    # prefetch: bit copy; unused slots untouched
    ref_pref = dataflow.prefetch(wb, ref, oc)
    gp = bits(w_pref)
    for r in range(shape.R):
        for b in range(shape.B):
            if ref.slot_expert[r, b] >= 0:
                assert np.array_equal(gp[r * shape.B + b], ref_pref[r, b])
            else:
                assert np.all(gp[r * shape.B + b] == SENT)
    # dispatch: bit copy
    ref_xp = dataflow.dispatch(xb, ref, oc)
    assert np.array_equal(bits(xperm), ref_xp)
    # grouped GEMM on the oracle's own permuted rows and prefetched weights
    ref_y = dataflow.grouped_gemm(ref_xp, wb, ref_pref, ref, oc)
    rows_close(bits(y), ref_y)
    # combine: end to end, and on the oracle's y (isolates the combine)
    ref_out = dataflow.combine(ref_y, gates, ref, oc)
    rows_close(bits(out), ref_out)
    y_ref_dev = W.from_bits(ref_y, "cuda")
    out2 = torch.zeros_like(out)
    mx.moe_combine(c, plan, y_ref_dev, gates_t, out2)
    torch.cuda.synchronize()
    rows_close(bits(out2), ref_out, tol=1e-2)
    # determinism
    y2 = torch.zeros_like(y)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y2, 0, shape.R, ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_gemm_rank_range_leaves_other_ranks():
    shape = W.SKEWED
    c, oc = cfgs(shape)
    ids, _, _, _ = W.routing_zipf(shape, 10.0)
    ref = make_plan(ids, oc)
    plan, _ = gpu_plan(shape, ids)
    x = W.randn_bf16((shape.tokens, shape.H), 7, "cuda")
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), 8, "cuda")
    w_pref = torch.zeros((shape.R * shape.B, shape.H, shape.Hp), dtype=torch.bfloat16, device="cuda")
    xperm = torch.zeros((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    y = torch.full((shape.R * shape.SK, shape.Hp), 0, dtype=torch.int16,
                   device="cuda").fill_(SENT).view(torch.bfloat16)
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    announce("rank range 3..5")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, 3, 5, ws)
    torch.cuda.synchronize()
    xb, wb = bits(x), bits(w_home)
    ref_xp = dataflow.dispatch(xb, ref, oc)
    ref_y = dataflow.grouped_gemm(ref_xp, wb, dataflow.prefetch(wb, ref, oc), ref, oc, ranks=[3, 4])
    yb = bits(y)
    SK = shape.SK
    rows_close(yb[3 * SK:5 * SK], ref_y[3 * SK:5 * SK])
    assert np.all(yb[:3 * SK] == SENT) and np.all(yb[5 * SK:] == SENT)
    with pytest.raises(mx.MoeError):
        mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, 5, 3, ws)


@pytest.mark.parametrize("shape,kind,arg", [
    (W.TINY.with_(H=64, Hp=48), "uniform", 0),
    (W.TINY.with_(H=72, Hp=40, S=37), "uniform", 1),
    (W.TINY.with_(R=2, E=4, S=300, K=2, B=2, H=136, Hp=264), "hot", 0),
    (W.SKEWED.with_(H=256, Hp=256), "zipf", 10.0),
    (W.SKEWED.with_(H=256, Hp=128, name="skewed_adv"), "theorem2", 0),
    # 12 tiles per item: the per-XCD chunks of the weight gradient start
    # inside items
    (W.SKEWED.with_(H=520, Hp=776, name="skewed_wide"), "zipf", 10.0)],
    ids=lambda v: str(getattr(v, "name", v)))
def test_backward_path(shape, kind, arg):
    announce("backward", shape, kind, arg)
    c, oc = cfgs(shape)
    ids, _ = routing(shape, kind, arg)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    x = W.randn_bf16((shape.tokens, shape.H), 21, "cuda")
    dy = W.randn_bf16((shape.R * shape.SK, shape.Hp), 22, "cuda")
    xperm = torch.zeros((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    gh = torch.full((shape.E, shape.H, shape.Hp), 7.0, dtype=torch.float32, device="cuda")
    gp = torch.full((shape.R * shape.B, shape.H, shape.Hp), -3.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm_wgrad(c, plan, xperm, dy, gh, gp, ws)
    torch.cuda.synchronize()
    ref_xp = dataflow.dispatch(bits(x), ref, oc)
    rh, rp = dataflow.wgrad(ref_xp, bits(dy), ref, oc)
    ghn, gpn = gh.cpu().numpy(), gp.cpu().numpy().reshape(shape.R, shape.B, shape.H, shape.Hp)
    for e in range(shape.E):
        if not rh[e].any():
            assert not ghn[e].any(), e                 # empty home row: zeros
        else:
            rows_close(ghn[e], rh[e])
    for r in range(shape.R):
        for b in range(shape.B):
            if ref.slot_expert[r, b] >= 0:
                rows_close(gpn[r, b], rp[r, b])
            else:
                assert np.all(gpn[r, b] == -3.0)       # untouched

    # reduce_grad on seeded inputs (not on the GPU's wgrad output)
    gen = torch.Generator(device="cuda").manual_seed(5)
    h0 = torch.randn(gh.shape, generator=gen, device="cuda")
    p0 = torch.randn(gp.shape, generator=gen, device="cuda") * 3
    h0n, p0n = h0.cpu().numpy(), p0.cpu().numpy().reshape(shape.R, shape.B, shape.H, shape.Hp)
    mx.moe_reduce_grad(c, plan, h0, p0)
    torch.cuda.synchronize()
    eh, ep = dataflow.reduce_grad(h0n, p0n, ref, oc)
    terms = dataflow.reduce_terms_abs(h0n, p0n, ref, oc)
    got_h = h0.cpu().numpy()
    assert np.all(np.abs(got_h - eh) <= REDUCE_TOL * terms + 1e-30)
    got_p = p0.cpu().numpy().reshape(shape.R, shape.B, shape.H, shape.Hp)
    assert np.array_equal(got_p, ep.astype(np.float32))   # zeros and untouched slots exact


def test_reduce_grad_known_constants():
    shape = W.ADVERSARIAL.with_(S=64, H=16, Hp=24)
    c, oc = cfgs(shape)
    ids = W.routing_theorem2(shape)
    ref = make_plan(ids, oc)
    plan, _ = gpu_plan(shape, ids)
    gh = torch.full((shape.E, shape.H, shape.Hp), 0.5, device="cuda")
    vals = torch.tensor([(r + 1) * 1000.0 + b for r in range(shape.R) for b in range(shape.B)],
                        device="cuda")
    gp = vals[:, None, None].expand(-1, shape.H, shape.Hp).contiguous()
    announce("reduce constants")
    mx.moe_reduce_grad(c, plan, gh, gp)
    torch.cuda.synchronize()
    ghn, gpn = gh.cpu().numpy(), gp.cpu().numpy().reshape(shape.R, shape.B, shape.H, shape.Hp)
    for e in range(shape.E):
        add = sum((r + 1) * 1000 + b for r in range(shape.R) for b in range(shape.B)
                  if ref.slot_expert[r, b] == e)
        assert np.all(ghn[e] == np.float32(0.5 + add))
    for r in range(shape.R):
        for b in range(shape.B):
            want = 0.0 if ref.slot_expert[r, b] >= 0 else (r + 1) * 1000.0 + b
            assert np.all(gpn[r, b] == want)


def test_wgrad_rejects_inference_mode():
    shape = W.TINY.with_(B=1, mode=1)
    c, _ = cfgs(shape)
    plan = mx.Plan(c)
    t = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mx.MoeError):
        mx.moe_grouped_gemm_wgrad(c, plan, torch.zeros(shape.R * shape.SK * shape.H,
                                                       dtype=torch.bfloat16, device="cuda"),
                                  torch.zeros(shape.R * shape.SK * shape.Hp,
                                              dtype=torch.bfloat16, device="cuda"),
                                  torch.zeros(shape.E * shape.H * shape.Hp, device="cuda"),
                                  torch.zeros(shape.R * shape.B * shape.H * shape.Hp, device="cuda"),
                                  torch.zeros(mx.moe_gemm_workspace_size(c), dtype=torch.uint8,
                                              device="cuda"))
    del t


@pytest.mark.parametrize("R,E,S,K,H,Hp,kind", [
    (64, 2048, 64, 8, 16, 8, "theorem2_rev"),  # 2048 slot entries: the receivers' slots
                                               # lie in the second compaction window
    (128, 2048, 32, 8, 72, 40, "theorem2"),   # a row of 360 vectors (not a multiple of 256)
    (32, 1024, 128, 8, 64, 24, "zipf"),
    (8, 64, 64, 4, 8, 8, "hot"),              # one vector per thread at most
])
def test_prefetch_many_slots(R, E, S, K, H, Hp, kind):
    """Every used slot bit-exact and every unused slot untouched, whether a
    few or most slots hold an expert and across several windows of slot
    entries."""
    shape = W.TINY.with_(name="pf", R=R, E=E, S=S, K=K, H=H, Hp=Hp, B=E // R)
    announce("prefetch many slots", shape, kind)
    c, oc = cfgs(shape)
    if kind == "theorem2_rev":
        # Theorem-2 routing with expert ids mirrored: the last rank's experts
        # get no tokens, so the last ranks receive
        ids = shape.E - 1 - W.routing_theorem2(shape)
    else:
        ids, _ = routing(shape, kind, 10.0 if kind == "zipf" else 0)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), 91, "cuda")
    w_pref = torch.full((shape.R * shape.B, shape.H, shape.Hp), SENT, dtype=torch.int16,
                        device="cuda").view(torch.bfloat16)
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    torch.cuda.synchronize()
    ref_pref = dataflow.prefetch(bits(w_home), ref, oc).reshape(shape.R * shape.B, H, Hp)
    used = ref.slot_expert.reshape(-1) >= 0
    gp = bits(w_pref)
    announce("slots used", int(used.sum()), "of", used.size)
    assert used.sum() > 0
    assert np.array_equal(gp[used], ref_pref[used])
    assert np.all(gp[~used] == SENT)


@pytest.mark.parametrize("H,Hp", [(72, 520), (600, 72)])
def test_long_segments_band_order(H, Hp):
    """Segments of 2,600 rows (10 full row tiles and a ragged one: one band of
    8 row tiles and a second band of 3) over several column tiles: the
    forward GEMM (3 column tiles when H'=520) and the data-gradient GEMM (3
    column tiles when H=600), every output row against the oracle, with a
    home segment on rank 0 and a prefetch-slot segment on rank 1."""
    shape = W.TINY.with_(name="band", R=2, E=2, S=2600, K=1, B=1, H=H, Hp=Hp)
    announce("long segments", shape)
    c, oc = cfgs(shape)
    ids = W.routing_hot(shape)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    assert (np.diff(ref.cu_seqlens, axis=1).max(axis=1) > 8 * 256).all()
    x = W.randn_bf16((shape.tokens, H), 41, "cuda")
    w_home = W.randn_bf16((shape.E, H, Hp), 42, "cuda")
    dy = W.randn_bf16((shape.R * shape.SK, Hp), 43, "cuda")
    w_pref = torch.empty((shape.R * shape.B, H, Hp), dtype=torch.bfloat16, device="cuda")
    xperm = torch.empty((shape.R * shape.SK, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((shape.R * shape.SK, Hp), dtype=torch.bfloat16, device="cuda")
    dxp = torch.empty((shape.R * shape.SK, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, 0, shape.R, ws)
    mx.moe_grouped_gemm_dgrad(c, dy, w_home, w_pref, plan.cu_seqlens, dxp, 0, shape.R, ws)
    torch.cuda.synchronize()
    wb = bits(w_home)
    ref_pref = dataflow.prefetch(wb, ref, oc)
    ref_xp = dataflow.dispatch(bits(x), ref, oc)
    assert np.array_equal(bits(xperm), ref_xp)
    rows_close(bits(y), dataflow.grouped_gemm(ref_xp, wb, ref_pref, ref, oc))
    rows_close(bits(dxp), dataflow.dgrad(bits(dy), wb, ref_pref, ref, oc))
