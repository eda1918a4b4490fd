"""GPU parity at the full workload sizes, in the launch configuration the
bench times (one grouped-GEMM launch over all ranks), checked on sampled
outputs the oracle computes one by one (its sampled forms, each pinned to
the full form on small shapes):

* bench shape (R=8, S=8192, E=384, K=8, H=7168, H'=2048), at every maxvio
  of the sweep (0.2 / 1 / 10 / 20, one shared seed) with both planner
  policies: plan bit-exact; dispatch and prefetch bit-exact on sampled
  rows/slots; grouped GEMM on 4096 sampled rows; combine on sampled tokens
  of a generated y; at maxvio 1 also combine end to end (the oracle's own y
  rows of the tokens' routes);
* bench shape, zipf maxvio 1: weight gradients of sampled home and prefetch
  segments on sampled h rows;
* Theorem-2 worst case in inference mode (B=4, overflow rows read from home
  rows): sampled GEMM rows of overflow segments;
* Theorem-2 worst case in train mode: weight gradients on sampled elements
  (home rows, empty home rows, prefetch rows), reduce_grad on seeded inputs;
* Large-E shape (R=64, E=896, K=16): plan + dispatch for all 64 ranks, GEMM
  of one rank's [65536, 7168] buffer against its [910, 7168, 2048] view.
"""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import (REDUCE_TOL, DeviceRows, OraclePref, announce, assert_plan_equal, bits,
                         cfgs, free, gpu_plan, rows_close, sample_rows, sample_segments)
from oracle import dataflow
from oracle.plan import make_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


_BENCH_INPUTS = {}


def bench_inputs():
    """x, w_home and a generated y at the bench shape, made once per module."""
    if not _BENCH_INPUTS:
        s = W.BENCH
        _BENCH_INPUTS["x"] = W.randn_bf16((s.tokens, s.H), 31, "cuda")
        _BENCH_INPUTS["w_home"] = W.randn_bf16((s.E, s.H, s.Hp), 32, "cuda", chunk_rows=1)
        _BENCH_INPUTS["y"] = W.randn_bf16((s.R * s.SK, s.Hp), 33, "cuda")
        _BENCH_INPUTS["dy"] = W.randn_bf16((s.R * s.SK, s.Hp), 34, "cuda")
    return _BENCH_INPUTS


def forward_buffers(shape, seed):
    x = W.randn_bf16((shape.tokens, shape.H), seed, "cuda")
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), seed + 1, "cuda", chunk_rows=1)
    w_pref = torch.empty((max(1, shape.R * shape.B), shape.H, shape.Hp), dtype=torch.bfloat16,
                         device="cuda")
    xperm = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((shape.R * shape.SK, shape.Hp), dtype=torch.bfloat16, device="cuda")
    return x, w_home, w_pref, xperm, y


def check_dispatch_sampled(shape, oc, ref, x, xperm, rng, n=8192):
    rows = np.unique(rng.integers(0, shape.R * shape.SK, n))
    want = dataflow.dispatch_rows(rows, DeviceRows(x), ref, oc)
    got = bits(xperm.index_select(0, torch.as_tensor(rows, device="cuda")))
    assert np.array_equal(got, want)


def check_prefetch(shape, ref, w_home, w_pref):
    for r in range(shape.R):
        for b in range(shape.B):
            e = int(ref.slot_expert[r, b])
            if e >= 0:
                assert torch.equal(w_pref[r * shape.B + b].view(torch.int16),
                                   w_home[e].view(torch.int16)), (r, b, e)


@pytest.mark.parametrize("policy", [mx.PLAN_ASCENDING, mx.PLAN_LARGEST_FIRST],
                         ids=["ascending", "largest_first"])
@pytest.mark.parametrize("target", W.MAXVIO_SWEEP["bench"])
def test_bench_shape_forward(target, policy):
    shape = W.BENCH
    c, oc = cfgs(shape)
    ids, gates, _, mv = W.routing_zipf(shape, target)
    announce("bench forward maxvio", target, mv, "policy", policy)
    ref = make_plan(ids, oc, policy)
    plan, g = gpu_plan(shape, ids, policy=policy)
    assert_plan_equal(g, ref, shape)
    inp = bench_inputs()
    x, w_home, y_gen = inp["x"], inp["w_home"], inp["y"]
    w_pref = torch.empty((shape.R * shape.B, shape.H, shape.Hp), dtype=torch.bfloat16,
                         device="cuda")
    xperm = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((shape.R * shape.SK, shape.Hp), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((shape.tokens, shape.Hp), dtype=torch.bfloat16, device="cuda")
    out_gen = torch.empty_like(out)
    gates_t = torch.from_numpy(gates).cuda()
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, 0, shape.R, ws)
    mx.moe_combine(c, plan, y, gates_t, out)
    mx.moe_combine(c, plan, y_gen, gates_t, out_gen)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    check_dispatch_sampled(shape, oc, ref, x, xperm, rng)
    check_prefetch(shape, ref, w_home, w_pref)
    segs = sample_segments(ref, shape, rng, per_rank=6)
    rows = sample_rows(ref, shape, segs, rng, total=4096)
    xr, wr = DeviceRows(x), DeviceRows(w_home)
    ref_y = dataflow.gemm_rows(rows, xr, wr, OraclePref(wr, ref), ref, oc)
    got = bits(y.index_select(0, torch.as_tensor(rows, device="cuda")))
    worst = rows_close(got, ref_y)
    announce("bench gemm rows", rows.size, "worst rel err", worst)
    # combine of a generated y on 1024 sampled tokens
    toks = np.unique(rng.integers(0, shape.tokens, 1024))
    tt = torch.as_tensor(toks, device="cuda")
    rows_close(bits(out_gen.index_select(0, tt)),
               dataflow.combine_tokens(toks, DeviceRows(y_gen), gates, ref, oc))
    if target == 1.0:
        # end to end on 128 tokens: the oracle's y rows of their K routes
        toks = np.unique(rng.integers(0, shape.tokens, 128))
        kr = ref.route.reshape(-1, shape.K)[toks].reshape(-1)
        yk = dataflow.gemm_rows(kr, xr, wr, OraclePref(wr, ref), ref, oc)

        class _YRows:                    # the oracle's y, addressed by row number
            pos = {int(q): i for i, q in enumerate(kr)}

            def __getitem__(self, qs):
                return yk[[self.pos[int(q)] for q in np.atleast_1d(qs)]]

        rows_close(bits(out.index_select(0, torch.as_tensor(toks, device="cuda"))),
                   dataflow.combine_tokens(toks, _YRows(), gates, ref, oc))


def test_bench_shape_wgrad_zipf():
    """Weight gradients at the bench shape on the step's own routing (zipf
    maxvio 1, the ascending planner): sampled home and prefetch segments,
    64 sampled h rows each, against the oracle's sampled form."""
    shape = W.BENCH
    c, oc = cfgs(shape)
    ids, _, _, mv = W.routing_zipf(shape, 1.0)
    announce("bench wgrad zipf maxvio", mv)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    inp = bench_inputs()
    x, dy = inp["x"], inp["dy"]
    xperm = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    gh = torch.full((shape.E, shape.H, shape.Hp), 9.0, device="cuda")
    gp = torch.full((shape.R * shape.B, shape.H, shape.Hp), -9.0, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm_wgrad(c, plan, xperm, dy, gh, gp, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    checks = []
    for r in range(shape.R):
        home = [j for j in range(r * shape.n, (r + 1) * shape.n)]
        lens = [ref.seg_len[r, j] for j in home]
        checks += [(r, home[int(np.argmax(lens))]), (r, home[int(np.argmin(lens))]),
                   (r, int(rng.choice(home)))]
        for b in range(shape.B):
            if ref.slot_expert[r, b] >= 0:
                checks.append((r, shape.E + b))
    xr, dr = DeviceRows(x), DeviceRows(dy)
    worst = 0.0
    for r, j in checks:
        hs = np.unique(np.concatenate([[0, shape.H - 1], rng.integers(0, shape.H, 62)]))
        want = dataflow.wgrad_entries(r, j, hs, xr, dr, ref, oc)
        outt = gh[j] if j < shape.E else gp[r * shape.B + j - shape.E]
        got = outt.index_select(0, torch.as_tensor(hs, device="cuda")).cpu().numpy()
        if not want.any():
            assert not got.any(), (r, j)
            continue
        worst = max(worst, rows_close(got, want))
    announce("bench wgrad segments", len(checks), "worst rel err", worst)
    # slots that hold no expert are not written
    unused = torch.as_tensor(ref.slot_expert.reshape(-1) < 0, device="cuda")
    assert torch.all(gp[unused] == -9.0)


def test_adversarial_inference_overflow():
    shape = W.ADVERSARIAL_INFER
    c, oc = cfgs(shape)
    ids = W.routing_theorem2(shape)
    ref = make_plan(ids, oc)
    announce("adversarial infer B=4")
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    x, w_home, w_pref, xperm, y = forward_buffers(shape, 41)
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, 0, shape.R, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    check_prefetch(shape, ref, w_home, w_pref)
    # overflow segments: rows j < E on ranks that do not own j
    segs = []
    for r in range(shape.R):
        for j in np.nonzero(ref.seg_len[r])[0]:
            if j < shape.E and j // shape.n != r:
                segs.append((r, int(j)))
    assert len(segs) > 0
    rng.shuffle(segs)
    segs = segs[:24] + [(0, shape.E), (0, shape.E + 3), (1, shape.E + 1)]
    rows = sample_rows(ref, shape, segs, rng, total=2048)
    xr, wr = DeviceRows(x), DeviceRows(w_home)
    ref_y = dataflow.gemm_rows(rows, xr, wr, OraclePref(wr, ref), ref, oc)
    rows_close(bits(y.index_select(0, torch.as_tensor(rows, device="cuda"))), ref_y)


def test_adversarial_backward():
    shape = W.ADVERSARIAL
    c, oc = cfgs(shape)
    ids = W.routing_theorem2(shape)
    ref = make_plan(ids, oc)
    announce("adversarial backward")
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    x = W.randn_bf16((shape.tokens, shape.H), 51, "cuda")
    dy = W.randn_bf16((shape.R * shape.SK, shape.Hp), 52, "cuda")
    xperm = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    gh = torch.full((shape.E, shape.H, shape.Hp), 9.0, device="cuda")
    gp = torch.full((shape.R * shape.B, shape.H, shape.Hp), -9.0, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm_wgrad(c, plan, xperm, dy, gh, gp, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    checks = [(0, 0), (0, 5), (1, shape.E + 0), (3, shape.E + 10), (7, shape.E + 0), (4, 4 * 48 + 7),
              (7, 7 * 48 + 47)]
    xr, dr = DeviceRows(x), DeviceRows(dy)
    for r, j in checks:
        lo, hi = ref.cu_seqlens[r, j], ref.cu_seqlens[r, j + 1]
        if j < shape.E:
            out = gh[j]
        else:
            out = gp[r * shape.B + j - shape.E]
        if hi == lo:
            if j < shape.E:
                assert not out.any(), (r, j)
            else:
                assert torch.all(out == -9.0), (r, j)
            continue
        hs = rng.integers(0, shape.H, 64)
        want = dataflow.wgrad_entries(r, j, hs, xr, dr, ref, oc)    # [64, Hp]
        got = out.index_select(0, torch.as_tensor(hs, device="cuda")).cpu().numpy()
        rows_close(got, want)
    # every home row of rank 0 is empty in this routing and must be zero
    assert not gh[:shape.n].any()
    # reduce_grad on seeded gradients; sampled elements against the oracle
    gen = torch.Generator(device="cuda").manual_seed(9)
    gh.normal_(generator=gen)
    gp.normal_(generator=gen)
    idx = torch.as_tensor(rng.integers(0, shape.H * shape.Hp, 4096), device="cuda")
    h_before = gh.view(shape.E, -1).index_select(1, idx).cpu().numpy()
    p_before = gp.view(shape.R * shape.B, -1).index_select(1, idx).cpu().numpy()
    mx.moe_reduce_grad(c, plan, gh, gp)
    torch.cuda.synchronize()
    h_after = gh.view(shape.E, -1).index_select(1, idx).cpu().numpy()
    p_after = gp.view(shape.R * shape.B, -1).index_select(1, idx).cpu().numpy()
    pb = p_before.reshape(shape.R, shape.B, -1)
    eh, ep = dataflow.reduce_grad(h_before, pb, ref, oc)
    terms = dataflow.reduce_terms_abs(h_before, pb, ref, oc)
    assert np.all(np.abs(h_after - eh) <= REDUCE_TOL * terms + 1e-30)
    assert np.array_equal(p_after.reshape(shape.R, shape.B, -1), ep.astype(np.float32))
    consumed = torch.as_tensor((ref.slot_expert.reshape(-1) >= 0), device="cuda")
    assert not gp[consumed].any()


def test_large_e_plan_dispatch_and_one_rank_gemm():
    shape = W.LARGE_E
    c, oc = cfgs(shape)
    ids, _, _, mv = W.routing_zipf(shape, 10.0)
    announce("large_e maxvio", mv)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    x = W.randn_bf16((shape.tokens, shape.H), 61, "cuda")
    xperm = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    mx.moe_dispatch(c, plan, x, xperm)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    check_dispatch_sampled(shape, oc, ref, x, xperm, rng, n=16384)
    # the rank with the most active segments (ties: lowest id)
    active = (ref.seg_len > 0).sum(axis=1)
    r = int(np.argmax(active))
    announce("large_e one-rank gemm rank", r, "active segments", int(active[r]))
    need = sorted({j for j in np.nonzero(ref.seg_len[r])[0] if j < shape.E} |
                  {int(e) for e in ref.slot_expert[r] if e >= 0})
    w_home = torch.zeros((shape.E, shape.H, shape.Hp), dtype=torch.bfloat16, device="cuda")
    for e in need:                       # only experts this rank touches get values
        w_home[e] = W.randn_bf16((shape.H, shape.Hp), 1000 + e, "cuda")
    w_pref = torch.empty((shape.R * shape.B, shape.H, shape.Hp), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((shape.R * shape.SK, shape.Hp), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, r, r + 1, ws)
    torch.cuda.synchronize()
    segs = [(r, int(j)) for j in np.nonzero(ref.seg_len[r])[0]]
    rows = sample_rows(ref, shape, segs, rng, total=4096)
    xr, wr = DeviceRows(x), DeviceRows(w_home)
    ref_y = dataflow.gemm_rows(rows, xr, wr, OraclePref(wr, ref), ref, oc)
    rows_close(bits(y.index_select(0, torch.as_tensor(rows, device="cuda"))), ref_y)
