"""GPU parity at the full workload sizes, in the launch configuration the
bench times (one grouped-GEMM launch over all ranks), checked on sampled
outputs the oracle computes one by one:

* bench shape (R=8, S=8192, E=384, K=8, H=7168, H'=2048), maxvio 1, with
  both planner policies (the bench runs the largest-first one): plan
  bit-exact; dispatch and prefetch bit-exact on sampled rows/slots; grouped
  GEMM on 4096 sampled rows; combine on sampled tokens;
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
from oracle import bf16, dataflow
from oracle.plan import make_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


def forward_buffers(shape, seed):
    x = W.randn_bf16((shape.tokens, shape.H), seed, "cuda")
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), seed + 1, "cuda", chunk_rows=1)
    w_pref = torch.empty((max(1, shape.R * shape.B), shape.H, shape.Hp), dtype=torch.bfloat16,
                         device="cuda")
    xperm = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((shape.R * shape.SK, shape.Hp), dtype=torch.bfloat16, device="cuda")
    return x, w_home, w_pref, xperm, y


def check_dispatch_sampled(shape, ref, x, xperm, rng, n=8192):
    slots = rng.integers(0, ref.route.size, n)
    dst = torch.as_tensor(ref.route[slots], device="cuda")
    tok = torch.as_tensor(slots // shape.K, device="cuda")
    assert torch.equal(xperm.index_select(0, dst).view(torch.int16),
                       x.index_select(0, tok).view(torch.int16))


def check_prefetch(shape, ref, w_home, w_pref):
    for r in range(shape.R):
        for b in range(shape.B):
            e = int(ref.slot_expert[r, b])
            if e >= 0:
                assert torch.equal(w_pref[r * shape.B + b].view(torch.int16),
                                   w_home[e].view(torch.int16)), (r, b, e)


@pytest.mark.parametrize("policy", [mx.PLAN_ASCENDING, mx.PLAN_LARGEST_FIRST])
def test_bench_shape_forward(policy):
    shape = W.BENCH
    c, oc = cfgs(shape)
    ids, gates, _, mv = W.routing_zipf(shape, 1.0)
    announce("bench forward maxvio", mv, "policy", policy)
    ref = make_plan(ids, oc, policy)
    plan, g = gpu_plan(shape, ids, policy=policy)
    assert_plan_equal(g, ref, shape)
    x, w_home, w_pref, xperm, y = forward_buffers(shape, 31)
    out = torch.empty((shape.tokens, shape.Hp), dtype=torch.bfloat16, device="cuda")
    gates_t = torch.from_numpy(gates).cuda()
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, 0, shape.R, ws)
    mx.moe_combine(c, plan, y, gates_t, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    check_dispatch_sampled(shape, ref, x, xperm, rng)
    check_prefetch(shape, ref, w_home, w_pref)
    segs = sample_segments(ref, shape, rng, per_rank=6)
    rows = sample_rows(ref, shape, segs, rng, total=4096)
    xr, wr = DeviceRows(x), DeviceRows(w_home)
    ref_y = dataflow.gemm_rows(rows, xr, wr, OraclePref(wr, ref), ref, oc)
    got = bits(y.index_select(0, torch.as_tensor(rows, device="cuda")))
    worst = rows_close(got, ref_y)
    announce("bench gemm rows", rows.size, "worst rel err", worst)
    # combine on 128 sampled tokens, from oracle y of their K rows
    toks = np.unique(rng.integers(0, shape.tokens, 128))
    kr = ref.route.reshape(-1, shape.K)[toks].reshape(-1)
    yk = dataflow.gemm_rows(kr, xr, wr, OraclePref(wr, ref), ref, oc)
    acc = np.zeros((toks.size, shape.Hp))
    for k in range(shape.K):
        acc += gates[toks, k:k + 1].astype(np.float64) * bf16.bits_to_f64(yk[k::shape.K])
    ref_out = bf16.f64_to_bits(acc)
    rows_close(bits(out.index_select(0, torch.as_tensor(toks, device="cuda"))), ref_out)


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
    inv = np.empty(ref.route.size, np.int64)
    inv[ref.route] = np.arange(ref.route.size)
    checks = [(0, 0), (0, 5), (1, shape.E + 0), (3, shape.E + 10), (7, shape.E + 0), (4, 4 * 48 + 7),
              (7, 7 * 48 + 47)]
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
        rows = np.arange(r * shape.SK + lo, r * shape.SK + hi)
        toks = inv[rows] // shape.K
        xs = bf16.bits_to_f64(DeviceRows(x)[toks])                  # [len, H]
        ds = bf16.bits_to_f64(DeviceRows(dy)[rows])                 # [len, Hp]
        hs = rng.integers(0, shape.H, 64)
        ref_rows = xs[:, hs].T @ ds                                 # [64, Hp]
        got = out.index_select(0, torch.as_tensor(hs, device="cuda")).cpu().numpy()
        rows_close(got, ref_rows)
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
    check_dispatch_sampled(shape, ref, x, xperm, rng, n=16384)
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
