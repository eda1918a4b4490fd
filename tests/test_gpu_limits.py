"""Parity at the size limit of the GEMMs' 32-bit buffer offsets.

The grouped GEMMs address one rank's permuted rows with 32-bit byte offsets,
which the header guards with S*K*max(H, H')*2 < 2^32.  Here one rank holds
131,072 rows of H = 16,000 (4,194,304,000 bytes, 97.7 % of 2^32) in two
segments of 65,536 rows (E = 2, K = 2: every token goes to both experts),
with a ragged H' = 264.  Checked against the oracle on sampled outputs:
dispatch rows bit-exact; forward GEMM rows and data-gradient rows within
2e-2 per row (first and last row of each segment plus seeded rows, and the
last rows of the buffer); weight-gradient rows G[h, :] for seeded h
(including the last) within 2e-2, each the float64 sum over all 65,536 rows
of its segment, from the generated x and dy.  2,048 more tokens per rank
exceed the guard, which the host check rejects with MOE_ELIMIT.
"""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import (DeviceRows, announce, assert_plan_equal, bits, cfgs, free, gpu_plan,
                         rows_close)
from oracle import dataflow
from oracle.plan import make_plan

pytestmark = pytest.mark.gpu

SHAPE = W.TINY.with_(name="offset_limit", R=1, S=65536, E=2, K=2, H=16000, Hp=264, B=2,
                     cfg_id=7)


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


def test_gemms_at_the_offset_limit():
    s = SHAPE
    assert 0.97 * 2 ** 32 < s.S * s.K * s.H * 2 < 2 ** 32
    c, oc = cfgs(s)
    big = mx.make_cfg(s.R, s.S + 2048, s.E, s.K, s.H, s.Hp, s.B, s.mode)
    with pytest.raises(mx.MoeError) as ei:
        mx.moe_plan_sizes(big)
    assert ei.value.code == mx.MOE_ELIMIT
    ids, gates = W.routing_uniform(s)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(s, ids)
    assert_plan_equal(g, ref, s)
    announce("offset limit: dispatch + forward")
    rows = s.R * s.SK
    bf = dict(dtype=torch.bfloat16, device="cuda")
    x = W.randn_bf16((s.tokens, s.H), 71, "cuda")
    w = W.randn_bf16((s.E, s.H, s.Hp), 72, "cuda")
    wp = torch.zeros((s.R * s.B, s.H, s.Hp), **bf)
    xp = torch.empty((rows, s.H), **bf)
    y = torch.empty((rows, s.Hp), **bf)
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w, wp)
    mx.moe_dispatch(c, plan, x, xp)
    mx.moe_grouped_gemm(c, xp, w, wp, plan.cu_seqlens, y, 0, s.R, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    cu = ref.cu_seqlens[0]
    segs = [(int(cu[j]), int(cu[j + 1])) for j in range(s.E + s.B) if cu[j + 1] > cu[j]]
    sample = {rows - 1, rows - 2}
    for lo, hi in segs:
        sample |= {lo, hi - 1}
        sample |= set(int(v) for v in rng.integers(lo, hi, 200))
    sample = np.array(sorted(sample), np.int64)
    idx = torch.as_tensor(sample, device="cuda")
    xr = DeviceRows(x)
    assert np.array_equal(bits(xp.index_select(0, idx)),
                          dataflow.dispatch_rows(sample, xr, ref, oc))
    wr = DeviceRows(w)
    rows_close(bits(y.index_select(0, idx)),
               dataflow.gemm_rows(sample, xr, wr, None, ref, oc))
    del y

    announce("offset limit: data gradient")
    dy = W.randn_bf16((rows, s.Hp), 73, "cuda")
    dxp = torch.empty((rows, s.H), **bf)
    mx.moe_grouped_gemm_dgrad(c, dy, w, wp, plan.cu_seqlens, dxp, 0, s.R, ws)
    torch.cuda.synchronize()
    ref_dx = dataflow.dgrad_rows(sample, DeviceRows(dy), wr, None, ref, oc)
    rows_close(bits(dxp.index_select(0, idx)), ref_dx)
    del dxp

    announce("offset limit: weight gradient")
    gh = torch.full((s.E, s.H, s.Hp), 3.0, dtype=torch.float32, device="cuda")
    gp = torch.full((s.R * s.B, s.H, s.Hp), 3.0, dtype=torch.float32, device="cuda")
    mx.moe_grouped_gemm_wgrad(c, plan, xp, dy, gh, gp, ws)
    torch.cuda.synchronize()
    hs = np.unique(np.concatenate([[0, s.H - 1], rng.integers(0, s.H, 30)]))
    hcols = torch.as_tensor(hs, device="cuda")
    # the sampled h columns of x, as an input of the oracle's sampled form
    xcols = DeviceRows(x.index_select(1, hcols).contiguous())
    for j in range(s.E):                       # R = 1: both experts are home rows
        want = dataflow.wgrad_entries(0, j, np.arange(hs.size), xcols, DeviceRows(dy), ref, oc)
        got = gh[j].index_select(0, hcols).cpu().numpy()
        rows_close(got, want)


@pytest.mark.parametrize("hp", [1398104, 1 << 21])
def test_wgrad_rejects_gradient_tiles_beyond_2gib(hp):
    """The weight gradient stores a 384-row fp32 tile through one buffer
    window of 2 GiB, so 384 H' 4 bytes must stay below 2^31 (H' <= 1398101);
    beyond, the host check returns MOE_ELIMIT before any launch."""
    c = mx.make_cfg(1, 4, 2, 1, 8, hp, 2, mx.MODE_TRAIN)
    plan = mx.Plan(c)
    xperm = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    dy = torch.zeros((4, hp), dtype=torch.bfloat16, device="cuda")
    gh = torch.empty((2, 8, hp), dtype=torch.float32, device="cuda")
    gp = torch.empty((2, 8, hp), dtype=torch.float32, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MoeError) as ei:
        mx.moe_grouped_gemm_wgrad(c, plan, xperm, dy, gh, gp, ws)
    assert ei.value.code == mx.MOE_ELIMIT


def test_wgrad_at_the_2gib_tile_window():
    """The largest H' the weight gradient takes (1,398,096, a multiple of 8
    at or below 1,398,101): a full 384-row tile then spans 384 H' 4 =
    2,147,475,456 bytes of its store window, 8 KB short of 2^31, and H = 400
    leaves a second, 16-row tile.  Sampled gradient rows (both tiles, their
    first and last rows) of both experts against the oracle's sampled form,
    within 2e-2 per row."""
    hp = 1398096
    assert 384 * hp * 4 < 2 ** 31 <= 384 * (hp + 8) * 4
    s = W.TINY.with_(name="wgrad_window", R=1, S=32, E=2, K=1, H=400, Hp=hp, B=2, cfg_id=8)
    c, oc = cfgs(s)
    ids, _ = W.routing_uniform(s)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(s, ids)
    assert_plan_equal(g, ref, s)
    announce("weight gradient at the 2 GiB tile window", s)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    rows = s.R * s.SK
    x = W.randn_bf16((s.tokens, s.H), 81, "cuda")
    dy = W.randn_bf16((rows, s.Hp), 82, "cuda")
    xp = torch.empty((rows, s.H), **bf)
    gh = torch.full((s.E, s.H, s.Hp), 3.0, dtype=torch.float32, device="cuda")
    gp = torch.full((s.R * s.B, s.H, s.Hp), 3.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_dispatch(c, plan, x, xp)
    mx.moe_grouped_gemm_wgrad(c, plan, xp, dy, gh, gp, ws)
    torch.cuda.synchronize()
    hs = np.array([0, 1, 200, 382, 383, 384, 390, 399], np.int64)
    hcols = torch.as_tensor(hs, device="cuda")
    xcols = DeviceRows(x.index_select(1, hcols).contiguous())
    for j in range(s.E):                       # R = 1: both experts are home rows
        want = dataflow.wgrad_entries(0, j, np.arange(hs.size), xcols, DeviceRows(dy), ref, oc)
        got = gh[j].index_select(0, hcols).cpu().numpy()
        rows_close(got, want)
    # one rank: no prefetch slot, so the prefetch gradients stay as they were
    assert bool((gp[:, ::97, ::4099] == 3.0).all())
