"""GPU parity of the forward-type GEMM schedules: tile-height classes.

The forward, data-gradient and SwiGLU GEMMs split each step's row tiles into
classes by rows (a segment's last row tile of at most 64 rows: class 1, of
65..128 rows: class 2, otherwise class 4), run each class as its own launch
whose tiles multiply only the row blocks they need, and fold small classes
into larger ones when a cost model says that is cheaper.  Whatever the
classes and folds, every output row must equal the oracle's:

* hand-made segment layouts (the GEMMs take cu_seqlens as input) with last
  tiles of 1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200 and 255 rows,
  full tiles before them, and empty segments, on a configuration whose
  average segment is short enough for the class-2 and class-1 launches to
  run; every row of y, dxperm, act and h13 against the oracle;
* the bench's expert shape at decode size (R=8, S=256, E=384, K=8, H=7168,
  H'=2048: about 42 rows per segment), planned by moe_plan_run, in the
  launch configuration the bench uses: 4096 sampled rows of the forward and
  the data gradient;
* a layout with both short and long segments given twice with the segments
  in another order: the outputs of every segment must not change.
"""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import (DeviceRows, OraclePref, announce, assert_plan_equal, bits, cfgs, free,
                         gpu_plan, rows_close, sample_rows, sample_segments)
from oracle import dataflow, swiglu
from oracle.plan import Cfg, make_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


class Layout:
    """cu_seqlens of hand-made segments (all the oracle's GEMMs read)."""

    def __init__(self, lens):
        self.seg_len = np.asarray(lens, np.int64)
        self.cu_seqlens = np.concatenate([np.zeros((lens.shape[0], 1), np.int64),
                                          np.cumsum(self.seg_len, axis=1)], axis=1)


TAILS = [1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200, 255]


def hand_layout(R, E, rng):
    """Per rank: segments with 0..2 full row tiles plus each tail size, some
    empty segments, shuffled over the E rows."""
    lens = np.zeros((R, E), np.int64)
    for r in range(R):
        segs = [256 * int(rng.integers(0, 3)) + t for t in TAILS] + [256, 512, 0, 0]
        rng.shuffle(segs)
        lens[r, :len(segs)] = segs
    return lens


@pytest.mark.parametrize("H,Hp", [(136, 72), (264, 520)])
def test_every_tile_class_forward_dgrad_swiglu(H, Hp):
    R, E = 2, 32
    rng = np.random.default_rng(H)
    lens = hand_layout(R, E, rng)
    SK = int(lens.sum(axis=1).max())
    lens[:, -1] += SK - lens.sum(axis=1)          # pad every rank to S*K rows
    lay = Layout(lens)
    # S*K*R / E stays well below the small-class gate (512 rows per segment)
    c = mx.make_cfg(R, SK, E, 1, H, Hp, 0, mx.MODE_INFER)
    oc = Cfg(R, SK, E, 1, H, Hp, 0, 1)
    announce("tile classes H", H, "Hp", Hp, "SK", SK)
    cu = torch.as_tensor(lay.cu_seqlens.astype(np.int32), device="cuda")
    xperm = W.randn_bf16((R * SK, H), 201, "cuda")
    dy = W.randn_bf16((R * SK, Hp), 202, "cuda")
    w = W.randn_bf16((E, H, Hp), 203, "cuda")
    w13 = W.randn_bf16((E, H, 2 * Hp), 204, "cuda")
    y = torch.empty((R * SK, Hp), dtype=torch.bfloat16, device="cuda")
    dxp = torch.empty((R * SK, H), dtype=torch.bfloat16, device="cuda")
    act = torch.empty((R * SK, Hp), dtype=torch.bfloat16, device="cuda")
    h13 = torch.empty((R * SK, 2 * Hp), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_grouped_gemm(c, xperm, w, None, cu, y, 0, R, ws)
    mx.moe_grouped_gemm_dgrad(c, dy, w, None, cu, dxp, 0, R, ws)
    mx.moe_grouped_gemm_swiglu(c, xperm, w13, None, cu, act, h13, 0, R, ws)
    torch.cuda.synchronize()
    xb, wb, db = bits(xperm), bits(w), bits(dy)
    empty = np.zeros((R, 0, H, Hp), np.uint16)
    rows_close(bits(y), dataflow.grouped_gemm(xb, wb, empty, lay, oc))
    rows_close(bits(dxp), dataflow.dgrad(db, wb, empty, lay, oc))
    ra, rh = swiglu.swiglu_gemm(xb, bits(w13), np.zeros((R, 0, H, 2 * Hp), np.uint16), lay, oc)
    rows_close(bits(act), ra)
    rows_close(bits(h13), rh)


def test_segment_order_does_not_change_results():
    R, E, H, Hp = 1, 32, 264, 136
    rng = np.random.default_rng(7)
    lens = hand_layout(R, E, rng)
    SK = int(lens.sum())
    c = mx.make_cfg(R, SK, E, 1, H, Hp, 0, mx.MODE_INFER)
    announce("segment order, SK", SK)
    w = W.randn_bf16((E, H, Hp), 211, "cuda")
    xperm = W.randn_bf16((SK, H), 212, "cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    outs = []
    perm = rng.permutation(E)
    for order in (np.arange(E), perm):
        l2 = lens[:, order]
        cu_np = np.concatenate([[0], np.cumsum(l2[0])])
        # the same rows and weights, placed in the new segment order
        src = np.concatenate([np.arange(np.cumsum(lens[0])[e] - lens[0, e], np.cumsum(lens[0])[e])
                              for e in order]).astype(np.int64)
        xp = xperm.index_select(0, torch.as_tensor(src, device="cuda"))
        wp = w.index_select(0, torch.as_tensor(order, device="cuda")).contiguous()
        y = torch.empty((SK, Hp), dtype=torch.bfloat16, device="cuda")
        mx.moe_grouped_gemm(c, xp, wp, None, torch.as_tensor(cu_np.astype(np.int32),
                                                              device="cuda"), y, 0, 1, ws)
        torch.cuda.synchronize()
        back = torch.empty_like(y)
        back[torch.as_tensor(src, device="cuda")] = y
        outs.append(back)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_decode_size_bench_experts():
    shape = W.BENCH.with_(name="decode256", S=256)
    c, oc = cfgs(shape)
    ids, _, _, mv = W.routing_zipf(shape, 1.0)
    announce("decode-size forward and data gradient, maxvio", mv)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    x = W.randn_bf16((shape.tokens, shape.H), 221, "cuda")
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), 222, "cuda", chunk_rows=1)
    dy = W.randn_bf16((shape.R * shape.SK, shape.Hp), 223, "cuda")
    w_pref = torch.empty((shape.R * shape.B, shape.H, shape.Hp), dtype=torch.bfloat16,
                         device="cuda")
    xperm = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((shape.R * shape.SK, shape.Hp), dtype=torch.bfloat16, device="cuda")
    dxp = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_dispatch(c, plan, x, xperm)
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y, 0, shape.R, ws)
    mx.moe_grouped_gemm_dgrad(c, dy, w_home, w_pref, plan.cu_seqlens, dxp, 0, shape.R, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    segs = sample_segments(ref, shape, rng, per_rank=12)
    rows = sample_rows(ref, shape, segs, rng, total=4096)
    xr, wr = DeviceRows(x), DeviceRows(w_home)
    idx = torch.as_tensor(rows, device="cuda")
    worst = rows_close(bits(y.index_select(0, idx)),
                       dataflow.gemm_rows(rows, xr, wr, OraclePref(wr, ref), ref, oc))
    rows_close(bits(dxp.index_select(0, idx)),
               dataflow.dgrad_rows(rows, DeviceRows(dy), wr, OraclePref(wr, ref), ref, oc))
    announce("decode-size rows", rows.size, "worst rel err", worst)
