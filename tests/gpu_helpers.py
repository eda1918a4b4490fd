"""Shared helpers of the GPU parity tests (no tests here).

Inputs come from ``workloads`` (seeded); expected values come only from
``oracle``; the HIP path is reached only through the C-ABI binding.
"""
import sys

import numpy as np
import torch

import moe_expert_load_amd as mx
import workloads as W
from oracle import bf16
from oracle.plan import Cfg, make_plan

GEMM_TOL = 2e-2       # per output row: max|gpu - ref| / max|ref|
REDUCE_TOL = 1e-5     # per element: |gpu - ref| <= tol * sum |terms|


def announce(*msg):
    print("[gpu-case]", *msg, file=sys.stderr, flush=True)


def cfgs(shape):
    c = mx.make_cfg(shape.R, shape.S, shape.E, shape.K, shape.H, shape.Hp, shape.B, shape.mode)
    o = Cfg(shape.R, shape.S, shape.E, shape.K, shape.H, shape.Hp, shape.B, shape.mode)
    return c, o


def gpu_plan(shape, ids_np, plan=None, policy=0):
    c, _ = cfgs(shape)
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    if plan is None:
        plan = mx.Plan(c)
    if policy:
        mx.moe_plan_run_policy(c, ids, plan, policy)
    else:
        mx.moe_plan_run(c, ids, plan)
    torch.cuda.synchronize()
    return plan, {k: v.cpu().numpy() for k, v in plan.views().items()}


def assert_plan_equal(g, ref, shape):
    """Bit-exact comparison of every plan output with the oracle."""
    nm = len(ref.moves)
    assert int(g["status"][2]) == ref.status, (g["status"], ref.status)
    assert int(g["status"][0]) == len(ref.fills)
    assert int(g["status"][1]) == nm
    assert np.array_equal(g["counts"], ref.counts)
    assert np.array_equal(g["load0"], ref.load0)
    assert np.array_equal(g["n_redundant"], ref.n_redundant)
    assert np.array_equal(g["src_rank"], ref.src_rank)
    assert np.array_equal(g["slot_expert"], ref.slot_expert)
    assert np.array_equal(g["cu_seqlens"], ref.cu_seqlens)
    assert np.array_equal(g["moves"][:nm], ref.moves)
    assert np.array_equal(g["route"], ref.route)


def bits(t):
    return W.bf16_bits(t)


def rows_close(gpu_bits, ref_bits, tol=GEMM_TOL):
    g = bf16.bits_to_f64(gpu_bits) if gpu_bits.dtype == np.uint16 else np.asarray(gpu_bits, np.float64)
    r = bf16.bits_to_f64(ref_bits) if ref_bits.dtype == np.uint16 else np.asarray(ref_bits, np.float64)
    g = g.reshape(g.shape[0], -1)
    r = r.reshape(r.shape[0], -1)
    err = np.abs(g - r).max(axis=1)
    scale = np.abs(r).max(axis=1)
    bad = err > tol * np.maximum(scale, 1e-30)
    assert not bad.any(), "rows %s: err %s scale %s" % (
        np.nonzero(bad)[0][:8], err[bad][:8], scale[bad][:8])
    return float((err / np.maximum(scale, 1e-30)).max(initial=0.0))


class DeviceRows:
    """Index a GPU bf16 tensor by rows and get host bf16 bits (lazy copy)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, idx):
        if isinstance(idx, tuple):
            return bits(self.t[idx])
        if np.isscalar(idx) or isinstance(idx, (int, np.integer)):
            return bits(self.t[int(idx)])
        idx = torch.as_tensor(np.asarray(idx, np.int64), device=self.t.device)
        return bits(self.t.index_select(0, idx))


class OraclePref:
    """The oracle's prefetch result, w_pref[r, b] = w_home[slot_expert[r, b]]."""

    def __init__(self, w_home_rows, plan):
        self.w = w_home_rows
        self.plan = plan

    def __getitem__(self, rb):
        r, b = rb
        e = int(self.plan.slot_expert[r, b])
        assert e >= 0
        return self.w[e]


def sample_segments(plan, shape, rng, per_rank=6):
    """(r, j) of a few non-empty segments per rank: first, last, largest,
    smallest and up to two prefetch rows, then random others."""
    out = []
    E = shape.E
    for r in range(shape.R):
        lens = plan.seg_len[r]
        nz = np.nonzero(lens)[0]
        if nz.size == 0:
            continue
        pick = {int(nz[0]), int(nz[-1]), int(nz[np.argmax(lens[nz])]), int(nz[np.argmin(lens[nz])])}
        slots = [j for j in nz if j >= E]
        for j in slots[:2]:
            pick.add(int(j))
        rest = [int(j) for j in nz if int(j) not in pick]
        rng.shuffle(rest)
        for j in rest[:max(0, per_rank - len(pick))]:
            pick.add(j)
        out += [(r, j) for j in sorted(pick)]
    return out


def sample_rows(plan, shape, segs, rng, total=4096):
    """First and last row of each listed segment plus seeded rows inside them."""
    SK = shape.SK
    rows = []
    for r, j in segs:
        lo, hi = plan.cu_seqlens[r, j], plan.cu_seqlens[r, j + 1]
        rows += [r * SK + lo, r * SK + hi - 1]
    extra = max(0, total - len(rows))
    for k in range(extra):
        r, j = segs[rng.integers(len(segs))]
        lo, hi = plan.cu_seqlens[r, j], plan.cu_seqlens[r, j + 1]
        rows.append(r * SK + int(rng.integers(lo, hi)))
    return np.unique(np.array(rows, np.int64))


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


__all__ = ["announce", "cfgs", "gpu_plan", "assert_plan_equal", "rows_close", "DeviceRows",
           "OraclePref", "sample_segments", "sample_rows", "free", "make_plan", "bits"]
