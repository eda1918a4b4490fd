"""The allocation-free forward GEMM (moe_grouped_gemm_noalloc) against the
workspace entry point (moe_grouped_gemm) it shares its kernels with.

Two calls in a row through the C ABI, the second on a smaller input, each
compared bit for bit with moe_grouped_gemm on the same inputs (same kernels,
same work list, so the outputs must be identical); a rank range; and a work
list beyond the fixed scratch array, rejected on the host before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import announce, cfgs, free, gpu_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


def run_both(shape, ids, rb, re, seed):
    c, _ = cfgs(shape)
    plan, _ = gpu_plan(shape, ids)
    x = W.randn_bf16((shape.tokens, shape.H), seed, "cuda")
    w_home = W.randn_bf16((shape.E, shape.H, shape.Hp), seed + 1, "cuda")
    w_pref = torch.empty((max(1, shape.R * shape.B), shape.H, shape.Hp), dtype=torch.bfloat16,
                         device="cuda")
    xperm = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    mx.moe_prefetch_weight(c, plan, w_home, w_pref)
    mx.moe_dispatch(c, plan, x, xperm)
    sent = torch.full((shape.R * shape.SK, shape.Hp), 0x7E57, dtype=torch.int16, device="cuda")
    y_ws = sent.clone().view(torch.bfloat16)
    y_na = sent.clone().view(torch.bfloat16)
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y_ws, rb, re, ws)
    mx.moe_grouped_gemm_noalloc(c, xperm, w_home, w_pref, plan.cu_seqlens, y_na, rb, re)
    torch.cuda.synchronize()
    return y_ws.view(torch.int16), y_na.view(torch.int16)


def test_noalloc_equals_workspace_gemm_twice_then_smaller():
    big = W.SKEWED.with_(H=264, Hp=136)
    ids, _, _, mv = W.routing_zipf(big, 10.0)
    announce("noalloc first call: skewed maxvio", mv)
    a, b = run_both(big, ids, 0, big.R, 101)
    assert torch.equal(a, b)
    assert not torch.all(b == 0x7E57)
    small = W.TINY
    ids2, _ = W.routing_uniform(small, salt=4)
    announce("noalloc second call: tiny")
    a2, b2 = run_both(small, ids2, 0, small.R, 103)
    assert torch.equal(a2, b2)
    announce("noalloc third call: skewed ranks 2..5")
    a3, b3 = run_both(big, ids, 2, 5, 105)
    assert torch.equal(a3, b3)
    SK = big.SK
    assert torch.all(b3[:2 * SK] == 0x7E57) and torch.all(b3[5 * SK:] == 0x7E57)


def test_noalloc_rejects_work_lists_beyond_its_array():
    lib = mx.load()
    # R' * (ceil(S*K/256) + E + B) * 24 + 256 bytes > MOE_NOALLOC_SCRATCH_BYTES:
    # rejected before any pointer is looked at (null pointers stay unused)
    c = mx.make_cfg(1024, 16, 2048, 2, 128, 64, 2)
    assert lib.moe_grouped_gemm_noalloc(ctypes.byref(c), None, None, None, None, None, 0, 1024,
                                        None) == mx.MOE_ELIMIT
    # the same configuration over few enough ranks fits, then needs pointers
    assert lib.moe_grouped_gemm_noalloc(ctypes.byref(c), None, None, None, None, None, 0, 8,
                                        None) == mx.MOE_EINVAL
