"""GPU parity of the dedup route encoding and the two-phase dispatch it
drives: route_enc bit-exact with the oracle; the deduplicated dispatch
bit-exact with the oracle's dispatch (small shapes, full buffers); at the
bench shape, sampled tokens' encodings and sampled rows against the oracle's
sampled forms, and the whole 7.5 GB buffer equal to the plain dispatch's
(compared on the device)."""
import numpy as np
import pytest
import torch

import moe_expert_load_amd as mx
import workloads as W
from gpu_helpers import DeviceRows, announce, assert_plan_equal, bits, cfgs, free, gpu_plan
from oracle import dataflow
from oracle.plan import make_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    free()
    yield
    free()


CASES = [(W.TINY, "uniform"), (W.TINY, "hot"), (W.TINY.with_(B=1, mode=1), "uniform"),
         (W.TINY.with_(R=2, E=8, K=3, S=10, B=4), "uniform"), (W.SKEWED, "zipf"),
         (W.SKEWED.with_(name="skewed_adv"), "theorem2"),
         (W.TINY.with_(name="repeated_ids", K=3), "repeat")]


def ids_of(shape, kind):
    if kind == "hot":
        return W.routing_hot(shape)
    if kind == "theorem2":
        return W.routing_theorem2(shape)
    if kind == "zipf":
        return W.routing_zipf(shape, 10.0)[0]
    if kind == "repeat":                            # an expert named twice in a row
        ids = W.routing_uniform(shape, salt=2)[0].copy()
        ids[::3, 1] = ids[::3, 0]
        return ids
    return W.routing_uniform(shape, salt=2)[0]


@pytest.mark.parametrize("shape,kind", CASES, ids=lambda v: str(getattr(v, "name", v)))
def test_route_encode_and_dedup_dispatch(shape, kind):
    announce("dedup", shape, kind)
    c, oc = cfgs(shape)
    ids = ids_of(shape, kind)
    ref = make_plan(ids, oc)
    plan, _ = gpu_plan(shape, ids)
    enc = torch.empty(shape.tokens * shape.K, dtype=torch.int32, device="cuda")
    mx.moe_route_encode(c, plan, enc)
    x = W.randn_bf16((shape.tokens, shape.H), 81, "cuda")
    xp = torch.zeros((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    mx.moe_dispatch_dedup(c, enc, x, xp)
    torch.cuda.synchronize()
    ref_enc = dataflow.route_encode(ref, oc)
    assert np.array_equal(enc.cpu().numpy(), ref_enc)
    assert np.array_equal(bits(xp), dataflow.dispatch(bits(x), ref, oc))


def test_route_encode_without_plan_marks_no_destination():
    shape = W.TINY
    c, oc = cfgs(shape)
    ids = W.routing_uniform(shape, salt=0)[0].copy()
    ids[3, 1] = shape.E + 5                        # out of range: no plan, route -1
    plan, g = gpu_plan(shape, ids)
    assert int(g["status"][2]) & mx.STATUS_BAD_ID
    enc = torch.zeros(shape.tokens * shape.K, dtype=torch.int32, device="cuda")
    mx.moe_route_encode(c, plan, enc)
    torch.cuda.synchronize()
    assert torch.all(enc == -(2 ** 31))


def test_bench_shape_dedup_dispatch_equals_plain():
    shape = W.BENCH
    c, oc = cfgs(shape)
    ids, _, _, mv = W.routing_zipf(shape, 1.0)
    announce("bench dedup dispatch maxvio", mv)
    ref = make_plan(ids, oc)
    plan, g = gpu_plan(shape, ids)
    assert_plan_equal(g, ref, shape)
    enc = torch.empty(shape.tokens * shape.K, dtype=torch.int32, device="cuda")
    mx.moe_route_encode(c, plan, enc)
    x = W.randn_bf16((shape.tokens, shape.H), 91, "cuda")
    a = torch.empty((shape.R * shape.SK, shape.H), dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    mx.moe_dispatch(c, plan, x, a)
    mx.moe_dispatch_dedup(c, enc, x, b)
    torch.cuda.synchronize()
    # the whole 7.5 GB buffer equals the plain dispatch's, compared on the device
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    rng = np.random.default_rng(5)
    # sampled tokens' encodings against the oracle's, on the oracle's plan
    toks = np.unique(rng.integers(0, shape.tokens, 4096))
    got = enc.view(-1, shape.K).index_select(0, torch.as_tensor(toks, device="cuda"))
    assert np.array_equal(got.cpu().numpy().astype(np.int64),
                          dataflow.route_encode_tokens(toks, ref, oc))
    # sampled rows of the two-phase dispatch against the oracle's dispatch
    rows = np.unique(rng.integers(0, shape.R * shape.SK, 8192))
    assert np.array_equal(bits(b.index_select(0, torch.as_tensor(rows, device="cuda"))),
                          dataflow.dispatch_rows(rows, DeviceRows(x), ref, oc))
