"""Seeded synthetic workloads shared by the tests, the bench and smoke().

This module holds input generators only -- no step of the method (no
planning, permuting, GEMM or combine).  Both the HIP path and the CPU oracle
consume what it produces; neither is imported here.

Shapes follow the workloads the pages describe: the MoonEP comparison setup
(S=8192 tokens per rank, E=384, H=7168, K=8, H'=2048, EP=8, maxvio swept over
0.2 / 1 / 10 / 20 with one shared seed), the K3 Large-E shape (E=896, K=16,
R=64), a tiny shape for brute-force optima, and the Theorem-2 worst case.

Routing recipes:

* ``uniform``  -- logits ~ U(0, 1) per (token, expert); top-K.
* ``zipf``     -- logits = N(0, 1) + b_e with b_e = -s * ln(1 + pi(e)), pi a
  seeded permutation of the experts; s is found by bisection so that the
  resulting maxvio is within 2 % of the target.  The noise, the permutation
  and every other stream are the same for every target (shared seed).
* ``theorem2`` -- slot i = t*K + k goes to expert n + (i mod (E - n)),
  n = E/R: rank 0's experts get nothing and the other E(R-1)/R experts share
  all R*S*K slots as equally as integers allow (remainder to the lowest ids).
* ``hot``      -- every token picks experts 0..K-1 (maximum skew).

Gates are the softmax of the K selected logits (fp32), or 1/K where stated.
x, W, dy are N(0, 1) rounded to bf16, drawn with torch generators so that
multi-GB tensors can be made on the device.
"""
from dataclasses import dataclass, replace
import zlib

import numpy as np
import torch


@dataclass(frozen=True)
class Shape:
    name: str
    R: int
    S: int
    E: int
    K: int
    H: int
    Hp: int
    B: int
    mode: int = 0          # 0 = train (B = E/R), 1 = inference (B < E/R allowed)
    cfg_id: int = 0

    @property
    def n(self):
        return self.E // self.R

    @property
    def SK(self):
        return self.S * self.K

    @property
    def tokens(self):
        return self.R * self.S

    def with_(self, **kw):
        return replace(self, **kw)


TINY = Shape("tiny", R=4, S=16, E=8, K=2, H=128, Hp=64, B=2, cfg_id=1)
SKEWED = Shape("skewed", R=8, S=1024, E=64, K=4, H=1024, Hp=512, B=8, cfg_id=2)
BENCH = Shape("bench", R=8, S=8192, E=384, K=8, H=7168, Hp=2048, B=48, cfg_id=3)
LARGE_E = Shape("large_e", R=64, S=4096, E=896, K=16, H=7168, Hp=2048, B=14,
                cfg_id=4)
ADVERSARIAL = Shape("adversarial", R=8, S=8192, E=384, K=8, H=7168, Hp=2048,
                    B=48, cfg_id=5)
ADVERSARIAL_INFER = ADVERSARIAL.with_(name="adversarial_infer", B=4, mode=1)

SHAPES = {s.name: s for s in (TINY, SKEWED, BENCH, LARGE_E, ADVERSARIAL,
                              ADVERSARIAL_INFER)}

MAXVIO_SWEEP = {
    "skewed": (0.2, 1.0, 10.0, 15.0),   # 20 exceeds E/K - 1 = 15: run 15
    "bench": (0.2, 1.0, 10.0, 20.0),
    "large_e": (1.0, 10.0),
}


def rng(shape, stream, salt=0):
    """numpy Generator for one named stream of one workload."""
    key = zlib.crc32(stream.encode())
    return np.random.default_rng(np.random.SeedSequence([0, shape.cfg_id, key, salt]))


def torch_seed(shape, stream, salt=0):
    key = zlib.crc32(stream.encode())
    return (shape.cfg_id * 1_000_003 + key * 7919 + salt) % (2 ** 62)


def _topk(logits, K):
    t = torch.from_numpy(logits)
    vals, idx = torch.topk(t, K, dim=1, largest=True, sorted=True)
    return idx.numpy().astype(np.int32), vals.numpy().astype(np.float64)


def _softmax_rows(v):
    v = v - v.max(axis=1, keepdims=True)
    e = np.exp(v)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def _maxvio_of(ids, shape):
    c = np.bincount(ids.reshape(-1), minlength=shape.E)
    return c.max() / (shape.R * shape.S * shape.K / shape.E) - 1.0


def routing_uniform(shape, salt=0):
    """Uniform random logits -> top-K ids [R*S, K] int32 and softmax gates."""
    g = rng(shape, "logits_uniform", salt)
    logits = g.random((shape.tokens, shape.E), dtype=np.float32)
    ids, vals = _topk(logits, shape.K)
    return ids, _softmax_rows(vals)


class ZipfRouter:
    """Gaussian noise plus a Zipf-shaped per-expert bias, tuned for maxvio."""

    def __init__(self, shape, salt=0):
        self.shape = shape
        g = rng(shape, "logits_noise", salt)
        self.noise = g.standard_normal((shape.tokens, shape.E), dtype=np.float32)
        perm = rng(shape, "expert_perm", salt).permutation(shape.E)
        self.logw = np.log1p(perm.astype(np.float64))

    def route(self, s):
        bias = (-s * self.logw).astype(np.float32)
        logits = self.noise + bias[None, :]
        ids, vals = _topk(logits, self.shape.K)
        return ids, vals

    def for_target(self, target, rel_tol=0.02, iters=60):
        """Bisection on s until |maxvio - target| <= rel_tol * target."""
        tol = rel_tol * target

        def at(s):
            ids, vals = self.route(s)
            return ids, vals, _maxvio_of(ids, self.shape)

        ids, vals, mv = at(0.0)
        if abs(mv - target) <= tol:
            return ids, _softmax_rows(vals), 0.0, mv
        if mv > target:
            raise ValueError("noise alone exceeds target maxvio %.3f" % mv)
        lo, hi = 0.0, 1.0
        while True:
            ids, vals, mv = at(hi)
            if abs(mv - target) <= tol:
                return ids, _softmax_rows(vals), hi, mv
            if mv > target:
                break
            if hi > 1e4:
                raise ValueError("maxvio %.3f unreachable (max %.3f)" % (target, mv))
            lo, hi = hi, hi * 2
        for _ in range(iters):
            mid = 0.5 * (lo + hi)
            ids, vals, mv = at(mid)
            if abs(mv - target) <= tol:
                return ids, _softmax_rows(vals), mid, mv
            if mv < target:
                lo = mid
            else:
                hi = mid
        raise ValueError("could not reach maxvio %.3f (got %.3f)" % (target, mv))


_ZIPF_CACHE = {}


def routing_zipf(shape, target, salt=0):
    """(ids, gates, s, maxvio) for one point of the shared-seed maxvio sweep."""
    key = (shape.name, shape.R, shape.S, shape.E, shape.K, salt)
    router = _ZIPF_CACHE.get(key)
    if router is None:
        _ZIPF_CACHE.clear()
        router = ZipfRouter(shape, salt)
        _ZIPF_CACHE[key] = router
    return router.for_target(target)


def routing_theorem2(shape):
    """Theorem-2 worst case: rank 0's experts idle, the rest share all slots."""
    n = shape.n
    i = np.arange(shape.tokens * shape.K, dtype=np.int64)
    ids = (n + i % (shape.E - n)).astype(np.int32).reshape(shape.tokens, shape.K)
    return ids


def routing_hot(shape):
    """Every token picks experts 0..K-1."""
    return np.tile(np.arange(shape.K, dtype=np.int32), (shape.tokens, 1))


def gates_uniform(shape):
    return np.full((shape.tokens, shape.K), 1.0 / shape.K, dtype=np.float32)


def randn_bf16(shape_tuple, seed, device="cpu", chunk_rows=None):
    """N(0, 1) rounded to bf16 (torch's round-to-nearest-even cast).

    Drawn in float32 in chunks along dim 0 (each chunk from its own seeded
    generator) so multi-GB tensors need little temporary memory and any
    chunk can be regenerated alone.
    """
    out = torch.empty(shape_tuple, dtype=torch.bfloat16, device=device)
    rows = shape_tuple[0]
    per = int(np.prod(shape_tuple[1:])) if len(shape_tuple) > 1 else 1
    if chunk_rows is None:
        chunk_rows = max(1, (1 << 24) // max(per, 1))
    gen = torch.Generator(device=device)
    for c0 in range(0, rows, chunk_rows):
        c1 = min(rows, c0 + chunk_rows)
        gen.manual_seed((int(seed) * 65537 + c0) % (2 ** 62))
        tmp = torch.randn((c1 - c0,) + tuple(shape_tuple[1:]), generator=gen,
                          device=device, dtype=torch.float32)
        out[c0:c1].copy_(tmp)
        del tmp
    return out


def bf16_bits(t):
    """torch bf16 tensor -> numpy uint16 bit array (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(bits, device="cpu"):
    """numpy uint16 bit array -> torch bf16 tensor."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
