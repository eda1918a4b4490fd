"""Oracle for the two-projection SwiGLU expert (test infrastructure only).

[MoonEP-news] "核心思想": every expert projection is its own contiguous
[E+B, H_in, H_out] weight tensor addressed by row index, cu_seqlens picks
the active rows, and H' is the expert FFN's intermediate size.  The pages
do not name the activation; the reading taken here is the gated SwiGLU FFN
of this model family:

* first projection  W13 [E+B, H, 2H'] -- gate columns [0, H'), up columns
  [H', 2H'), the two side by side in one row-addressed tensor;
* act = silu(gate) * up, silu(z) = z * sigmoid(z), rounded once to bf16;
  gate and up are the exact products (float64 here), not their bf16 copies;
* second projection W2 [E+B, H', H] -- the plain grouped GEMM with the
  projection's own widths (oracle.dataflow.grouped_gemm with H <- H',
  H' <- H).

Training keeps h13 = bf16(x @ W13) for the backward; swiglu_backward works
from those stored bf16 values:
  d up   = d act * silu(gate)
  d gate = d act * up * sigmoid(gate) * (1 + gate * (1 - sigmoid(gate)))
each rounded once to bf16, laid out like h13 ([d gate | d up]).

Pinned by tests/test_oracle_swiglu.py: silu against the tanh form of the
logistic function and its symmetry, the fused GEMM against closed forms with
W13[e] = [c_e I | d_e I] and against a brute-force loop, and the backward
against central finite differences of the forward map.
"""
import numpy as np

from . import bf16
from .dataflow import weight_row


def sigmoid(z):
    """Logistic function 1 / (1 + exp(-z)) in float64 (exp may overflow to inf)."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """silu(z) = z * sigmoid(z)."""
    z = np.asarray(z, np.float64)
    return z * sigmoid(z)


def swiglu_gemm(xperm_bits, w13_home_bits, w13_pref_bits, plan, cfg, ranks=None):
    """First projection fused with the activation, per (rank, weight row) segment.

    ``cfg.Hp`` is the intermediate size H'; W13 rows are [H, 2H'].  For the
    rows of segment j on rank r: h = xperm[rows] @ W13(r, j) in float64,
    act = bf16(silu(h[:, :H']) * h[:, H':]) and h13 = bf16(h).  Returns
    (act [R*S*K, H'], h13 [R*S*K, 2H']) bit arrays; rows of ranks not in
    ``ranks`` stay zero.
    """
    R, SK, E, B, Hp = cfg.R, cfg.SK, cfg.E, cfg.B, cfg.Hp
    act = np.zeros((R * SK, Hp), np.uint16)
    h13 = np.zeros((R * SK, 2 * Hp), np.uint16)
    for r in (range(R) if ranks is None else ranks):
        for j in range(E + B):
            lo, hi = plan.cu_seqlens[r, j], plan.cu_seqlens[r, j + 1]
            if hi == lo:
                continue
            a = bf16.bits_to_f64(xperm_bits[r * SK + lo:r * SK + hi])
            w = bf16.bits_to_f64(weight_row(w13_home_bits, w13_pref_bits, r, j, cfg))
            h = a @ w
            act[r * SK + lo:r * SK + hi] = bf16.f64_to_bits(silu(h[:, :Hp]) * h[:, Hp:])
            h13[r * SK + lo:r * SK + hi] = bf16.f64_to_bits(h)
    return act, h13


def swiglu_gemm_rows(rows, x_bits, w13_home_bits, w13_pref_bits, plan, cfg):
    """``swiglu_gemm`` for selected destination rows only (large shapes).

    Row q = r*S*K + offset holds token route^-1(q) // K of the segment that
    contains the offset.  Returns (act, h13) for those rows.
    """
    SK, Hp = cfg.SK, cfg.Hp
    rows = np.asarray(rows, np.int64)
    inv = np.empty(plan.route.size, np.int64)
    inv[plan.route] = np.arange(plan.route.size)
    seg = np.empty(rows.size, np.int64)
    for idx, q in enumerate(rows):
        r, off = divmod(int(q), SK)
        seg[idx] = np.searchsorted(plan.cu_seqlens[r], off, side="right") - 1
    act = np.zeros((rows.size, Hp), np.uint16)
    h13 = np.zeros((rows.size, 2 * Hp), np.uint16)
    keys = (rows // SK) * (cfg.E + cfg.B) + seg
    for key in np.unique(keys):
        sel = np.nonzero(keys == key)[0]
        r, j = divmod(int(key), cfg.E + cfg.B)
        tok = inv[rows[sel]] // cfg.K
        a = bf16.bits_to_f64(np.asarray(x_bits[tok]))
        w = bf16.bits_to_f64(weight_row(w13_home_bits, w13_pref_bits, r, j, cfg))
        h = a @ w
        act[sel] = bf16.f64_to_bits(silu(h[:, :Hp]) * h[:, Hp:])
        h13[sel] = bf16.f64_to_bits(h)
    return act, h13


def swiglu_backward_f64(gate, up, dact):
    """Gradients of act = silu(gate) * up in float64: (d gate, d up)."""
    gate = np.asarray(gate, np.float64)
    up = np.asarray(up, np.float64)
    dact = np.asarray(dact, np.float64)
    s = sigmoid(gate)
    dup = dact * gate * s
    dgate = dact * up * s * (1.0 + gate * (1.0 - s))
    return dgate, dup


def swiglu_backward(h13_bits, dact_bits):
    """d h13 = [d gate | d up] as bf16 bits from stored h13 and d act.

    h13 is [rows, 2H'] (gate columns first), d act is [rows, H'].
    """
    h = bf16.bits_to_f64(h13_bits)
    Hp = h.shape[-1] // 2
    dgate, dup = swiglu_backward_f64(h[..., :Hp], h[..., Hp:], bf16.bits_to_f64(dact_bits))
    return bf16.f64_to_bits(np.concatenate([dgate, dup], axis=-1))
