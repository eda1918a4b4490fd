"""Pins for oracle.bf16 against a library routine and hand-worked ties."""
import numpy as np
import torch

from oracle import bf16


def _torch_bits(x32):
    t = torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_matches_torch_cast_on_float32():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(200_000).astype(np.float32),
        (g.standard_normal(50_000) * 1e30).astype(np.float32),
        (g.standard_normal(50_000) * 1e-38).astype(np.float32),   # subnormals
        g.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    assert np.array_equal(bf16.f64_to_bits(x.astype(np.float64)), _torch_bits(x))


def test_ties_to_even():
    one = 1.0
    q = 2.0 ** -7                       # bf16 spacing just above 1
    cases = {
        one + q / 2: 0x3F80,            # halfway 1 .. 1+q -> even (1)
        one + 3 * q / 2: 0x3F82,        # halfway 1+q .. 1+2q -> even (1+2q)
        one + q / 2 + 2 ** -30: 0x3F81, # just above halfway -> up
        -(one + q / 2): 0xBF80,
        2.0 ** -133 / 2: 0x0000,        # half the smallest subnormal -> 0 (even)
        3 * 2.0 ** -134: 0x0002,        # 1.5 subnormal quanta -> 2 (even)
        (2 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,  # halfway above max -> inf
        (2 - 2.0 ** -7) * 2.0 ** 127: 0x7F7F,  # max finite
    }
    for v, want in cases.items():
        assert int(bf16.f64_to_bits(np.float64(v))) == want, (v, want)


def test_single_rounding_from_float64():
    # 1 + q/2 + 2^-40 lies above the tie in float64 but collapses onto the
    # tie if first rounded to float32; the oracle must round once (up).
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert int(bf16.f64_to_bits(np.float64(v))) == 0x3F81


def test_bits_roundtrip_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.bits_to_f64(bits)
    keep = ~np.isnan(vals)
    assert np.array_equal(bf16.f64_to_bits(vals[keep]), bits[keep])
    assert np.all(bf16.f64_to_bits(vals[~keep]) == 0x7FC0)
