"""bfloat16 helpers for the oracle (test infrastructure only).

bf16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits,
7 stored significand bits (8 bits of precision), same exponent range as
binary32.  Rounding is to nearest, ties to even.  The pages fix bf16 as the
payload type of activations and weights ([K3-blog] "在线规划、零拷贝、静态
shape": a token vector is about 7 KB in BF16); the rounding mode is the IEEE
default.

Pinned by tests/test_oracle_bf16.py against torch's CPU float32->bfloat16
cast (a library routine) on float32 inputs, and against hand-picked ties.
"""
import numpy as np

_BF16_MAX_EXP = 127          # largest unbiased exponent of a finite bf16
_BF16_MIN_NORMAL_EXP = -126  # smallest unbiased exponent of a normal bf16
_BF16_PREC = 8               # bits of precision (1 implicit + 7 stored)


def bits_to_f64(bits):
    """Raw bf16 bits (uint16 array) -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bits(v):
    """float64 -> bf16 bits, round to nearest, ties to even (single rounding).

    For |v| in [2^e, 2^(e+1)) a bf16 normal has quantum 2^(e-7); below the
    smallest normal 2^-126 the quantum stays 2^-133 (gradual underflow).
    ``np.rint`` rounds half to even, which is exactly the IEEE tie rule on
    the integer count of quanta.  Magnitudes that round to 2^128 or above
    overflow to infinity.
    """
    v0 = np.asarray(v, dtype=np.float64)
    v = v0.reshape(-1)
    out = np.zeros(v.shape, dtype=np.uint16)
    sign = np.signbit(v).astype(np.uint16) << np.uint16(15)
    a = np.abs(v)
    nan = np.isnan(v)
    finite = np.isfinite(v)
    nz = finite & (a > 0)
    if np.any(nz):
        an = a[nz]
        _, ex = np.frexp(an)                      # an = m * 2^ex, m in [0.5, 1)
        e_unb = ex - 1                            # an in [2^e_unb, 2^(e_unb+1))
        qexp = np.maximum(e_unb, _BF16_MIN_NORMAL_EXP) - (_BF16_PREC - 1)
        count = np.rint(np.ldexp(an, -qexp))      # whole quanta, ties to even
        rounded = np.ldexp(count, qexp)
        mag = np.zeros(an.shape, dtype=np.uint16)
        over = rounded >= 2.0 ** (_BF16_MAX_EXP + 1)
        mag[over] = 0x7F80
        ok = ~over
        # rounded has at most 8 significant bits and quantum >= 2^-133, so it
        # is exactly representable in binary32 and its low 16 bits are zero.
        b32 = rounded[ok].astype(np.float32).view(np.uint32)
        mag[ok] = (b32 >> np.uint32(16)).astype(np.uint16)
        out[nz] = mag
    inf = np.isinf(v)
    out[inf] = 0x7F80
    out = out | sign
    out[nan] = 0x7FC0
    return out.reshape(v0.shape)


def round_f64(v):
    """Round float64 values to the nearest bf16 value (returned as float64)."""
    return bits_to_f64(f64_to_bits(v))
