"""bfloat16 storage for the oracle (test infrastructure only).

bfloat16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent bits,
7 stored mantissa bits.  Decoding is exact into float64; encoding rounds the
float64 value to the nearest bfloat16, ties to the even mantissa (the reading
taken for every bf16 rounding in the path, since the pages fix none).
"""

import numpy as np


def decode(bits):
    """uint16 bfloat16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def encode_rne(x):
    """float64 values -> uint16 bfloat16 bit patterns, round to nearest even.

    Written from the format: with |x| = f * 2**e (1 <= f < 2, e clamped at the
    smallest normal exponent -126), the representable neighbours are multiples
    of 2**(e-7); numpy.rint rounds half to even, and every step is exact in
    float64.  Finite inputs only (the path never produces others).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 encode: non-finite input")
    ax = np.abs(x)
    _, E = np.frexp(ax)                     # ax = m * 2**E, 0.5 <= m < 1
    e = np.maximum(E - 1, -126)             # floor(log2 ax), clamped to the normal range
    ulp = np.ldexp(1.0, e - 7)
    q = np.rint(ax / ulp) * ulp             # rounded magnitude, exact in float64
    q = np.where(ax == 0.0, 0.0, q)
    v = np.copysign(q, x).astype(np.float32)   # exactly representable in binary32
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
