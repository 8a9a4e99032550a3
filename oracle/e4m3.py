"""OCP FP8 E4M3FN codec, written from the format definition (test infrastructure only).

The pages say only that the cache is kept in FP8 (ithome page, cost-analysis
paragraph; dpshk page, FAQ on KV-cache size).  Reading: OCP E4M3FN -- 1 sign
bit, 4 exponent bits with bias 7, 3 mantissa bits; no infinities; the single
NaN pattern per sign is S.1111.111; largest finite magnitude 448; smallest
normal 2**-6; subnormals (m/8) * 2**-6 down to 2**-9.

Encoding rounds to nearest with ties to the even mantissa over the whole range
(subnormals included), saturates every magnitude >= 448 to 448 and never emits
NaN.  A value whose magnitude rounds to zero is encoded as +0 (code 0x00), so
that the sign of an accumulated zero never decides a stored byte.
"""

import numpy as np

MAX_FINITE = 448.0
MAX_CODE = 0x7E          # 0.1111.110 -> 448


def decode_table():
    """All 256 codes -> float64 (NaN for 0x7F and 0xFF), from the definition."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if (c >> 7) else 1.0
        E = (c >> 3) & 0xF
        M = c & 0x7
        if E == 0xF and M == 0x7:
            out[c] = np.nan
        elif E == 0:
            out[c] = s * (M / 8.0) * 2.0 ** -6
        else:
            out[c] = s * (1.0 + M / 8.0) * 2.0 ** (E - 7)
    return out


_TABLE = decode_table()


def decode(codes):
    """uint8 codes -> float64 values (exact)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_rne(x):
    """float values -> uint8 E4M3FN codes (RNE, saturating, zero -> 0x00).

    With e = max(floor(log2|x|), -6), the representable magnitudes near |x| are
    the multiples of 2**(e-3); q = rint(|x| / 2**(e-3)) is the rounded count of
    those steps (8 <= q <= 16 for normals, 0 <= q <= 8 below 2**-6) and the
    magnitude code is ((e + 7) << 3) + q - 8, where q = 16 carries into the
    exponent field and the subnormal range falls out with e = -6.  Codes above
    0x7E (448) saturate.  All arithmetic is exact in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("e4m3 encode: NaN input")
    ax = np.abs(x)
    inf = np.isinf(ax)
    ax = np.where(inf, 2.0 * MAX_FINITE, ax)     # any magnitude past 448 saturates
    _, E = np.frexp(ax)
    e = np.maximum(E - 1, -6)
    q = np.rint(ax / np.ldexp(1.0, e - 3))
    mag = ((e + 7) << 3) + q.astype(np.int64) - 8
    mag = np.minimum(mag, MAX_CODE)
    mag = np.where(ax == 0.0, 0, mag)
    sign = np.where((x < 0) & (mag != 0), 0x80, 0)
    return (mag + sign).astype(np.uint8)
