"""OCP E4M3FN 8-bit float codec — oracle side (test infrastructure only).

The pages store the latent KV cache "in FP8, e4m3" instead of BF16, halving
its size ("Smaller, faster, safer: running Kimi and GLM at scale", section
"Quantizing the KV cache").  They do not name the e4m3 variant; the reading
taken here is the OCP 8-bit floating point E4M3FN encoding (native on gfx950):

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 encodes subnormals ``±2^-6 * m/8``;
* otherwise ``±2^(e-7) * (1 + m/8)``;
* ``S.1111.111`` is NaN; there are no infinities; the largest finite value is 448.

Encoding is round-to-nearest, ties to the even code (mantissa LSB 0),
saturating to ±448; NaN encodes to ``0x7F`` with the input's sign; the sign of
a result that rounds to zero is kept.
"""

from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0


def decode_value(code: int) -> float:
    """Closed form of one code (float64; NaN for the two NaN codes)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def decode_table() -> np.ndarray:
    """float64[256]: the value of every code."""
    return np.array([decode_value(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()
# codes 0x00..0x7E hold the finite non-negative values in increasing order
_POS = _TABLE[:0x7F].copy()
_MID = (_POS[:-1] + _POS[1:]) / 2.0  # exact in float64


def decode(codes: np.ndarray) -> np.ndarray:
    """Codes (uint8 array) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint8 codes: nearest finite E4M3FN value, ties to even,
    saturating at ±448, NaN -> 0x7F|sign."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    sign = ((bits >> np.uint32(31)).astype(np.uint8)) << np.uint8(7)
    a = np.abs(x.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, MAX_FINITE))
    # hi = index of the first finite value >= a; lo = hi - 1
    hi = np.searchsorted(_POS, a, side="left")
    hi = np.minimum(hi, _POS.size - 1)
    lo = np.maximum(hi - 1, 0)
    exact = _POS[hi] == a
    mid = _MID[lo]
    above = a > mid
    tie = a == mid
    pick = np.where(above, hi, lo)
    # ties go to the code with even mantissa: of lo and hi exactly one is even
    pick = np.where(tie, np.where((lo & 1) == 0, lo, hi), pick)
    pick = np.where(exact, hi, pick)
    code = pick.astype(np.uint8) | sign
    code = np.where(nan, np.uint8(0x7F) | sign, code)
    return code.astype(np.uint8)
