"""OCP E4M3 (fp8) written out from the format definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix what the fp8 cache is: one byte per element instead of two, an
exact 2x in capacity ([P2] "Quantising the cache"), in the E4M3 layout of four
exponent and three mantissa bits ([P3] anti-patterns, quantisation item (b)).
They do not say which E4M3 variant, how values are rounded or how they are
scaled.  Readings taken here:

* Variant: OCP E4M3 ("FN"): sign, 4-bit exponent with bias 7, 3-bit mantissa;
  exponent 0 encodes subnormals m/8 * 2^-6; no infinities; only S.1111.111 is
  NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
* Quantisation: the finite code nearest to the value, ties to the code with an
  even mantissa, magnitudes at or above 448 saturate to +-448, and the sign is
  kept (a negative value that rounds to zero gives code 0x80).
* Scaling: one fp32 scale per (layer, kv head), separate for K and for V.  The
  stored code is quantise(fp32(x / scale)) - the division is one correctly
  rounded fp32 operation, so both this oracle and the device take the rounding
  decision on the same fp32 value - and the stored value reads back as
  decode(code) * scale.
"""

from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0


def decode_code(code: int) -> float:
    """Value of one E4M3 byte, from sign / exponent / mantissa fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Decoded value of every code, index = code.
TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# Non-negative finite magnitudes, codes 0x00..0x7E; they increase with the code.
_POS = TABLE[:0x7F].copy()


def decode(codes) -> np.ndarray:
    """Element-wise decode of a uint8 array to float64."""
    return TABLE[np.asarray(codes, dtype=np.uint8)]


def quantise(x) -> np.ndarray:
    """Round float values (no NaN) to E4M3 codes: nearest, ties to even, saturate."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # hi = first magnitude >= a; lo = the one below it.
    hi = np.searchsorted(_POS, a, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= MAX_FINITE, 0x7E, code)
    sign = np.signbit(x)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantise_scaled(x, scale) -> np.ndarray:
    """Codes for values ``x`` stored with fp32 ``scale`` (broadcast on x)."""
    xs = np.asarray(x, dtype=np.float32) / np.asarray(scale, dtype=np.float32)
    return quantise(xs.astype(np.float32))


def dequantise(codes, scale) -> np.ndarray:
    """float64 values of stored codes: decode(code) * scale."""
    return decode(codes) * np.asarray(scale, dtype=np.float64)
