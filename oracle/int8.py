"""Symmetric INT8 storage for the KV cache, written out from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name an INT8 KV cache beside the fp8 one, with the same 2x saving
in capacity and a small loss in quality ([P3] "M.65 Inference Serving": the
three primitives beyond PagedAttention, item (c) on quantisation; and the
failure mode of ignoring quantisation, item (d) on quantising the KV cache).
They give no format.  Readings taken here, the plainest the rest supports:

* A stored element is a signed 8-bit integer code c in [-127, 127] (two's
  complement byte; -128 is never written), and it reads back as c * scale.
* Scaling follows the fp8 cache: one fp32 scale per (layer, kv head),
  separate for K and for V.
* Quantisation: c = round-half-to-even(fp32(x / scale)), clamped to
  [-127, 127].  The division is one correctly rounded fp32 operation, so the
  oracle and the device take the rounding decision on the same fp32 value.
"""

from __future__ import annotations

import numpy as np

MAX_CODE = 127


def quantise(x) -> np.ndarray:
    """Round values (already divided by the scale; no NaN) to int8 codes:
    nearest integer, ties to even, clamped to +-127."""
    r = np.rint(np.asarray(x, dtype=np.float64))  # numpy's rint rounds half to even
    return np.clip(r, -MAX_CODE, MAX_CODE).astype(np.int8)


def quantise_scaled(x, scale) -> np.ndarray:
    """Codes for values ``x`` stored with fp32 ``scale`` (broadcast on x)."""
    xs = np.asarray(x, dtype=np.float32) / np.asarray(scale, dtype=np.float32)
    return quantise(xs.astype(np.float32))


def dequantise(codes, scale) -> np.ndarray:
    """float64 values of stored codes: code * scale."""
    return np.asarray(codes, dtype=np.int8).astype(np.float64) * np.asarray(scale, dtype=np.float64)
