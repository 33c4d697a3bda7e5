"""softmax(q K^T / sqrt(d)) V in float64, for decode and for a causal chunk.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method reaches exactly (up to rounding order) the plain attention result:
paging changes where K/V live, not the result ([P2] "PagedAttention -
operating-system virtual memory, applied to attention": outputs are identical),
and the tiled online softmax with a running max and normaliser is a
reformulation of one softmax over the whole row ([P1] "FlashAttention: why the
mechanism this whole layer runs on isn't compute-bound").  So this module
writes out that plain definition and nothing else: no tiling, no running max,
no split over the keys.

Readings where the pages are silent:

* Score scale 1/sqrt(d).
* Grouped-query heads: query head h reads kv head h // G with G = Hq / Hkv
  (each kv head repeated G times in a row, the repeat_interleave named in
  [P1] "Kernel engineering: the layer underneath everything else here").
* Decode: the query attends to every cached token 0..L-1 (its own K/V is
  written before attention runs).
* Chunked prefill ([P1] "Serving systems: the layer that survives real
  traffic"; [P3] "prefill vs decode phase separation", item (e)): a chunk of C
  queries is the last C of L cached tokens, so query i sits at absolute
  position L - C + i and attends keys 0..L-C+i (causal, aligned at the bottom
  right).  A chunk of C = 1 is a decode step.

Shapes: q [Hq, d] (decode) or [C, Hq, d] (chunk); K, V [L, Hkv, d].  All inputs
are converted to float64 first.
"""

from __future__ import annotations

import numpy as np


def _group(hq: int, hkv: int) -> int:
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    return hq // hkv


def decode(q, K, V) -> np.ndarray:
    """One query per head over L cached tokens.  Returns [Hq, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    hq, d = q.shape
    L, hkv, _ = K.shape
    if L == 0:
        raise ValueError("decode needs at least one cached token")
    g = _group(hq, hkv)
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        j = h // g
        s = K[:, j, :] @ q[h] / np.sqrt(d)
        w = np.exp(s - s.max())
        out[h] = (w @ V[:, j, :]) / w.sum()
    return out


def prefill_chunk(q, K, V) -> np.ndarray:
    """C queries, the last C of L tokens, causal.  Returns [C, Hq, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    C, hq, d = q.shape
    L, hkv, _ = K.shape
    if C > L:
        raise ValueError("chunk longer than the cached sequence")
    g = _group(hq, hkv)
    P = L - C
    out = np.empty((C, hq, d), dtype=np.float64)
    for h in range(hq):
        j = h // g
        S = q[:, h, :] @ K[:, j, :].T / np.sqrt(d)  # [C, L]
        for i in range(C):
            row = S[i, : P + i + 1]
            w = np.exp(row - row.max())
            out[i, h] = (w @ V[: P + i + 1, j, :]) / w.sum()
    return out


def decode_rows(q, K, V, heads) -> np.ndarray:
    """``decode`` restricted to the listed query heads (for sampled checks)."""
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    hkv = np.asarray(K).shape[1]
    g = _group(hq, hkv)
    d = q.shape[1]
    out = np.empty((len(heads), d), dtype=np.float64)
    for n, h in enumerate(heads):
        j = h // g
        Kj = np.asarray(K[:, j, :], dtype=np.float64)
        Vj = np.asarray(V[:, j, :], dtype=np.float64)
        s = Kj @ q[h] / np.sqrt(d)
        w = np.exp(s - s.max())
        out[n] = (w @ Vj) / w.sum()
    return out


def prefill_rows(q, K, V, rows) -> np.ndarray:
    """Chosen queries of a chunk: q [C, Hq, d] are the last C of the L tokens in
    K, V [L, Hkv, d]; for each query index i in ``rows`` (attending keys
    0..L-C+i, as in ``prefill_chunk``) returns [len(rows), Hq, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    C, hq, d = q.shape
    L = np.asarray(K).shape[0]
    if C > L:
        raise ValueError("chunk longer than the cached sequence")
    out = np.empty((len(rows), hq, d), dtype=np.float64)
    for n, i in enumerate(rows):
        last = L - C + int(i) + 1
        out[n] = decode(q[int(i)], np.asarray(K[:last]), np.asarray(V[:last]))
    return out
