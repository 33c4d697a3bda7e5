"""Seeded synthetic inputs shared by the oracle side and the HIP side of tests
and of the benchmark.

This module holds no arithmetic of the method (no attention, no allocator, no
quantisation): it only draws lengths, block placements, query/key/value values
and the script of pool operations that builds each workload.  Both sides replay
the same script through their own allocator and write the same values through
their own slots.

Workloads (shapes from the configurations the benchmarks are quoted on):

* ``tiny``          4 sequences of 300 / 2000 / 600 / 4400 cached tokens (the
                    contiguous-allocation example of [P2] "PagedAttention -
                    operating-system virtual memory, applied to attention"),
                    8 query / 2 kv heads, d = 128, fp32.
* ``llama8b``       64 sequences, lengths uniform on 512..8192, 32 / 8 heads,
                    d = 128, bf16; pool 1.2x the blocks needed.
* ``shared_prefix`` 256 sequences sharing one 2000-token prefix (125 blocks),
                    unique suffixes uniform on 50..1000 tokens, 64 / 8 heads,
                    bf16; one sequence forks another mid-block, so exactly one
                    copy-on-write of a partial shared block happens.
* ``chunked``       one 1024-token query chunk over P cached tokens of context
                    (P in 16K..128K) plus 32 decode sequences of 4096 tokens,
                    64 / 8 heads, bf16.
* ``fp8_long``      16 sequences of 131072 tokens, 64 / 8 heads, bf16 queries,
                    K/V stored as fp8 E4M3 with per-head fp32 scales.
* ``int8_long``     the same shape with K/V stored as int8 codes with per-head
                    fp32 scales.

Values: K, V ~ N(0, 1) and Q ~ N(0, 1) ("plain"), or Q ~ N(0, 4^2) ("peaked":
the softmax concentrates on a few tokens so outputs are O(1)), or plain values
with "needles": keys planted at chosen positions so that one query head attends
almost only to that token.  Random numbers come from torch generators seeded
per (workload seed, purpose, index), on the device the caller names.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK = 16


@dataclass
class Op:
    """One pool operation of a workload script.

    kind: 'create' | 'append' | 'share_prefix' | 'fork' | 'free'.
    For 'append', ``n`` tokens of fresh values (drawn for ``op_id``) are written.
    Sequence ids are assigned 0, 1, 2, ... in creation order by both sides.
    """

    kind: str
    seq: int = -1
    n: int = 0
    op_id: int = -1


@dataclass
class Workload:
    name: str
    hq: int
    hkv: int
    d: int
    kv_dtype: str  # 'f32' | 'bf16' | 'fp8' | 'int8'
    q_dtype: str  # 'f32' | 'bf16'
    num_blocks: int
    placement: np.ndarray  # int32 permutation: order in which blocks are first handed out
    script: list  # list[Op]
    batch: list  # sequence ids, one per batch row
    q_lens: list  # query tokens per batch row (1 = decode)
    seed: int
    variant: str = "plain"
    # fp8 and int8 only: per kv-head fp32 scales for K and V (one layer).
    k_scale: np.ndarray | None = None
    v_scale: np.ndarray | None = None
    # positions of the tokens each sequence wrote itself: seq -> list of (start, stop)
    own_ranges: dict = field(default_factory=dict)
    num_layers: int = 1
    # shared_prefix only: tokens of the prefix every sequence shares
    shared_prefix_tokens: int = 0

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def value_dtype(self) -> torch.dtype:
        """dtype of the K/V values handed to the cache write."""
        return torch.float32 if self.kv_dtype == "f32" else torch.bfloat16

    def torch_q_dtype(self) -> torch.dtype:
        return torch.float32 if self.q_dtype == "f32" else torch.bfloat16


def _gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    h = 0
    for k in key:
        h = (h * 1000003 + int(k)) % (2**61 - 1)
    g.manual_seed(h)
    return g


def _stable_str(s: str) -> int:
    # str hash is salted per process; use a fixed code instead
    return sum((i + 1) * ord(c) for i, c in enumerate(s))


def placement(num_blocks: int, seed: int) -> np.ndarray:
    """Seeded random order in which the pool first hands out its blocks."""
    rng = np.random.default_rng(seed + 1000)
    return rng.permutation(num_blocks).astype(np.int32)


def _pool_size(logical_blocks: int, factor: float = 1.2) -> int:
    return int(math.ceil(factor * logical_blocks))


def _blocks(n_tokens: int) -> int:
    return -(-n_tokens // BLOCK)


def tiny(seed: int = 1, variant: str = "plain") -> Workload:
    lens = [300, 2000, 600, 4400]
    script, own = [], {}
    for s, L in enumerate(lens):
        script.append(Op("create"))
        script.append(Op("append", s, L, op_id=s))
        own[s] = [(0, L)]
    nb = _pool_size(sum(_blocks(L) for L in lens))
    return Workload("tiny", 8, 2, 128, "f32", "f32", nb, placement(nb, seed), script,
                    list(range(4)), [1] * 4, seed, variant, own_ranges=own)


def llama8b(seed: int = 2, variant: str = "plain", batch: int = 64,
            min_len: int = 512, max_len: int = 8192) -> Workload:
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(min_len, max_len + 1, size=batch)]
    script, own = [], {}
    for s, L in enumerate(lens):
        script.append(Op("create"))
        script.append(Op("append", s, L, op_id=s))
        own[s] = [(0, L)]
    nb = _pool_size(sum(_blocks(L) for L in lens))
    return Workload("llama8b", 32, 8, 128, "bf16", "bf16", nb, placement(nb, seed), script,
                    list(range(batch)), [1] * batch, seed, variant, own_ranges=own)


def shared_prefix(seed: int = 3, variant: str = "plain", nseq: int = 256,
                  prefix: int = 2000, min_suffix: int = 50, max_suffix: int = 1000,
                  hq: int = 64, hkv: int = 8, suffixes=None) -> Workload:
    """Sequence 0 writes the prefix; sequences 1..nseq-2 share its blocks and add
    their own suffix.  The last sequence forks sequence nseq-2 when that one
    holds prefix + r tokens (r not a multiple of 16), then both append the rest
    of their own suffixes: the first of them to write triggers the one copy.
    ``suffixes`` (one per sequence; the last two at least 2) replaces the drawn
    suffix lengths."""
    rng = np.random.default_rng(seed)
    suffix = [int(x) for x in rng.integers(min_suffix, max_suffix + 1, size=nseq)]
    if suffixes is not None:
        suffix = [int(x) for x in suffixes]
    script, own = [], {}
    op = 0
    script.append(Op("create"))
    script.append(Op("append", 0, prefix, op_id=op)); op += 1
    script.append(Op("append", 0, suffix[0], op_id=op)); op += 1
    own[0] = [(0, prefix + suffix[0])]
    for s in range(1, nseq - 1):
        script.append(Op("share_prefix", 0, prefix))
        if s < nseq - 2:
            script.append(Op("append", s, suffix[s], op_id=op)); op += 1
            own[s] = [(prefix, prefix + suffix[s])]
    # sequence nseq-2: first r tokens of its suffix, then fork, then the rest
    p = nseq - 2
    r = int(rng.integers(1, min(suffix[p], 64)))
    if r % BLOCK == 0:
        r += 1
    r = min(r, suffix[p] - 1)
    script.append(Op("append", p, r, op_id=op)); op += 1
    script.append(Op("fork", p))  # creates sequence nseq-1 with prefix + r tokens
    c = nseq - 1
    script.append(Op("append", c, suffix[c], op_id=op)); op += 1
    script.append(Op("append", p, suffix[p] - r, op_id=op)); op += 1
    own[p] = [(prefix, prefix + suffix[p])]
    own[c] = [(prefix + r, prefix + r + suffix[c])]
    logical = sum(_blocks(prefix + suffix[s]) for s in range(nseq - 1)) + _blocks(prefix + r + suffix[c])
    nb = _pool_size(logical)
    return Workload("shared_prefix", hq, hkv, 128, "bf16", "bf16", nb, placement(nb, seed), script,
                    list(range(nseq)), [1] * nseq, seed, variant, own_ranges=own, shared_prefix_tokens=prefix)


def chunked(context: int = 16384, chunk: int = 1024, n_decode: int = 32, decode_len: int = 4096,
            seed: int = 4, variant: str = "plain", hq: int = 64, hkv: int = 8) -> Workload:
    """Batch rows 0..n_decode-1 are decode sequences (one query each); the last
    row is the prefill chunk: its ``context`` earlier tokens and its ``chunk``
    new tokens are all in the cache, and its ``chunk`` queries are the new ones."""
    script, own = [], {}
    op = 0
    for s in range(n_decode):
        script.append(Op("create"))
        script.append(Op("append", s, decode_len, op_id=op)); op += 1
        own[s] = [(0, decode_len)]
    s = n_decode
    script.append(Op("create"))
    if context > 0:
        script.append(Op("append", s, context, op_id=op)); op += 1
    script.append(Op("append", s, chunk, op_id=op)); op += 1
    own[s] = [(0, context + chunk)]
    logical = n_decode * _blocks(decode_len) + _blocks(context + chunk)
    nb = _pool_size(logical)
    return Workload("chunked", hq, hkv, 128, "bf16", "bf16", nb, placement(nb, seed), script,
                    list(range(n_decode + 1)), [1] * n_decode + [chunk], seed, variant, own_ranges=own)


def fp8_long(seed: int = 5, variant: str = "plain", batch: int = 16, length: int = 131072,
             hq: int = 64, hkv: int = 8) -> Workload:
    script, own = [], {}
    for s in range(batch):
        script.append(Op("create"))
        script.append(Op("append", s, length, op_id=s))
        own[s] = [(0, length)]
    nb = _pool_size(batch * _blocks(length))
    rng = np.random.default_rng(seed + 77)
    k_scale = (1.0 / rng.uniform(48.0, 80.0, size=hkv)).astype(np.float32)
    v_scale = (1.0 / rng.uniform(48.0, 80.0, size=hkv)).astype(np.float32)
    return Workload("fp8_long", hq, hkv, 128, "fp8", "bf16", nb, placement(nb, seed), script,
                    list(range(batch)), [1] * batch, seed, variant,
                    k_scale=k_scale, v_scale=v_scale, own_ranges=own)


def int8_long(seed: int = 6, variant: str = "plain", batch: int = 16, length: int = 131072,
              hq: int = 64, hkv: int = 8) -> Workload:
    w = fp8_long(seed, variant, batch, length, hq, hkv)
    w.name = "int8_long"
    return scaled_int8(w)


def _scaled(w: Workload, kv_dtype: str) -> Workload:
    if kv_dtype == "fp8":
        return scaled_fp8(w)
    if kv_dtype == "int8":
        return scaled_int8(w)
    return w


def custom(lens, hq: int, hkv: int, kv_dtype: str = "bf16", seed: int = 11, variant: str = "plain",
           pool_factor: float = 1.2, name: str = "custom") -> Workload:
    """Decode rows of the given lengths (edge cases, small parity cases)."""
    script, own = [], {}
    for s, L in enumerate(lens):
        script.append(Op("create"))
        script.append(Op("append", s, int(L), op_id=s))
        own[s] = [(0, int(L))]
    nb = max(1, _pool_size(sum(_blocks(int(L)) for L in lens), pool_factor))
    w = Workload(name, hq, hkv, 128, "f32" if kv_dtype == "f32" else ("bf16" if kv_dtype == "bf16" else "bf16"),
                 "f32" if kv_dtype == "f32" else "bf16", nb, placement(nb, seed), script,
                 list(range(len(lens))), [1] * len(lens), seed, variant, own_ranges=own)
    return _scaled(w, kv_dtype)


def chunks(rows, hq: int = 64, hkv: int = 8, kv_dtype: str = "bf16", seed: int = 12, n_decode: int = 0,
           decode_len: int = 300, variant: str = "plain") -> Workload:
    """Decode rows first, then chunk rows given as (context, chunk) pairs: the
    context tokens and the chunk's own tokens are written, and the chunk's
    queries are the new ones."""
    script, own, q_lens = [], {}, []
    op = 0
    s = 0
    for _ in range(n_decode):
        script.append(Op("create"))
        script.append(Op("append", s, decode_len, op_id=op)); op += 1
        own[s] = [(0, decode_len)]
        q_lens.append(1)
        s += 1
    logical = n_decode * _blocks(decode_len)
    for ctx, c in rows:
        script.append(Op("create"))
        if ctx > 0:
            script.append(Op("append", s, ctx, op_id=op)); op += 1
        script.append(Op("append", s, c, op_id=op)); op += 1
        own[s] = [(0, ctx + c)]
        q_lens.append(c)
        logical += _blocks(ctx + c)
        s += 1
    nb = _pool_size(logical)
    w = Workload("chunks", hq, hkv, 128, "bf16", "bf16", nb, placement(nb, seed), script,
                 list(range(s)), q_lens, seed, variant, own_ranges=own)
    return _scaled(w, kv_dtype)


def scaled_fp8(w: Workload) -> Workload:
    """Give a bf16 workload fp8 storage with seeded per-head scales."""
    rng = np.random.default_rng(w.seed + 77)
    w.kv_dtype = "fp8"
    w.k_scale = (1.0 / rng.uniform(48.0, 80.0, size=w.hkv)).astype(np.float32)
    w.v_scale = (1.0 / rng.uniform(48.0, 80.0, size=w.hkv)).astype(np.float32)
    return w


def scaled_int8(w: Workload) -> Workload:
    """Give a bf16 workload int8 storage with seeded per-head scales: 1/24 ..
    1/32, so N(0, 1) values use most of the code range and the largest ones
    (beyond 4 to 5.3 standard deviations) reach the clamp at +-127."""
    rng = np.random.default_rng(w.seed + 78)
    w.kv_dtype = "int8"
    w.k_scale = (1.0 / rng.uniform(24.0, 32.0, size=w.hkv)).astype(np.float32)
    w.v_scale = (1.0 / rng.uniform(24.0, 32.0, size=w.hkv)).astype(np.float32)
    return w


# ---------------------------------------------------------------------------
# values


def replay_lengths(w: Workload):
    """Bookkeeping only: the final token count of every sequence id and the
    position at which each 'append' op starts writing."""
    lens, starts = {}, {}
    nxt = 0
    for op in w.script:
        if op.kind == "create":
            lens[nxt] = 0
            nxt += 1
        elif op.kind == "append":
            starts[op.op_id] = lens[op.seq]
            lens[op.seq] += op.n
        elif op.kind == "share_prefix":
            lens[nxt] = op.n
            nxt += 1
        elif op.kind == "fork":
            lens[nxt] = lens[op.seq]
            nxt += 1
        elif op.kind == "free":
            del lens[op.seq]
    return lens, starts


def query_row(w: Workload, row: int, device="cpu") -> torch.Tensor:
    """Queries of one batch row: [q_lens[row], Hq, d] in the query dtype."""
    g = _gen(device, w.seed, _stable_str("q"), row)
    q = torch.randn((w.q_lens[row], w.hq, w.d), generator=g, device=device, dtype=torch.float32)
    if w.variant == "peaked":
        q = q * 4.0
    return q.to(w.torch_q_dtype())


def queries(w: Workload, device="cpu") -> torch.Tensor:
    """Queries for every batch row, concatenated: [sum(q_lens), Hq, d]."""
    return torch.cat([query_row(w, b, device) for b in range(len(w.q_lens))], 0)


def needle_positions(w: Workload, row: int, length: int, split_hint: int = 512) -> list:
    """Positions (one per query head of a group) for planted keys of one batch
    row: the first and last token, a block boundary pair, split boundaries and
    seeded interior positions, restricted to tokens the sequence wrote itself."""
    seq = w.batch[row]
    ranges = w.own_ranges.get(seq, [])
    cand = [0, length - 1, 15, 16, split_hint - 1, split_hint, 2 * split_hint - 1]
    rng = np.random.default_rng(w.seed * 7919 + row)
    cand += [int(x) for x in rng.integers(0, max(length, 1), size=w.group)]
    ok = [t for t in cand if 0 <= t < length and any(a <= t < b for a, b in ranges)]
    out = []
    for t in ok:
        if t not in out:
            out.append(t)
    return out[: w.group]


def append_values(w: Workload, op: Op, device="cpu", start: int | None = None, final_len: int | None = None):
    """K and V values [n, Hkv, d] written by one 'append' op.

    For the 'needle' variant, ``start`` (where the op starts writing) and
    ``final_len`` (the sequence's final length) place the planted keys: for kv
    head j and the i-th query head h of its group, the key at the i-th needle
    position is 4 * sqrt(d) * q_h / |q_h|, so head h's score there is about
    4 |q_h|, far above every other score."""
    g = _gen(device, w.seed, _stable_str("kv"), op.op_id)
    k = torch.randn((op.n, w.hkv, w.d), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((op.n, w.hkv, w.d), generator=g, device=device, dtype=torch.float32)
    if w.variant == "needle":
        if start is None or final_len is None:
            lens, starts = replay_lengths(w)
            start, final_len = starts[op.op_id], lens[op.seq]
        for row, seq in enumerate(w.batch):
            if seq != op.seq or w.q_lens[row] != 1:
                continue
            q = query_row(w, row, device)[0].to(torch.float32)
            for i, t in enumerate(needle_positions(w, row, final_len)):
                if start <= t < start + op.n:
                    for j in range(w.hkv):
                        qh = q[j * w.group + i]
                        k[t - start, j] = 4.0 * math.sqrt(w.d) * qh / qh.norm()
    return k.to(w.value_dtype()), v.to(w.value_dtype())
