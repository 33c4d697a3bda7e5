"""Builds one workload on both sides from the same seeded inputs.

HIP side: the library's allocator replays the workload script, its kernels
write the values into the device cache (and run the copy-on-write copies), and
its attention kernels produce the outputs under test.

Oracle side: the oracle's pool model replays the same script; a token store
records, for every slot, which generated value was written there (op id and
offset), so a row's K/V are read back through the oracle's own tables; fp8
and int8 values are quantised by the oracle's codecs.  Attention is the oracle's fp64
definition.  Nothing on this side reads anything the HIP side produced.
"""

from __future__ import annotations

import numpy as np
import torch

import workloads as W
from oracle import attention as OA
from oracle import fp8 as OF
from oracle import int8 as OI
from oracle import pool as OP

# int8 codes convert to bf16 exactly, so an int8 cache runs the bf16 path's
# arithmetic on the same stored values: the bf16 bound applies.
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "int8": 2e-2}


def blocks(n: int) -> int:
    return -(-n // 16)


class HipSide:
    def __init__(self, w: W.Workload, device="cuda", placement=None, layer=0, num_layers=1, fill_byte=None):
        import paged_kv_cache_263_amd as pk

        self.pk = pk
        self.w = w
        self.device = device
        self.layer = layer
        order = w.placement if placement is None else placement
        self.pool = pk.kv_pool_create(w.num_blocks, order)
        ks = vs = None
        if w.kv_dtype in ("fp8", "int8"):
            ks = np.tile(w.k_scale, (num_layers, 1))
            vs = np.tile(w.v_scale, (num_layers, 1))
        self.cache = pk.KVCache(w.kv_dtype, num_layers, w.num_blocks, w.hkv, device, k_scale=ks, v_scale=vs)
        if fill_byte is not None:  # unwritten slots hold this byte pattern (0xFF: NaN in every dtype)
            self.cache.k_pool.view(torch.uint8).fill_(fill_byte)
            self.cache.v_pool.view(torch.uint8).fill_(fill_byte)
        lens, starts = W.replay_lengths(w)
        self.n_copies = 0
        for op in w.script:
            if op.kind == "create":
                pk.seq_create(self.pool)
            elif op.kind == "append":
                slots, copies = pk.seq_append(self.pool, op.seq, op.n)
                if copies:
                    pk.kv_copy_blocks(self.cache, copies)
                    self.n_copies += len(copies)
                k, v = W.append_values(w, op, device, starts[op.op_id], lens[op.seq])
                pk.kv_cache_write(self.cache, k, v, torch.tensor(slots, dtype=torch.int32, device=device),
                                  layer=layer)
                del k, v
            elif op.kind == "share_prefix":
                pk.seq_share_prefix(self.pool, op.seq, op.n)
            elif op.kind == "fork":
                pk.seq_fork(self.pool, op.seq)
            elif op.kind == "free":
                pk.seq_free(self.pool, op.seq)
        self.lens = [pk.seq_len(self.pool, s) for s in w.batch]
        self.max_blocks = max(blocks(L) for L in self.lens)
        table, klens = pk.block_table_build(self.pool, w.batch, self.max_blocks)
        self.table_host = table
        self.table = table.to(device)
        self.kv_lens = klens.to(device)
        self.max_kv_len = max(self.lens)
        self.q = W.queries(w, device)

    def decode(self, **kw):
        return self.pk.paged_attn_decode(self.cache, self.q, self.table, self.kv_lens, self.max_kv_len,
                                         layer=self.layer, **kw)

    def prefill(self, **kw):
        w = self.w
        cu = [0]
        for n in w.q_lens:
            cu.append(cu[-1] + n)
        nd = 0
        while nd < len(w.q_lens) and w.q_lens[nd] == 1:
            nd += 1
        cu_q = torch.tensor(cu, dtype=torch.int32, device=self.device)
        mdl = max(self.lens[:nd]) if nd else 0
        mq = max(w.q_lens[nd:]) if nd < len(w.q_lens) else 0
        return self.pk.paged_attn_prefill_chunk(self.cache, self.q, cu_q, self.table, self.kv_lens,
                                                self.max_kv_len, nd, mq, layer=self.layer,
                                                max_decode_kv_len=mdl, **kw)


class OracleSide:
    def __init__(self, w: W.Workload, device="cuda"):
        self.w = w
        self.device = device
        self.pool = OP.PoolModel(w.num_blocks, order=w.placement)
        self.store = OP.TokenStore(w.num_blocks, (), np.int64)
        self.final_lens, self.starts = W.replay_lengths(w)
        self.ops = {}
        for op in w.script:
            if op.kind == "create":
                self.pool.seq_create()
            elif op.kind == "append":
                slots, copies = self.pool.append(op.seq, op.n)
                for c in copies:
                    self.store.copy_block(c)
                self.store.write(slots, (np.int64(op.op_id) << 32) + np.arange(op.n, dtype=np.int64))
                self.ops[op.op_id] = op
            elif op.kind == "share_prefix":
                self.pool.share_prefix(op.seq, op.n)
            elif op.kind == "fork":
                self.pool.fork(op.seq)
            elif op.kind == "free":
                self.pool.seq_free(op.seq)
        self._vals = {}

    def row_len(self, row: int) -> int:
        return self.pool.seq_len(self.w.batch[row])

    def _op_values(self, op_id: int):
        if op_id not in self._vals:
            if len(self._vals) > 4:
                self._vals.pop(next(iter(self._vals)))
            op = self.ops[op_id]
            self._vals[op_id] = W.append_values(self.w, op, self.device, self.starts[op_id],
                                                self.final_lens[op.seq])
        return self._vals[op_id]

    def row_kv(self, row: int, kvh: int, upto: int | None = None, quantised: bool = True):
        """float64 K, V [L, d] of one row and kv head, read through the oracle's
        table (and, for fp8 and int8, through the oracle's quantiser unless
        ``quantised`` is False: then the values before storage)."""
        seq = self.w.batch[row]
        L = self.pool.seq_len(seq) if upto is None else upto
        ids = self.store.gather(self.pool.seq_blocks(seq), L)
        op_ids, offs = ids >> 32, ids & 0xFFFFFFFF
        K = np.empty((L, self.w.d), dtype=np.float64)
        V = np.empty((L, self.w.d), dtype=np.float64)
        for oid in np.unique(op_ids):
            sel = np.nonzero(op_ids == oid)[0]
            k, v = self._op_values(int(oid))
            idx = torch.as_tensor(offs[sel], device=k.device)
            kk = k[idx, kvh].float().cpu().numpy()
            vv = v[idx, kvh].float().cpu().numpy()
            codec = {"fp8": OF, "int8": OI}.get(self.w.kv_dtype)
            if codec is not None and quantised:
                kk = codec.dequantise(codec.quantise_scaled(kk, self.w.k_scale[kvh]), self.w.k_scale[kvh])
                vv = codec.dequantise(codec.quantise_scaled(vv, self.w.v_scale[kvh]), self.w.v_scale[kvh])
            K[sel] = kk
            V[sel] = vv
        return K, V

    def decode(self, row: int, heads=None, quantised: bool = True) -> np.ndarray:
        """Oracle output [len(heads), d] for a decode row (over the values
        before fp8 / int8 storage if ``quantised`` is False)."""
        w = self.w
        heads = list(range(w.hq)) if heads is None else list(heads)
        q = W.query_row(w, row, self.device)[0].float().cpu().numpy()
        out = np.empty((len(heads), w.d))
        for j in sorted({h // w.group for h in heads}):
            hs = [h for h in heads if h // w.group == j]
            K, V = self.row_kv(row, j, quantised=quantised)
            o = OA.decode_rows(q[hs], K[:, None, :], V[:, None, :], list(range(len(hs))))
            for h, oo in zip(hs, o):
                out[heads.index(h)] = oo
        return out

    def chunk_rows(self, row: int, tokens, heads=None) -> np.ndarray:
        """Oracle output [len(tokens), len(heads), d] for chosen queries of a chunk row."""
        w = self.w
        heads = list(range(w.hq)) if heads is None else list(heads)
        q = W.query_row(w, row, self.device).float().cpu().numpy()  # [C, Hq, d]
        C = q.shape[0]
        L = self.row_len(row)
        out = np.empty((len(tokens), len(heads), w.d))
        for j in sorted({h // w.group for h in heads}):
            hs = [h for h in heads if h // w.group == j]
            K, V = self.row_kv(row, j)
            o = OA.prefill_rows(q[:, hs], K[:, None, :], V[:, None, :], tokens)
            for a, h in enumerate(hs):
                out[:, heads.index(h)] = o[:, a]
        del C, L
        return out


def q_offsets(w: W.Workload):
    off = [0]
    for n in w.q_lens:
        off.append(off[-1] + n)
    return off


def compare(got: np.ndarray, ref: np.ndarray, tol: float, what: str):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref).max()
    rel = err / max(np.abs(ref).max(), 1e-30)
    print(f"{what}: max|err| {err:.3e} (tol {tol:g}), max|ref| {np.abs(ref).max():.3e}, rel {rel:.2e}", flush=True)
    assert err <= tol, f"{what}: max abs error {err} > {tol}"
    return err
