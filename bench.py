"""Paged GQA decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b]

One step is one decode step of the whole hot path for a batch of sequences
whose K/V already sit in the paged cache in HBM:
  1. host allocator: one new token for every sequence (a new block every 16
     tokens, copy-on-write if the tail block is shared), slots returned;
  2. cache write: the new tokens' K/V to their slots, device block table and
     lengths kept up to date in the same kernel, which reads the slots and
     positions straight from the pinned host memory the allocator wrote;
  3. paged decode: the decode kernel (the blocks of all rows divided evenly
     among the wavefronts of each kv head, each wavefront taking the prefix
     sum of blocks per row itself), and the merge kernel for rows cut between
     wavefronts.
``value`` is the KV bytes every step attends (sum of lengths x kv heads x 128
x 2 x element bytes) divided by the measured step time.  The line also
carries the roofline of the dominant kernel (the decode kernel, timed
with HIP events recorded on its stream by the library around it), and the
CPU oracle timed on a bounded sample of the same workload.

Default workload: a Llama-3-8B-shaped decode layer: 64 sequences, lengths
uniform on 512..8192, 32 query / 8 kv heads, d = 128, bf16, 16-token blocks
placed by a seeded shuffle in a pool 1.2x the blocks needed.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
DTYPE_LABEL = {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 kv / bf16 q", "int8": "int8 kv / bf16 q"}
WORKLOADS = ("llama8b", "tiny", "shared_prefix", "fp8_long", "int8_long", "chunked", "swap", "prefix_cache")


class TimingEvents:
    """n x k hipEvents for timing kernels on one stream.  They are created with
    hipEventDisableSystemFence: a default event's record also writes back and
    invalidates the caches at system scope, which holds the next kernel back by
    several microseconds; nothing waits on these events, they only carry
    timestamps."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int, k: int):
        import ctypes

        import paged_kv_cache_263_amd as pk

        vp = ctypes.c_void_p
        self._create = pk._hip_fn("hipEventCreateWithFlags", ctypes.c_int, [ctypes.POINTER(vp), ctypes.c_uint])
        self._record = pk._hip_fn("hipEventRecord", ctypes.c_int, [vp, vp])
        self._elapsed = pk._hip_fn("hipEventElapsedTime", ctypes.c_int, [ctypes.POINTER(ctypes.c_float), vp, vp])
        self._destroy = pk._hip_fn("hipEventDestroy", ctypes.c_int, [vp])
        self.ev = []
        for _ in range(n):
            row = []
            for _ in range(k):
                e = vp()
                if self._create(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
                row.append(e.value)
            self.ev.append(row)

    def handles(self, i: int, idx=None):
        return [self.ev[i][j] for j in (idx if idx is not None else range(len(self.ev[i])))]

    def record(self, i: int, j: int, stream) -> None:
        if self._record(self.ev[i][j], stream.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i: int, a: int, b: int) -> float:
        import ctypes

        out = ctypes.c_float()
        if self._elapsed(ctypes.byref(out), self.ev[i][a], self.ev[i][b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def __del__(self):
        for row in getattr(self, "ev", []):
            for e in row:
                self._destroy(e)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b", choices=WORKLOADS)
    ap.add_argument("--decode-parts", type=int, default=0, help="wavefronts per kv head (0 = auto)")
    ap.add_argument("--context", type=int, default=16384, help="chunked: cached context before the chunk")
    ap.add_argument("--chunk", type=int, default=1024, help="chunked: queries in the chunk")
    ap.add_argument("--prefill-parts", type=int, default=0, help="chunked: key ranges per query tile (0 = auto)")
    ap.add_argument("--kv", default="bf16", choices=("bf16", "fp8", "int8"), help="chunked: cache dtype")
    ap.add_argument("--fixed-len", type=int, default=0,
                    help="llama8b: every row this long instead of uniform 512..8192 (a balance control)")
    ap.add_argument("--placement", default="shuffled", choices=("shuffled", "identity"),
                    help="physical block order: the workload's seeded shuffle, or identity (a contiguous control)")
    ap.add_argument("--no-prefix-pass", action="store_true",
                    help="shared_prefix: do not pass the shared-prefix promise (every row reads the prefix itself)")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="decode workloads: extra steps after the timed ones, each after writing a 512 MiB scratch "
                         "buffer (more than the 256 MB last-level cache), timed with events only (reported apart)")
    ap.add_argument("--cold-flush", choices=["write", "read"], default="read",
                    help="how the cold-cache steps displace the cache: write the scratch buffer, or read it "
                         "(written once beforehand, so no dirty lines are left to write back)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=0, help="rows in the oracle sample (0 = auto)")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="print a summary of rocprofv3 CSV output (kernel trace, FETCH_SIZE pass, WRITE_SIZE pass) "
                         "and exit")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a dispatch of known size that "
                         "scales hardware byte counters)")
    return ap.parse_args()


def build_workload(name: str, args=None):
    import workloads as W

    if name == "chunked":
        w = W.chunked(context=args.context, chunk=args.chunk)
        return {"fp8": W.scaled_fp8, "int8": W.scaled_int8}.get(args.kv, lambda x: x)(w)
    if name == "llama8b" and args is not None and args.fixed_len:
        return W.llama8b(min_len=args.fixed_len, max_len=args.fixed_len)
    return {"llama8b": W.llama8b, "tiny": W.tiny, "shared_prefix": W.shared_prefix, "fp8_long": W.fp8_long,
            "int8_long": W.int8_long}[name]()


def describe(w) -> str:
    return {
        "llama8b": "Llama-3-8B-shaped paged GQA decode layer: batch 64, 32 q / 8 kv heads, d 128, bf16 K/V/Q, "
                   "KV lengths uniform 512-8192, 16-token blocks shuffled in a pool 1.2x need",
        "tiny": "tiny paged decode: 4 seqs of KV length 300/2000/600/4400, 8 q / 2 kv heads, d 128, fp32, "
                "16-token blocks shuffled in a pool",
        "shared_prefix": "shared-prefix paged decode: 256 seqs sharing a 2000-token prefix (125 blocks) + unique "
                         "suffix 50-1000, 64 q / 8 kv heads, bf16, one copy-on-write",
        "fp8_long": "long-context fp8 paged decode: batch 16, KV length 131072, 64 q / 8 kv heads, fp8 E4M3 K/V "
                    "with per-head fp32 scales, bf16 Q",
        "int8_long": "long-context int8 paged decode: batch 16, KV length 131072, 64 q / 8 kv heads, int8 K/V "
                     "with per-head fp32 scales, bf16 Q",
        "chunked": "chunked prefill: one 1024-query causal chunk over cached context, batched with 32 decode "
                   "rows of 4096 tokens, 64 q / 8 kv heads, d 128",
    }[w.name]


def run_chunked(args, w, device):
    """Times paged_attn_prefill_chunk on a fixed cache state (chunk K/V already
    written): the prefill kernel (MFMA-bound) and the decode rows' kernels."""
    import paged_kv_cache_263_amd as pk

    pool, cache = setup(w, device)
    lens = [pk.seq_len(pool, s) for s in w.batch]
    mb = max(-(-L // 16) for L in lens)
    table_h, lens_h = pk.block_table_build(pool, w.batch, mb)
    table, klens = table_h.to(device), lens_h.to(device)
    q = __import__("workloads").queries(w, device)
    nd = sum(1 for n in w.q_lens if n == 1)
    cu = [0]
    for n in w.q_lens:
        cu.append(cu[-1] + n)
    cu_q = torch.tensor(cu, dtype=torch.int32, device=device)
    out = torch.empty_like(q)
    total = args.warmup + args.steps
    ev = TimingEvents(total, 4)
    mdl = max(lens[:nd])
    a = pk._args(cache, q, out, table, klens, max(lens), 0, args.decode_parts, None, cu_q=cu_q, num_decode=nd,
                 max_decode_kv_len=mdl, max_q_len=max(w.q_lens), total_q=q.shape[0])
    a.prefill_parts = args.prefill_parts
    ws = torch.empty(max(16, pk.paged_attn_workspace_size(cache, a)), dtype=torch.uint8, device=device)
    torch.cuda.synchronize()

    def step(i):
        pk.paged_attn_prefill_chunk(cache, q, cu_q, table, klens, max(lens), nd, max(w.q_lens), out=out,
                                    max_decode_kv_len=mdl, decode_parts=args.decode_parts, workspace=ws,
                                    events=ev.handles(i), prefill_parts=args.prefill_parts)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, total):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    timed = range(args.warmup, total)
    dec_ms = float(np.mean([ev.ms(i, 0, 2) for i in timed]))  # decode + merge
    pre_ms = float(np.mean([ev.ms(i, 2, 3) for i in timed]))
    C = max(w.q_lens)
    P = lens[-1] - C
    flops = 4.0 * w.d * w.hq * (C * P + C * (C + 1) / 2)
    dec_bytes = sum(lens[:nd]) * w.hkv * w.d * 2 * elt_bytes(w)
    tflops = flops / (pre_ms / 1e3) / 1e12
    return {
        "metric": "chunked prefill + decode rows: prefill TFLOP/s (causal algorithmic flops)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE_LABEL[w.kv_dtype],
        "data": "synthetic",
        "config": {"workload": describe(w), "context": P, "chunk": C, "decode_rows": nd},
        "kernels_us": {"decode_part": round(dec_ms * 1e3, 2), "prefill": round(pre_ms * 1e3, 2)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_kernel"},
        "decode_part_gbs": round(dec_bytes / (dec_ms / 1e3) / 1e9, 1),
    }


def run_prefix_cache(args):
    """Serves the four reuse structures of the pages' table (few-shot, agent
    loop, multi-turn chat, RAG; seeded synthetic token ids) through the
    library's allocator with prefix caching: match, append the rest, register,
    append and register the reply, free (blocks retained).  Reports the hit
    rate (matched / prompt tokens), the prefill tokens saved, and the
    allocator's request rate on the host."""
    import paged_kv_cache_263_amd as pk
    from workloads import traffic as T

    pages = {"few_shot": "95%", "agent": "~90%", "chat": "90%+ by turn 6-8", "rag": "5-15%"}
    streams = {}
    t_all, n_all = 0.0, 0
    for name, make in T.STREAMS.items():
        reqs = make()
        pool = pk.kv_pool_create(200000, None)
        matched = []
        t0 = time.perf_counter()
        for r in reqs:
            s, m = pk.seq_create_cached(pool, 1, r.prompt)
            pk.seq_append(pool, s, len(r.prompt) - m)
            keyed = m // 16 + pk.seq_cache_tokens(pool, s, m, r.prompt[m:])
            if r.reply:
                full = r.prompt + r.reply
                pk.seq_append(pool, s, len(r.reply))
                pk.seq_cache_tokens(pool, s, 16 * keyed, full[16 * keyed:])
            pk.seq_free(pool, s)
            matched.append(m)
        t_all += time.perf_counter() - t0
        n_all += len(reqs)
        prompt = sum(len(r.prompt) for r in reqs)
        entry = {"requests": len(reqs), "prompt_tokens": prompt, "matched_tokens": sum(matched),
                 "hit_rate": round(sum(matched) / prompt, 4), "pages": pages[name]}
        if name == "chat":
            k = max(r.session for r in reqs) + 1
            entry["hit_rate_by_turn"] = [
                round(sum(matched[t * k:(t + 1) * k]) / sum(len(r.prompt) for r in reqs[t * k:(t + 1) * k]), 4)
                for t in range(len(reqs) // k)]
        streams[name] = entry
    total_prompt = sum(e["prompt_tokens"] for e in streams.values())
    total_matched = sum(e["matched_tokens"] for e in streams.values())
    return {
        "metric": "prefix caching with retention: prompt tokens matched (prefill saved), pages' reuse structures",
        "value": round(total_matched / total_prompt, 4), "unit": "fraction of prompt tokens",
        "n_gpus": 0, "steps": 1, "warmup": 0, "ms_per_step": round(t_all * 1e3, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32 token ids", "data": "synthetic",
        "config": {"workload": "few-shot / agent / chat / RAG request streams, 16-token blocks, one tenant"},
        "streams": streams, "requests_per_s_host": round(n_all / t_all, 1),
    }


def run_swap(args, device):
    """Swap one 8192-token sequence of a 32-layer, 8-kv-head bf16 cache (the
    Llama-3-8B shape: 512 blocks, 1.07 GB of K/V) out to pinned host memory and
    back into other blocks: seq_swap_out + kv_swap_out, then seq_swap_in +
    kv_swap_in, each timed with HIP events around the copy kernels.  Also
    times one plain 1.07 GB device-to-host and host-to-device copy of a
    contiguous buffer (the host link's DMA rate) for comparison.  The pages
    quote 34 ms for 1.07 GB over PCIe (~31.6 GB/s)."""
    import paged_kv_cache_263_amd as pk

    layers, hkv, tokens = 32, 8, 8192
    nblk = tokens // 16
    pool = pk.kv_pool_create(2 * nblk + 8, None)
    cache = pk.KVCache("bf16", layers, 2 * nblk + 8, hkv, device, zero=False)
    g = torch.Generator(device=device).manual_seed(7)
    cache.k_pool.view(torch.int16).random_(-32768, 32767, generator=g)
    cache.v_pool.view(torch.int16).random_(-32768, 32767, generator=g)
    seq = pk.seq_create(pool)
    pk.seq_append(pool, seq, tokens)
    slot = pk.kv_swap_block_bytes(cache)
    total = nblk * slot
    host = torch.empty(total, dtype=torch.uint8).pin_memory()
    ev = TimingEvents(args.warmup + args.steps, 4)
    stream = torch.cuda.current_stream()
    out_ms, in_ms, host_ms = [], [], []
    for i in range(args.warmup + args.steps):
        t0 = time.perf_counter()
        ids = pk.seq_swap_out(pool, seq)
        ev.record(i, 0, stream)
        pk.kv_swap_out(cache, ids, host)
        ev.record(i, 1, stream)
        new_ids = pk.seq_swap_in(pool, seq)
        ev.record(i, 2, stream)
        pk.kv_swap_in(cache, host, new_ids)
        ev.record(i, 3, stream)
        torch.cuda.synchronize()
        host_ms.append((time.perf_counter() - t0) * 1e3)
        if i >= args.warmup:
            out_ms.append(ev.ms(i, 0, 1))
            in_ms.append(ev.ms(i, 2, 3))
    # the host link's DMA rate on one contiguous buffer of the same size
    dev_buf = torch.empty(total, dtype=torch.uint8, device=device)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for _ in range(2):
        e0.record()
        host.copy_(dev_buf, non_blocking=True)
        e1.record()
        dev_buf.copy_(host, non_blocking=True)
        e2.record()
        torch.cuda.synchronize()
    d2h, h2d = e0.elapsed_time(e1), e1.elapsed_time(e2)
    gbs_out = total / (float(np.mean(out_ms)) / 1e3) / 1e9
    gbs_in = total / (float(np.mean(in_ms)) / 1e3) / 1e9
    return {
        "metric": "swap of one 8192-token sequence to pinned host memory and back: GB/s over the host link",
        "value": round(min(gbs_out, gbs_in), 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(float(np.mean(host_ms[args.warmup:])), 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap: 32 layers x 8 kv heads x 128 d bf16 cache, one 8192-token sequence "
                               "(512 blocks)", "bytes": total, "layers": layers, "kv_heads": hkv, "tokens": tokens},
        "swap_out_ms": round(float(np.mean(out_ms)), 3), "swap_in_ms": round(float(np.mean(in_ms)), 3),
        "swap_out_gbs": round(gbs_out, 2), "swap_in_gbs": round(gbs_in, 2),
        "dma_copy_gbs": {"d2h": round(total / (d2h / 1e3) / 1e9, 2), "h2d": round(total / (h2d / 1e3) / 1e9, 2)},
        "pages_gbs": round(1.07e9 / 34e-3 / 1e9, 2),
    }


def setup(w, device):
    """Fill the paged cache through the library: replay the workload script on
    the host allocator, write every append's values with the cache-write
    kernel (and run copy-on-write copies)."""
    import paged_kv_cache_263_amd as pk
    import workloads as W

    pool = pk.kv_pool_create(w.num_blocks, w.placement)
    ks = vs = None
    if w.kv_dtype in ("fp8", "int8"):
        ks, vs = w.k_scale.reshape(1, -1), w.v_scale.reshape(1, -1)
    cache = pk.KVCache(w.kv_dtype, 1, w.num_blocks, w.hkv, device, k_scale=ks, v_scale=vs, zero=False)
    lens, starts = W.replay_lengths(w)
    for op in w.script:
        if op.kind == "create":
            pk.seq_create(pool)
        elif op.kind == "append":
            slots, copies = pk.seq_append(pool, op.seq, op.n)
            if copies:
                pk.kv_copy_blocks(cache, copies)
            k, v = W.append_values(w, op, device, starts[op.op_id], lens[op.seq])
            pk.kv_cache_write(cache, k, v, torch.tensor(slots, dtype=torch.int32, device=device))
            del k, v
        elif op.kind == "share_prefix":
            pk.seq_share_prefix(pool, op.seq, op.n)
        elif op.kind == "fork":
            pk.seq_fork(pool, op.seq)
    torch.cuda.synchronize()
    return pool, cache


def cpu_baseline(w, device, rows: int, budget_s: float = 10.0, single_core_s: float = 0.0, gpu_row0=None):
    """The oracle as it stands, on a bounded sample of the same workload: the
    oracle's pool model replays the script; then, row after row (the first
    ``rows`` batch rows, in full passes, at most twenty), it reads each row's
    K/V through its own table (fp8, int8: through its own codecs) and computes fp64
    attention for all query heads, until ``budget_s`` seconds of oracle time
    have accumulated.  Reported in the metric's unit: KV bytes covered /
    oracle seconds.  Input generation and host transfer are not timed.

    BLAS runs on every core of this process's affinity mask; with
    ``single_core_s`` > 0 the same loop runs again limited to one thread for
    that long.  ``gpu_row0`` (a one-byte cache: the GPU output [Hq, d] of batch
    row 0 before any token was appended) is compared with the oracle over the
    stored codes and over the values before quantisation: the drift the cache
    format adds, reported and not gated."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import workloads as W
    from oracle import attention as OA
    from oracle import fp8 as OF
    from oracle import int8 as OI
    from oracle import pool as OP

    model = OP.PoolModel(w.num_blocks, order=w.placement)
    store = OP.TokenStore(w.num_blocks, (), np.int64)
    final, starts = W.replay_lengths(w)
    ops = {}
    for op in w.script:
        if op.kind == "create":
            model.seq_create()
        elif op.kind == "append":
            slots, copies = model.append(op.seq, op.n)
            for c in copies:
                store.copy_block(c)
            store.write(slots, (np.int64(op.op_id) << 32) + np.arange(op.n, dtype=np.int64))
            ops[op.op_id] = op
        elif op.kind == "share_prefix":
            model.share_prefix(op.seq, op.n)
        elif op.kind == "fork":
            model.fork(op.seq)
    cache = {}

    def inputs(row):
        seq = w.batch[row]
        L = model.seq_len(seq)
        ids = store.gather(model.seq_blocks(seq), L)
        op_ids, offs = ids >> 32, ids & 0xFFFFFFFF
        vals = {}
        for oid in np.unique(op_ids):
            if int(oid) not in cache:
                op = ops[int(oid)]
                k, v = W.append_values(w, op, device, starts[op.op_id], final[op.seq])
                if sum(kk.nbytes + vv.nbytes for kk, vv in cache.values()) > (4 << 30):
                    cache.clear()  # keep the host copy of the inputs under ~4 GiB
                cache[int(oid)] = (k.float().cpu().numpy(), v.float().cpu().numpy())
            vals[int(oid)] = cache[int(oid)]
        q = W.query_row(w, row, device)[0].float().cpu().numpy()
        return L, op_ids, offs, vals, q

    def gather(row, quantised=True):
        L, op_ids, offs, vals, q = inputs(row)
        K = np.empty((L, w.hkv, w.d))
        V = np.empty((L, w.hkv, w.d))
        for oid, (k, v) in vals.items():
            sel = np.nonzero(op_ids == oid)[0]
            kk, vv = k[offs[sel]], v[offs[sel]]
            codec = {"fp8": OF, "int8": OI}.get(w.kv_dtype)
            if codec is not None and quantised:
                ks, vs = w.k_scale[None, :, None], w.v_scale[None, :, None]
                kk = codec.dequantise(codec.quantise_scaled(kk, ks), ks)
                vv = codec.dequantise(codec.quantise_scaled(vv, vs), vs)
            K[sel], V[sel] = kk, vv
        return L, q, K, V

    def run(budget):
        spent, kv_bytes, done_rows, passes = 0.0, 0, 0, 0
        while spent < budget and passes < 20:
            for row in range(rows):
                L, op_ids, offs, vals, q = inputs(row)
                t0 = time.perf_counter()
                K = np.empty((L, w.hkv, w.d))
                V = np.empty((L, w.hkv, w.d))
                for oid, (k, v) in vals.items():
                    sel = np.nonzero(op_ids == oid)[0]
                    kk, vv = k[offs[sel]], v[offs[sel]]
                    codec = {"fp8": OF, "int8": OI}.get(w.kv_dtype)
                    if codec is not None:
                        ks, vs = w.k_scale[None, :, None], w.v_scale[None, :, None]
                        kk = codec.dequantise(codec.quantise_scaled(kk, ks), ks)
                        vv = codec.dequantise(codec.quantise_scaled(vv, vs), vs)
                    K[sel], V[sel] = kk, vv
                OA.decode(q, K, V)
                spent += time.perf_counter() - t0
                kv_bytes += L * w.hkv * w.d * 2 * elt_bytes(w)
                done_rows += 1
                if spent >= budget:
                    break
            passes += 1
        return spent, kv_bytes, done_rows

    ncores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=ncores):
        spent, kv_bytes, done_rows = run(budget_s)
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    res = {"value": kv_bytes / spent / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{done_rows} row-decodes over the first {rows} of {len(w.batch)} rows (all {w.hq} query "
                     f"heads, full lengths), {kv_bytes / 1e9:.3f} GB of KV in {spent:.2f} s; fp64 numpy",
           "seconds": round(spent, 3), "affinity_cores": ncores}
    if single_core_s > 0:
        with threadpool_limits(limits=1):
            s1, b1, r1 = run(single_core_s)
        res["single_core"] = {"value": b1 / s1 / 1e9, "unit": "GB/s", "cores": 1,
                              "sample": f"{r1} row-decodes, {b1 / 1e9:.3f} GB of KV in {s1:.2f} s"}
    if gpu_row0 is not None:
        _, q, K, V = gather(0, quantised=True)
        ref_q = OA.decode(q, K, V)
        _, q, K, V = gather(0, quantised=False)
        ref_u = OA.decode(q, K, V)
        g = np.asarray(gpu_row0, dtype=np.float64)
        drift = float(np.abs(g - ref_u).max())
        res["quant_drift"] = {
            "row": 0, "heads": w.hq,
            "max_abs_vs_unquantised": drift,
            "rel_vs_unquantised": drift / max(float(np.abs(ref_u).max()), 1e-30),
            "max_abs_vs_stored_codes": float(np.abs(g - ref_q).max()),
            "note": "GPU output vs the oracle over the values before fp8/int8 storage (reported, not gated) "
                    "and over the stored codes (the kernel's own error)"}
    return res


ROOT = os.path.dirname(os.path.abspath(__file__))
DECODE_SOURCES = ("paged_kv_cache_263_amd/csrc/decode.hip", "paged_kv_cache_263_amd/csrc/device.h")
PROFILE_SUMMARY = "profiles/decode_kernel_llama8b_batch64.txt"
CALIBRATION_KERNEL = "__amd_rocclr_copyBuffer"


def sources_sha256(paths=DECODE_SOURCES) -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _read_csv(path):
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for base, _, files in os.walk(dirpath):
        for name in files:
            if name.endswith(suffix):
                return os.path.join(base, name)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def summarize_profile(trace_dir, fetch_dir, write_dir) -> str:
    """Markdown summary of a rocprofv3 run of this benchmark: kernel durations
    from --kernel-trace --stats, and HBM bytes per dispatch of the decode
    kernel from FETCH_SIZE / WRITE_SIZE (KiB), each scaled by the same
    counter's reading for the 1 GiB device copy run first (--calibrate-copy-mib
    1024), since on this part FETCH_SIZE under-counts reads of a plain copy."""
    lines = []
    stats = _read_csv(_find(trace_dir, "kernel_stats.csv"))
    lines.append("| kernel | calls | average (us) | min (us) | max (us) |")
    lines.append("|---|---|---|---|---|")
    for r in stats:
        name = r["Name"]
        if "pkv::" not in name:
            continue
        short = name.split("(anonymous namespace)::")[1].split("(")[0]
        lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _read_csv(_find(d, "counter_collection.csv"))
        calib = [float(r["Counter_Value"]) for r in rows
                 if r["Counter_Name"] == counter and CALIBRATION_KERNEL in r["Kernel_Name"]]
        cal_kib = max(calib) if calib else float("nan")
        scale = (1 << 20) / cal_kib  # the copy moves exactly 1 GiB each way
        vals = [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == counter and "decode_kernel" in r["Kernel_Name"]]
        per[counter] = (float(np.mean(vals)) if vals else float("nan"), cal_kib, scale, len(vals))
    fetch = per["FETCH_SIZE"][0] * per["FETCH_SIZE"][2] * 1024
    write = per["WRITE_SIZE"][0] * per["WRITE_SIZE"][2] * 1024
    lines.append("")
    lines.append("| counter | decode_kernel KiB / dispatch (mean of n) | 1 GiB copy reads | scale | bytes / dispatch |")
    lines.append("|---|---|---|---|---|")
    for counter, (v, cal, sc, n) in per.items():
        lines.append(f"| {counter} | {v:.1f} (n={n}) | {cal:.1f} KiB | {sc:.4f} | {v * sc * 1024:.4e} |")
    lines.append("")
    lines.append(f"hbm_traffic_bytes_per_launch: {fetch + write:.6e}")
    lines.append(f"fetch_bytes_per_launch: {fetch:.6e}")
    lines.append(f"write_bytes_per_launch: {write:.6e}")
    lines.append(f"source_sha256: {sources_sha256()}")
    return "\n".join(lines)


def recorded_traffic():
    """HBM bytes per launch of the decode kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, PROFILE_SUMMARY)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            k, _, v = line.partition(":")
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != sources_sha256():
        return None
    try:
        return float(vals["hbm_traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def elt_bytes(w) -> int:
    return {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}[w.kv_dtype]


def main():
    args = parse()
    if args.summarize_profile:
        print(summarize_profile(*args.summarize_profile))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU: the paged decode path has no multi-GPU "
                                   "mode (no sharding or collectives); run with --gpus 1"}))
        sys.exit(2)
    if args.workload == "prefix_cache":  # host allocator only
        print(json.dumps(run_prefix_cache(args)), flush=True)
        return
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    import paged_kv_cache_263_amd as pk

    device = "cuda"
    torch.cuda.set_device(0)
    if args.workload == "chunked":
        print(json.dumps(run_chunked(args, build_workload("chunked", args), device)), flush=True)
        return
    if args.workload == "swap":
        print(json.dumps(run_swap(args, device)), flush=True)
        return
    if args.calibrate_copy_mib:
        src = torch.ones(args.calibrate_copy_mib << 20, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = build_workload(args.workload, args)
    if args.placement == "identity":
        w.placement = np.arange(w.num_blocks, dtype=np.int32)
    pool, cache = setup(w, device)
    B = len(w.batch)
    seqs = list(w.batch)
    lens = np.array([pk.seq_len(pool, s) for s in seqs], dtype=np.int64)
    total = args.warmup + args.steps
    n_steps = total + max(0, args.cold_steps)
    max_blocks = int(math.ceil((lens.max() + n_steps) / 16)) + 1
    table_h, lens_h = pk.block_table_build(pool, seqs, max_blocks)
    d_table = table_h.to(device)
    d_lens = lens_h.to(device)
    q = __import__("workloads").queries(w, device)
    out = torch.empty_like(q)
    g = torch.Generator(device=device).manual_seed(w.seed + 5)
    k_new = torch.randn((n_steps, B, w.hkv, w.d), generator=g, device=device).to(cache.value_dtype)
    v_new = torch.randn((n_steps, B, w.hkv, w.d), generator=g, device=device).to(cache.value_dtype)
    d_rows = torch.arange(B, dtype=torch.int32, device=device)
    # slots and positions of every step, in pinned host memory that the cache
    # write kernel reads directly (one row per step, so no step overwrites
    # values an earlier, still queued step has yet to read)
    h_io = torch.empty((n_steps, 2, B), dtype=torch.int32).pin_memory()
    ones = [1] * B
    # workspace sized for the longest row the run reaches
    # shared_prefix: every table starts with the prefix's blocks (125 for 2000 tokens)
    spb = w.shared_prefix_tokens // 16 if (w.name == "shared_prefix" and not args.no_prefix_pass) else 0
    a = pk._args(cache, q, out, d_table, d_lens, int(lens.max()) + n_steps, 0, args.decode_parts, None)
    a.shared_prefix_blocks = spb
    ws = torch.empty(max(16, pk.paged_attn_workspace_size(cache, a)), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream()
    ev = TimingEvents(n_steps, 4)
    torch.cuda.synchronize()

    kv_bytes_step = []
    unique_bytes_step = []  # distinct KV bytes: a prefix every row shares counts once
    copies_total = 0
    shared_tokens = w.shared_prefix_tokens if w.name == "shared_prefix" else 0

    def step(i):
        nonlocal copies_total
        slots, copies = pk.seq_append_batch(pool, seqs, ones, out_slots=h_io[i, 0])
        if copies:
            pk.kv_copy_blocks(cache, copies)
            copies_total += len(copies)
        h_io[i, 1].copy_(torch.from_numpy(lens.astype(np.int32)))  # position of the new token
        lens[:] += 1
        # Timed steps carry only the two events around the decode kernel (its
        # roofline); warmup steps also time the cache write and the merge.
        breakdown = i < args.warmup
        if breakdown:
            ev.record(i, 0, stream)
        pk.kv_cache_write(cache, k_new[i], v_new[i], h_io[i, 0], rows=d_rows, positions=h_io[i, 1],
                          block_table=d_table, kv_lens=d_lens)
        pk.paged_attn_decode(cache, q, d_table, d_lens, int(lens.max()), out=out, decode_parts=args.decode_parts,
                             workspace=ws, events=ev.handles(i, (1, 2, 3) if breakdown else (1, 2)),
                             shared_prefix_blocks=spb)
        kv_bytes_step.append(int(lens.sum()) * w.hkv * w.d * 2 * elt_bytes(w))
        unique_bytes_step.append((int(lens.sum()) - (B - 1) * shared_tokens) * w.hkv * w.d * 2 * elt_bytes(w))

    row0 = None
    if w.kv_dtype in ("fp8", "int8") and not args.no_cpu_baseline:
        # batch row 0 before any token is appended, for the drift report of the oracle leg
        pk.paged_attn_decode(cache, q, d_table, d_lens, int(lens.max()), out=out, workspace=ws)
        torch.cuda.synchronize()
        row0 = out[0].float().cpu().numpy()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    host = 0.0
    for i in range(args.warmup, total):
        h0 = time.perf_counter()
        step(i)
        host += time.perf_counter() - h0
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # cold-cache steps (after the timed ones; not part of value): the last-level
    # cache holds a scratch buffer, not KV, when each step starts
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=device) if args.cold_steps > 0 else None
    if scratch is not None and args.cold_flush == "read":
        scratch.fill_(1)
        scratch.view(torch.int32).sum()
    for i in range(total, n_steps):
        if args.cold_flush == "write":
            scratch.fill_(i & 0xFF)
        else:
            scratch.view(torch.int32).sum()
        step(i)
    torch.cuda.synchronize()
    cold_ms = [ev.ms(i, 1, 2) for i in range(total, n_steps)]
    del scratch

    timed = range(args.warmup, total)
    split_ms = [ev.ms(i, 1, 2) for i in timed]  # decode kernel
    late_warmup = range(max(1, args.warmup - 5), args.warmup)  # the first (cold) call left out
    merge_ms = [ev.ms(i, 2, 3) for i in late_warmup]
    write_ms = [ev.ms(i, 0, 1) for i in late_warmup]  # cache write (+ plan kernel, if any)

    def us(v):
        return round(float(np.mean(v)) * 1e3, 2) if v else None

    bytes_timed = kv_bytes_step[args.warmup:total]
    unique_timed = unique_bytes_step[args.warmup:total]
    ms_per_step = dt * 1e3 / args.steps
    value = sum(bytes_timed) / dt / 1e9
    tokens_per_s = sum(b / (w.hkv * w.d * 2 * elt_bytes(w)) for b in bytes_timed) / dt
    split_avg_s = float(np.mean(split_ms)) / 1e3
    achieved = float(np.mean(unique_timed)) / split_avg_s / 1e9

    result = {
        "metric": "paged GQA decode: achieved HBM GB/s (KV bytes) + seq-tokens attended/s, 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_LABEL[w.kv_dtype],
        "data": "synthetic",
        "config": {"workload": describe(w), "batch": B, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d,
                   "block_size": 16, "mean_kv_len": round(float(np.mean(lens)), 1),
                   "pool_blocks": w.num_blocks, "decode_parts": args.decode_parts or "auto",
                   "placement": args.placement, "shared_prefix_blocks": spb},
        "seq_tokens_per_s": round(tokens_per_s, 1),
        "kernels_us": {"decode": us(split_ms), "decode_merge_warmup": us(merge_ms),
                       "cache_write_warmup": us(write_ms)},
        "decode_us_p10_p50_p90": [round(float(np.percentile(split_ms, q)) * 1e3, 2) for q in (10, 50, 90)],
        "decode_us_cold": us(cold_ms),
        "cold_flush": args.cold_flush if cold_ms else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic() if w.name == "llama8b" and not args.decode_parts else None,
                     "algorithmic_bytes_per_launch": float(np.mean(unique_timed)),
                     "kernel": "decode_kernel (distinct KV bytes of all rows per launch, a prefix all rows share counted once, / "
                               "event-timed duration of the decode kernel and any shared-prefix pass; traffic = "
                               "HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary)"},
        "copy_on_write_copies": copies_total,
        "host_us_per_step": round(host * 1e6 / args.steps, 1),
    }
    if not args.no_cpu_baseline:
        rows = args.cpu_sample_rows or {"llama8b": 64, "tiny": 4, "shared_prefix": 256, "fp8_long": 2,
                                        "int8_long": 2}[w.name]
        result["cpu_baseline"] = cpu_baseline(w, device, rows,
                                              single_core_s=5.0 if w.name in ("llama8b", "tiny") else 0.0,
                                              gpu_row0=row0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
