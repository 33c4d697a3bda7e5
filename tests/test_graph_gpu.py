"""HIP graph capture of the attention calls (through torch's graph API).  A
decode or chunked-prefill call captured once and replayed gives the eager
call's output bit for bit on every replay, with the program's own eager work
and synchronisations between the replays.  The calls enqueue only kernels on
the caller's stream (no allocation, copy or memset inside), with the workspace
given by the caller or, for paged_attn_decode_noalloc, the library's fixed
array.  Covered: the per-row merge, the one-launch shared-prefix pass and its
merge, the merge over the decode wavefronts' records (more rows than
wavefronts), the plan kernel (more than 1024 rows) and a chunked-prefill call
with decode rows and key ranges."""

import numpy as np
import pytest
import torch

import workloads as W
from harness import HipSide

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REPLAYS = 4


def replays_match(call, out, want):
    """Capture call() (which writes out) after an eager warm-up on a side
    stream, then replay it REPLAYS times, clearing out eagerly before each."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(out, want), "eager warm-up differs from the reference call"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r} differs from the eager call"


def short_rows(n, lo, hi, seed, hq=64, hkv=8):
    lens = np.random.default_rng(seed).integers(lo, hi + 1, n).tolist()
    return W.custom(lens, hq, hkv, "bf16", seed=seed, variant="peaked")


@pytest.mark.parametrize("case", ["rows_16", "shared_prefix", "rows_300_short"])
def test_noalloc_decode_graph_replays_match_eager(case):
    import paged_kv_cache_263_amd as pk

    w, spb = {"rows_16": lambda: (W.llama8b(batch=16, variant="peaked", seed=61), 0),
              "shared_prefix": lambda: (W.shared_prefix(variant="peaked"), 125),
              "rows_300_short": lambda: (short_rows(300, 17, 48, 63), 0)}[case]()
    print(f"[case] graph noalloc decode {case}", flush=True)
    hip = HipSide(w)
    want = hip.decode(shared_prefix_blocks=spb)
    out = torch.empty_like(hip.q)
    replays_match(lambda: pk.paged_attn_decode_noalloc(hip.cache, hip.q, hip.table, hip.kv_lens, hip.max_kv_len,
                                                       out, shared_prefix_blocks=spb), out, want)


def test_decode_with_caller_workspace_graph_replays_match_eager():
    """1100 rows: above the in-kernel plan's 1024, so the plan kernel runs too."""
    import paged_kv_cache_263_amd as pk

    print("[case] graph decode 1100 rows, caller workspace", flush=True)
    hip = HipSide(short_rows(1100, 1, 96, 65, hq=8, hkv=2))
    want = hip.decode()
    out = torch.empty_like(hip.q)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=hip.q.device)
    replays_match(lambda: pk.paged_attn_decode(hip.cache, hip.q, hip.table, hip.kv_lens, hip.max_kv_len, out=out,
                                               workspace=ws), out, want)


def test_prefill_chunk_graph_replays_match_eager():
    import paged_kv_cache_263_amd as pk

    print("[case] graph prefill chunk", flush=True)
    w = W.chunks([(50, 70), (30, 40), (0, 33)], hq=8, hkv=2, n_decode=2, variant="peaked", seed=29)
    hip = HipSide(w)
    cu = [0]
    for n in w.q_lens:
        cu.append(cu[-1] + n)
    nd = 0
    while nd < len(w.q_lens) and w.q_lens[nd] == 1:
        nd += 1
    cu_q = torch.tensor(cu, dtype=torch.int32, device=hip.q.device)
    mdl = max(hip.lens[:nd]) if nd else 0
    mq = max(w.q_lens[nd:])
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=hip.q.device)

    def call(out=None, parts=3):
        return pk.paged_attn_prefill_chunk(hip.cache, hip.q, cu_q, hip.table, hip.kv_lens, hip.max_kv_len, nd, mq,
                                           out=out, max_decode_kv_len=mdl, workspace=ws, prefill_parts=parts)

    want = call().clone()
    out = torch.empty_like(hip.q)
    replays_match(lambda: call(out), out, want)
