"""GPU test of paged_attn_decode_noalloc (the decode entry point that
allocates nothing: its workspace is the library's fixed per-GPU array),
through the C ABI: on consecutive calls, the second and later with smaller
inputs than the first, its output equals paged_attn_decode's bit for bit (same
kernels, same partition) and the oracle's within the bf16 tolerance; a call
needing more workspace than the array holds is refused before any launch."""

import numpy as np
import pytest
import torch

import workloads as W
from harness import TOL, HipSide, OracleSide, compare

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_noalloc_decode_matches_decode_on_consecutive_calls():
    import paged_kv_cache_263_amd as pk

    big = W.shared_prefix(variant="peaked")  # 256 rows, 64 / 8 heads: plan, partials and prefix states
    small = W.llama8b(batch=16, variant="peaked", seed=49)
    tiny = W.custom([1, 17, 300], 8, 2, "bf16", seed=53, variant="peaked")
    # 300 rows of 2-3 blocks after the 256-row call: the merge runs over the
    # decode wavefronts' records of the rows they began, and only ~93 of the
    # 128 wavefronts per kv head have a range, so the records past them still
    # hold the previous call's rows and must not be read (checked on every row)
    many = W.custom(np.random.default_rng(57).integers(17, 49, 300).tolist(), 64, 8, "bf16", seed=57,
                    variant="peaked")
    runs = [(big, 125), (small, 0), (tiny, 0), (big, 0), (many, 0)]
    for w, spb in runs:
        print(f"[case] noalloc {w.name} rows={len(w.batch)} shared_prefix_blocks={spb}", flush=True)
        hip = HipSide(w)
        need = pk.paged_attn_workspace_size(hip.cache, pk._args(hip.cache, hip.q, hip.q, hip.table, hip.kv_lens,
                                                                 hip.max_kv_len, 0, 0, None))
        assert need <= pk.NOALLOC_SCRATCH_BYTES
        want = hip.decode(shared_prefix_blocks=spb)
        out = torch.full_like(hip.q, float("nan"))
        got = pk.paged_attn_decode_noalloc(hip.cache, hip.q, hip.table, hip.kv_lens, hip.max_kv_len, out,
                                           shared_prefix_blocks=spb)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(out, want), f"{w.name}: differs from paged_attn_decode"
        orc = OracleSide(w)
        rows = list(range(len(w.batch))) if w is many else [0, len(w.batch) // 2, len(w.batch) - 1]
        ref = np.stack([orc.decode(b) for b in rows])
        compare(out[rows].float().cpu().numpy(), ref, TOL["bf16"], f"noalloc {w.name}")


def test_noalloc_decode_refuses_oversized_calls_and_workspaces():
    import paged_kv_cache_263_amd as pk

    w = W.fp8_long(batch=2, length=4096, variant="peaked")
    hip = HipSide(w)
    print("[case] noalloc refusals", flush=True)
    out = torch.zeros_like(hip.q)
    # 4096 wavefronts per kv head: 8 x 4096 x 2 x 8 partial states of 130 floats, above 64 MiB
    with pytest.raises(pk.PagedKVError) as e:
        pk.paged_attn_decode_noalloc(hip.cache, hip.q, hip.table, hip.kv_lens, hip.max_kv_len, out,
                                     decode_parts=4096)
    assert e.value.code == "WORKSPACE"
    a = pk._args(hip.cache, hip.q, out, hip.table, hip.kv_lens, hip.max_kv_len, 0, 0, None)
    a.workspace = out.data_ptr()
    a.workspace_bytes = 16
    st = pk._lib.paged_attn_decode_noalloc(pk.ctypes.byref(hip.cache.desc), pk.ctypes.byref(a),
                                           pk._stream(None))
    assert st == -1
    torch.cuda.synchronize()
    assert (out == 0).all()  # nothing was launched
    # and a call that fits still works after the refusals
    got = pk.paged_attn_decode_noalloc(hip.cache, hip.q, hip.table, hip.kv_lens, hip.max_kv_len, out)
    want = hip.decode()
    torch.cuda.synchronize()
    assert torch.equal(got, want)
