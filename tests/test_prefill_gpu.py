"""GPU parity of chunked prefill batched with decode rows (through the C ABI)
against the fp64 oracle (max abs error 2e-2 for bf16 and int8 caches, 6e-2
for an fp8 cache)."""

import numpy as np
import pytest
import torch

import workloads as W
from harness import TOL, HipSide, OracleSide, compare, q_offsets

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def check_prefill(w, tokens=None, heads=None, hip=None, parts=0):
    print(f"[case] {w.name} variant={w.variant} kv={w.kv_dtype} q_lens={w.q_lens[:6]}... hq={w.hq} hkv={w.hkv} "
          f"prefill_parts={parts}", flush=True)
    hip = hip or HipSide(w)
    out = hip.prefill(prefill_parts=parts)
    torch.cuda.synchronize()
    orc = OracleSide(w)
    otable, olens = orc.pool.block_table(w.batch, hip.max_blocks)
    assert hip.table_host.tolist() == otable and hip.lens == olens
    heads = list(range(w.hq)) if heads is None else list(heads)
    off = q_offsets(w)
    got, ref = [], []
    for row, n in enumerate(w.q_lens):
        if n == 1 and (row == 0 or w.q_lens[row - 1] == 1):
            got.append(out[off[row]][heads].float().cpu().numpy()[None])
            ref.append(orc.decode(row, heads)[None])
        else:
            toks = list(range(n)) if tokens is None else [t for t in tokens if t < n]
            got.append(out[[off[row] + t for t in toks]][:, heads].float().cpu().numpy())
            ref.append(orc.chunk_rows(row, toks, heads))
    compare(np.concatenate(got), np.concatenate(ref), TOL[w.kv_dtype], f"{w.name}/{w.variant}")
    return hip, out


SMALL = [(0, 17), (5, 16), (100, 33), (0, 1), (1000, 64), (37, 200), (16, 15)]


@pytest.mark.parametrize("parts", [0, 1, 4])
@pytest.mark.parametrize("variant", ["plain", "peaked"])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
def test_small_chunks_with_decode_rows(kv, variant, parts):
    """Short chunks (1 to 200 queries over 0 to 1000 tokens of context) with
    decode rows; each query tile whole (parts = 1), or its keys split into
    ranges merged afterwards (auto: 3 here; 4), so that some ranges lie wholly
    past a query's diagonal or hold no iteration."""
    w = W.chunks(SMALL, hq=8, hkv=2, kv_dtype=kv, n_decode=3, variant=variant)
    check_prefill(w, parts=parts)


# group sizes G = Hq / Hkv: 8, 1, 16, 4, and the ones whose tiles leave rows
# unused (128 / G not whole: G = 3, 5, 6) or hold 64 tokens (G = 2)
@pytest.mark.parametrize("hq,hkv", [(64, 8), (4, 4), (16, 1), (12, 3), (4, 2), (6, 2), (10, 2), (12, 2)])
def test_group_sizes(hq, hkv):
    check_prefill(W.chunks([(50, 70), (0, 33)], hq=hq, hkv=hkv, n_decode=2, variant="peaked", seed=13))


# sampled chunk tokens: tile and block edges, the first and last query
CHUNK_TOKENS = [0, 1, 15, 16, 17, 63, 64, 65, 511, 512, 777, 1000, 1022, 1023]


def chunked_workload(context, kv):
    w = W.chunked(context=context)
    if kv == "fp8":
        w = W.scaled_fp8(w)
    elif kv == "int8":
        w = W.scaled_int8(w)
    w.variant = "peaked"
    return w


@pytest.mark.parametrize("kv,parts", [("bf16", 0), ("fp8", 0), ("int8", 0), ("bf16", 3)])
def test_chunked_1024_over_16k_context_with_32_decodes(kv, parts):
    check_prefill(chunked_workload(16384, kv), tokens=CHUNK_TOKENS, parts=parts)


@pytest.mark.parametrize("chunk,hq", [(512, 64), (1024, 32), (512, 32)])
def test_chunk_split_over_key_ranges_at_64k(chunk, hq):
    """Launches with fewer query tiles than compute units (a 512-query chunk
    at eight or four heads per kv head, or a 1024-query chunk at four) split
    every tile's 64K context into key ranges and merge them."""
    w = W.chunked(context=65536, chunk=chunk, hq=hq)
    w.variant = "peaked"
    check_prefill(w, tokens=[t for t in CHUNK_TOKENS if t < chunk])


@pytest.mark.parametrize("context,kv", [(32768, "bf16"), (65536, "bf16"), (131072, "bf16"), (65536, "fp8")])
def test_chunked_1024_over_long_context_with_32_decodes(context, kv):
    """The 1024-token chunk over 32K, 64K and 128K tokens of context (the
    rest of the 16K-128K sweep), all 64 heads of the sampled tokens and of
    every decode row."""
    check_prefill(chunked_workload(context, kv), tokens=CHUNK_TOKENS)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (64, 8)])
def test_row_with_more_queries_than_max_q_len_is_nan(hq, hkv):
    """A chunk row holding more queries than the stated max_q_len is invalid:
    all its outputs are NaN, also past the last tile the launch covers; the
    other rows are unaffected."""
    import paged_kv_cache_263_amd as pk

    w = W.chunks([(50, 70), (30, 40), (0, 33)], hq=hq, hkv=hkv, n_decode=2, variant="peaked", seed=29)
    hip = HipSide(w)
    cu = torch.tensor(q_offsets(w), dtype=torch.int32, device="cuda")
    out = torch.zeros_like(hip.q)
    print(f"[case] over-long chunk row hq={hq} hkv={hkv}", flush=True)
    # the first chunk row (70 queries) breaks the bound; the other two fit
    pk.paged_attn_prefill_chunk(hip.cache, hip.q, cu, hip.table, hip.kv_lens, hip.max_kv_len, 2, 40, out=out,
                                max_decode_kv_len=max(hip.lens[:2]))
    torch.cuda.synchronize()
    off = q_offsets(w)
    assert torch.isnan(out[off[2]:off[3]].float()).all()
    orc = OracleSide(w)
    for row in (0, 1):
        compare(out[off[row]].float().cpu().numpy(), orc.decode(row), TOL["bf16"], f"decode row {row}")
    for row in (3, 4):
        n = w.q_lens[row]
        compare(out[off[row]:off[row] + n].float().cpu().numpy(), orc.chunk_rows(row, list(range(n))),
                TOL["bf16"], f"chunk row {row}")


def test_last_chunk_row_matches_decode():
    """The last query of a chunk sees the whole sequence: same result as a
    decode step over it (both through the library)."""
    import paged_kv_cache_263_amd as pk

    w = W.chunks([(300, 50)], hq=8, hkv=2, n_decode=0, variant="peaked", seed=17)
    hip = HipSide(w)
    out = hip.prefill()
    q_last = hip.q[-1:].contiguous()
    dec = pk.paged_attn_decode(hip.cache, q_last, hip.table, hip.kv_lens, hip.max_kv_len)
    torch.cuda.synchronize()
    d = (out[-1].float() - dec[0].float()).abs().max().item()
    print(f"last row vs decode: {d:.3e}", flush=True)
    assert d <= 2 * TOL["bf16"]


def test_prefill_is_deterministic_and_placement_invariant():
    w = W.chunks([(200, 100), (0, 64)], hq=16, hkv=2, n_decode=2, variant="peaked", seed=19)
    a = HipSide(w).prefill()
    b = HipSide(w, placement=W.placement(w.num_blocks, 1234)).prefill()
    c = HipSide(w).prefill()
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_unwritten_slots_hold_nan(kv):
    w = W.chunks([(5, 16), (100, 33), (0, 1)], hq=8, hkv=2, kv_dtype=kv, n_decode=2, variant="peaked", seed=23)
    check_prefill(w, hip=HipSide(w, fill_byte=0xFF))
