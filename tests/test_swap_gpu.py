"""GPU checks of swapping blocks to pinned host memory and back (through the
C ABI): the host copy holds each block's bytes in the documented slot layout,
and a sequence swapped out, its blocks reused by another sequence, then swapped
back into different blocks decodes to the same bits as before, which match the
oracle within the cache dtype's tolerance."""

import numpy as np
import pytest
import torch

import workloads as W
from harness import TOL, HipSide, OracleSide, compare

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def case(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("kv,layers", [("bf16", 1), ("bf16", 2), ("int8", 1), ("fp8", 2)])
def test_swap_round_trip_is_bit_exact(kv, layers):
    import paged_kv_cache_263_amd as pk

    case(f"swap round trip kv={kv} layers={layers}")
    w = W.custom([100, 700, 40, 2000], 8, 2, kv, seed=91, variant="peaked", pool_factor=2.0)
    hip = HipSide(w, layer=layers - 1, num_layers=layers)
    before = hip.decode().clone()
    row = 1
    torch.cuda.synchronize()
    compare(before[[row]].float().cpu().numpy(), np.stack([OracleSide(w).decode(row)]), TOL[kv],
            f"swap kv={kv}: row {row} before the swap")
    seq = w.batch[row]
    ids = pk.seq_swap_out(hip.pool, seq)
    assert len(ids) == -(-700 // 16)
    slot = pk.kv_swap_block_bytes(hip.cache)
    host = torch.empty(len(ids) * slot, dtype=torch.uint8).pin_memory()
    pk.kv_swap_out(hip.cache, ids, host)
    torch.cuda.synchronize()
    # the host slots hold the blocks' bytes: [layer][K, V][kv heads' tiles]
    kb = hip.cache.k_pool.view(torch.uint8).cpu().numpy().reshape(layers, w.num_blocks, -1)
    vb = hip.cache.v_pool.view(torch.uint8).cpu().numpy().reshape(layers, w.num_blocks, -1)
    hb = host.numpy().reshape(len(ids), layers, 2, -1)
    for i, b in enumerate(ids):
        for layer in range(layers):
            assert np.array_equal(hb[i, layer, 0], kb[layer, b]) and np.array_equal(hb[i, layer, 1], vb[layer, b])
    # another sequence takes the freed blocks and overwrites them
    other = pk.seq_create(hip.pool)
    n_other = 16 * len(ids)
    slots, copies = pk.seq_append(hip.pool, other, n_other)
    assert not copies and {s // 16 for s in slots} >= set(ids)
    g = torch.Generator(device="cuda").manual_seed(5)
    vals = torch.randn((n_other, w.hkv, 128), generator=g, device="cuda").to(hip.cache.value_dtype)
    pk.kv_cache_write(hip.cache, vals, vals, torch.tensor(slots, dtype=torch.int32, device="cuda"),
                      layer=layers - 1)
    new_ids = pk.seq_swap_in(hip.pool, seq)
    assert len(new_ids) == len(ids) and not set(new_ids) & set(ids)
    pk.kv_swap_in(hip.cache, host, new_ids)
    table, lens = pk.block_table_build(hip.pool, w.batch, hip.max_blocks)
    assert table[row, : len(new_ids)].tolist() == new_ids
    out = pk.paged_attn_decode(hip.cache, hip.q, table.cuda(), lens.cuda(), hip.max_kv_len, layer=layers - 1)
    torch.cuda.synchronize()
    # the partition depends on the lengths only, so placement changes no bit
    assert torch.equal(out, before)


def test_swap_needs_pinned_memory_and_valid_ids():
    import paged_kv_cache_263_amd as pk

    case("swap argument checks")
    w = W.custom([40], 8, 2, "bf16", seed=92)
    hip = HipSide(w)
    ids = pk.seq_swap_out(hip.pool, w.batch[0])
    slot = pk.kv_swap_block_bytes(hip.cache)
    with pytest.raises(pk.PagedKVError) as e:
        pk.kv_swap_out(hip.cache, ids, torch.empty(len(ids) * slot, dtype=torch.uint8))  # not pinned
    assert e.value.code == "INVALID"
    host = torch.empty(len(ids) * slot, dtype=torch.uint8).pin_memory()
    with pytest.raises(pk.PagedKVError):
        pk.kv_swap_out(hip.cache, [w.num_blocks], host[:slot])  # id out of range
    with pytest.raises(pk.PagedKVError):
        pk.kv_swap_in(hip.cache, host, [ids[0], ids[0]])  # duplicate destination
    torch.cuda.synchronize()
