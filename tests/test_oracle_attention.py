"""Pins for the oracle's attention (oracle.attention), against things other
than itself: torch's scaled_dot_product_attention (the textbook definition,
float64 on the CPU, with its own grouped-query broadcast), closed forms, and
invariants the pages state (paging and chunking change no result)."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import pool as P


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def sdpa(q, K, V, causal=False):
    """q [C, Hq, d]; K, V [L, Hkv, d] -> [C, Hq, d] via torch (float64)."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("hq,hkv,L,scale", [(8, 2, 37, 1.0), (4, 4, 5, 4.0), (8, 1, 70, 4.0), (32, 8, 129, 1.0)])
def test_decode_matches_sdpa(hq, hkv, L, scale):
    d = 128 if hq != 32 else 64
    q = rnd((hq, d), 1, scale)
    K, V = rnd((L, hkv, d), 2), rnd((L, hkv, d), 3)
    ref = sdpa(q[None], K, V)[0]
    np.testing.assert_allclose(A.decode(q, K, V), ref, rtol=0, atol=1e-12)


def test_prefill_without_context_matches_causal_sdpa():
    C, hq, hkv, d = 23, 8, 2, 32
    q = rnd((C, hq, d), 4, 2.0)
    K, V = rnd((C, hkv, d), 5), rnd((C, hkv, d), 6)
    np.testing.assert_allclose(A.prefill_chunk(q, K, V), sdpa(q, K, V, causal=True), rtol=0, atol=1e-12)


def test_chunk_rows_equal_whole_prefill_rows():
    """A chunk is the last C queries of one causal prefill over all L tokens."""
    L, C, hq, hkv, d = 41, 9, 4, 2, 16
    qf = rnd((L, hq, d), 7, 2.0)
    K, V = rnd((L, hkv, d), 8), rnd((L, hkv, d), 9)
    whole = sdpa(qf, K, V, causal=True)
    np.testing.assert_allclose(A.prefill_chunk(qf[L - C:], K, V), whole[L - C:], rtol=0, atol=1e-12)


def test_chunking_changes_nothing_and_last_row_is_decode():
    L, hq, hkv, d = 50, 8, 2, 32
    qf = rnd((L, hq, d), 10, 3.0)
    K, V = rnd((L, hkv, d), 11), rnd((L, hkv, d), 12)
    one = A.prefill_chunk(qf[30:], K, V)  # one chunk of 20 over 30 of context
    a = A.prefill_chunk(qf[30:42], K[:42], V[:42])  # two chunks 12 + 8
    b = A.prefill_chunk(qf[42:], K, V)
    np.testing.assert_allclose(np.concatenate([a, b]), one, rtol=0, atol=1e-13)
    np.testing.assert_allclose(one[-1], A.decode(qf[-1], K, V), rtol=0, atol=1e-13)


def test_closed_forms():
    hq, hkv, d = 8, 2, 16
    K, V = rnd((9, hkv, d), 13), rnd((9, hkv, d), 14)
    q = rnd((hq, d), 15)
    # one cached token: the output is that token's value row, exactly
    o = A.decode(q, K[:1], V[:1])
    for h in range(hq):
        assert np.array_equal(o[h], V[0, h // 4])
    # a zero query weighs every token equally: the mean of V
    o = A.decode(np.zeros((hq, d)), K, V)
    for h in range(hq):
        np.testing.assert_allclose(o[h], V[:, h // 4].mean(0), rtol=0, atol=1e-14)
    # a constant V gives that constant
    Vc = np.full_like(V, 0.375)
    np.testing.assert_allclose(A.decode(q, K, Vc), 0.375, rtol=0, atol=1e-15)


def test_gqa_is_mha_on_repeated_kv_and_token_order_is_irrelevant():
    hq, hkv, d, L = 8, 2, 16, 33
    q = rnd((hq, d), 16)
    K, V = rnd((L, hkv, d), 17), rnd((L, hkv, d), 18)
    Kr, Vr = np.repeat(K, hq // hkv, axis=1), np.repeat(V, hq // hkv, axis=1)
    np.testing.assert_allclose(A.decode(q, K, V), A.decode(q, Kr, Vr), rtol=0, atol=1e-14)
    perm = np.random.default_rng(19).permutation(L)
    np.testing.assert_allclose(A.decode(q, K[perm], V[perm]), A.decode(q, K, V), rtol=0, atol=1e-13)


def test_brute_force_loops_tiny():
    """Per-token loops with math.exp and an explicit max, on tiny shapes."""
    import math

    hq, hkv, d, L = 4, 2, 8, 11
    q = rnd((hq, d), 20, 2.0)
    K, V = rnd((L, hkv, d), 21), rnd((L, hkv, d), 22)
    out = A.decode(q, K, V)
    for h in range(hq):
        j = h * hkv // hq
        s = [sum(q[h, i] * K[t, j, i] for i in range(d)) / math.sqrt(d) for t in range(L)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        for i in range(d):
            ref = sum(w[t] * V[t, j, i] for t in range(L)) / sum(w)
            assert abs(out[h, i] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_paging_changes_nothing():
    """Values written through a shuffled pool and read back through the block
    table give the same attention output bit for bit as the contiguous arrays."""
    hq, hkv, d = 8, 2, 16
    lens = [3, 16, 17, 40]
    rng = np.random.default_rng(23)
    pool = P.PoolModel(20, order=list(rng.permutation(20)))
    store = P.TokenStore(20, (2, hkv, d), np.float64)
    kv = {}
    for L in lens:
        s = pool.seq_create()
        K, V = rnd((L, hkv, d), 100 + L), rnd((L, hkv, d), 200 + L)
        slots, _ = pool.append(s, L)
        store.write(slots, np.stack([K, V], 1))
        kv[s] = (K, V)
    rows, L_ = pool.block_table(list(kv), 4)
    for s, (K, V) in kv.items():
        got = store.gather(rows[s], L_[s])
        q = rnd((hq, d), 300 + s, 3.0)
        assert np.array_equal(A.decode(q, got[:, 0], got[:, 1]), A.decode(q, K, V))


def test_rejects():
    with pytest.raises(ValueError):
        A.decode(np.zeros((4, 8)), np.zeros((0, 2, 8)), np.zeros((0, 2, 8)))
    with pytest.raises(ValueError):
        A.decode(np.zeros((3, 8)), np.zeros((2, 2, 8)), np.zeros((2, 2, 8)))


def test_prefill_rows_are_chunk_rows():
    L, C, hq, hkv, d = 45, 12, 8, 2, 16
    q = rnd((C, hq, d), 30, 2.0)
    K, V = rnd((L, hkv, d), 31), rnd((L, hkv, d), 32)
    full = A.prefill_chunk(q, K, V)
    rows = [0, 5, 11]
    np.testing.assert_allclose(A.prefill_rows(q, K, V, rows), full[rows], rtol=0, atol=1e-13)


@pytest.mark.parametrize("hq,hkv,L,scale", [(8, 2, 37, 1.0), (4, 4, 5, 4.0), (8, 1, 70, 4.0), (32, 8, 129, 1.0),
                                            (12, 2, 50, 4.0), (6, 3, 17, 2.0)])
def test_decode_rows_matches_sdpa_and_decode(hq, hkv, L, scale):
    """decode_rows (the sampled-head form every GPU decode comparison uses)
    gives the listed heads of torch SDPA's grouped-query attention and of
    decode, for head lists in any order, with repeats, across every kv head."""
    d = 128 if hq != 32 else 64
    q = rnd((hq, d), 41, scale)
    K, V = rnd((L, hkv, d), 42), rnd((L, hkv, d), 43)
    ref = sdpa(q[None], K, V)[0]
    full = A.decode(q, K, V)
    rng = np.random.default_rng(44)
    for heads in (list(range(hq)), list(range(hq))[::-1], rng.integers(0, hq, 7).tolist(), [hq - 1, 0, hq - 1]):
        got = A.decode_rows(q, K, V, heads)
        assert got.shape == (len(heads), d)
        np.testing.assert_allclose(got, ref[heads], rtol=0, atol=1e-12)
        np.testing.assert_allclose(got, full[heads], rtol=0, atol=1e-13)


def test_decode_rows_kv_head_of_each_query_head():
    """Each query head reads kv head h // G: with V constant per kv head
    (value j + 1 for kv head j), head h's output is exactly h // G + 1."""
    hq, hkv, d, L = 12, 3, 16, 9
    q = rnd((hq, d), 45, 3.0)
    K = rnd((L, hkv, d), 46)
    V = np.empty((L, hkv, d))
    for j in range(hkv):
        V[:, j, :] = j + 1.0
    heads = [11, 0, 4, 7, 8, 3]
    got = A.decode_rows(q, K, V, heads)
    for n, h in enumerate(heads):
        np.testing.assert_allclose(got[n], h // (hq // hkv) + 1.0, rtol=0, atol=1e-14)
