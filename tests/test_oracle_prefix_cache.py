"""Pins for the oracle's prefix cache with retention (oracle.pool): the hash
against FNV-1a's published test vectors, a script worked out by hand from the
documented policy, and invariants after every step of random request streams
whose token ids are written through the slots (so that a match can be checked
against the bytes it shares)."""

import random

import pytest

from oracle import pool as P


def test_fnv1a64_published_vectors():
    assert P.fnv1a64(b"") == 0xCBF29CE484222325
    assert P.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert P.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_block_key_is_a_chain():
    t = list(range(16))
    k0 = P.block_key(0, 1, t)
    assert k0 == P.fnv1a64(bytes(8) + (1).to_bytes(4, "little") + b"".join(i.to_bytes(4, "little") for i in t))
    assert P.block_key(k0, 1, t) != k0                  # the parent is part of the key
    assert P.block_key(0, 2, t) != k0                   # so is the tenant
    assert P.block_key(0, 1, t[::-1]) != k0             # and the order of the ids


def test_hand_worked_script():
    pool = P.PoolModel(8)
    prompt = list(range(100, 140))                      # 40 tokens: 2 full blocks + 8
    a, m = pool.create_cached(1, prompt)
    assert m == 0 and pool.seq_blocks(a) == []
    pool.append(a, 40)                                   # blocks 0, 1, 2
    assert pool.cache_tokens(a, 0, prompt) == 2          # blocks 0 and 1 keyed and registered
    assert pool.stats()["cached_blocks"] == 2
    pool.seq_free(a)                                     # 0, 1 retained (1 listed oldest), 2 freed
    assert pool.evictable == [1, 0] and pool.free_stack == [7, 6, 5, 4, 3, 2]
    b, m = pool.create_cached(1, prompt[:35])            # same 32 leading tokens, 3 left
    assert m == 32 and pool.seq_blocks(b) == [0, 1] and pool.evictable == [] and pool.ref[:2] == [1, 1]
    c, m = pool.create_cached(2, prompt[:35])            # another tenant never matches
    assert m == 0
    d, m = pool.create_cached(1, prompt[:32])            # at most 31 tokens may match: one block
    assert m == 16 and pool.seq_blocks(d) == [0] and pool.ref[0] == 2
    e, m = pool.create_cached(1, prompt[:16] + [7] * 20)  # second block differs
    assert m == 16
    st = pool.stats()
    assert st["matched_tokens"] == 32 + 16 + 16 and st["evictable_blocks"] == 0
    for s in (b, c, d, e):
        pool.seq_free(s)
    assert pool.evictable == [1, 0] and pool.ref == [0] * 8
    f = pool.seq_create()
    pool.append(f, 16 * 7)                               # the 6 free blocks, then the oldest retained one
    assert pool.seq_blocks(f) == [2, 3, 4, 5, 6, 7, 1]
    assert pool.evictable == [0] and pool.stats()["cached_blocks"] == 1   # block 1's entry went with it
    g, m = pool.create_cached(1, prompt)                 # block 0 still matches, block 1 no longer
    assert m == 16 and pool.seq_blocks(g) == [0]
    with pytest.raises(P.InvalidArgument):               # must start at the first unkeyed block
        pool.cache_tokens(g, 0, prompt[:16])
    with pytest.raises(P.OutOfBlocks):                   # nothing left: the pool is full
        pool.append(g, 17)


class Traffic:
    """Requests drawn from a few prompt families (shared beginnings of
    different lengths) plus random tails, for two tenants."""

    def __init__(self, rng):
        self.rng = rng
        self.families = [[rng.randrange(1000) for _ in range(n)] for n in (8, 40, 64, 100)]

    def prompt(self):
        fam = self.rng.choice(self.families)
        cut = len(fam) if self.rng.random() < 0.5 else self.rng.randrange(len(fam) + 1)
        return fam[:cut] + [self.rng.randrange(1000) for _ in range(self.rng.choice([1, 5, 16, 30]))]


def check(pool, streams):
    N = pool.num_blocks
    count = [0] * N
    for q in pool.seqs.values():
        for b in q.blocks:
            count[b] += 1
    assert count == pool.ref
    free, ev = set(pool.free_stack), set(pool.evictable)
    assert len(free) == len(pool.free_stack) and len(ev) == len(pool.evictable) and not free & ev
    assert len(free) + len(ev) + sum(1 for r in pool.ref if r > 0) == N
    assert all(pool.ref[b] == 0 and b in pool.key_of for b in ev)
    assert not free & set(pool.key_of)
    for key, e in pool.cache.items():
        assert pool.key_of[e.block] == key
    for s, q in pool.seqs.items():
        if not q.swapped:
            assert len(q.blocks) == -(-q.length // 16) and len(q.keys) <= len(q.blocks)
    # content: every entry's block holds its tokens; every sequence reads back its stream
    store = streams["store"]
    for e in pool.cache.values():
        assert list(store.gather([e.block], 16)) == list(e.tokens)
    for s, toks in streams["seq"].items():
        if s in pool.seqs and not pool.seqs[s].swapped:
            assert list(store.gather(pool.seq_blocks(s), len(toks))) == toks if toks else True


def random_step(pool, streams, traffic, rng):
    store = streams["store"]
    resident = [s for s, q in pool.seqs.items() if not q.swapped]
    kind = rng.choice(["request", "request", "decode", "decode", "register", "free", "free", "fork", "swap"])
    try:
        if kind == "request" or not resident:
            tenant = rng.choice([1, 2])
            prompt = traffic.prompt()
            s, m = pool.create_cached(tenant, prompt)
            assert m % 16 == 0 and m <= len(prompt) - 1
            streams["seq"][s] = list(prompt[:m])
            slots, copies = pool.append(s, len(prompt) - m)
            assert not copies
            store.write(slots, prompt[m:])
            streams["seq"][s] = list(prompt)
            pool.cache_tokens(s, m, prompt[m:])
        elif kind == "decode":
            s = rng.choice(resident)
            n = rng.choice([1, 3, 16])
            slots, copies = pool.append(s, n)
            for c in copies:
                store.copy_block(c)
            new = [rng.randrange(1000) for _ in range(n)]
            store.write(slots, new)
            streams["seq"][s] += new
        elif kind == "register":
            s = rng.choice(resident)
            k = 16 * len(pool.seqs[s].keys)
            pool.cache_tokens(s, k, streams["seq"][s][k:])
        elif kind == "fork":
            s = rng.choice(resident)
            c = pool.fork(s)
            streams["seq"][c] = list(streams["seq"][s])
        elif kind == "swap":
            s = rng.choice(resident)
            ids = pool.swap_out(s)
            host = list(store.gather(ids, pool.seq_len(s))) if ids else []
            new = pool.swap_in(s)
            store.write([new[t // 16] * 16 + t % 16 for t in range(len(host))], host)
        else:
            s = rng.choice(list(pool.seqs))
            pool.seq_free(s)
            streams["seq"].pop(s, None)
    except P.OutOfBlocks:
        pass


@pytest.mark.parametrize("seed", range(10))
def test_random_request_streams_keep_invariants(seed):
    import numpy as np

    rng = random.Random(seed)
    n = rng.choice([12, 24, 48])
    pool = P.PoolModel(n, order=rng.sample(range(n), n))
    streams = {"store": P.TokenStore(n, (), np.int64), "seq": {}}
    traffic = Traffic(rng)
    hits = 0
    for _ in range(400):
        before = pool.stats()["matched_tokens"]
        random_step(pool, streams, traffic, rng)
        hits += pool.stats()["matched_tokens"] > before
        check(pool, streams)
    assert hits > 0
