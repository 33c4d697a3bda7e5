"""Pins for the oracle's allocator model (oracle.pool): hand-worked fixtures,
the pages' closed forms, and the invariants the pages state, checked after
every operation of random and of exhaustively enumerated scripts."""

import itertools
import json
import os
import random

import pytest

from oracle import pool as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ids(spec: str) -> list:
    out = []
    for part in filter(None, spec.split(",")):
        if ".." in part:
            a, b = part.split("..")
            out += list(range(int(a), int(b) + 1))
        else:
            out.append(int(part))
    return out


def order_of(spec: str, n: int):
    if spec == "identity":
        return None
    out = []
    for part in spec.split(" then "):
        a, b = part.split("..")
        out += list(range(int(a), int(b) + 1))
    assert sorted(out) == list(range(n))
    return out


def run_golden(make_pool, script):
    pool = make_pool(script["num_blocks"], order_of(script["order"], script["num_blocks"]))
    for step in script["ops"]:
        op = step["op"]
        if op == "check":
            for s, spec in step.get("tables", {}).items():
                assert pool.seq_blocks(int(s)) == ids(spec), (script["name"], step)
            for spec, r in step.get("refs", {}).items():
                for b in ids(spec):
                    assert pool.ref[b] == r, (script["name"], b)
            for s, L in step.get("lens", {}).items():
                assert pool.seq_len(int(s)) == L
            st = pool.stats()
            for k, v in step.get("stats", {}).items():
                assert st[k] == v, (script["name"], k, st[k], v)
            continue
        err = step.get("expect_error")
        try:
            if op == "create":
                got = pool.seq_create()
            elif op == "append":
                got = pool.append(step["seq"], step["n"])
            elif op == "fork":
                got = pool.fork(step["seq"])
            elif op == "share_prefix":
                got = pool.share_prefix(step["seq"], step["n"])
            elif op == "free_seq":
                got = pool.seq_free(step["seq"])
            else:
                raise AssertionError(op)
        except P.PoolError as e:
            assert err == e.code, (script["name"], step, e)
            continue
        assert err is None, (script["name"], step)
        if "expect_seq" in step:
            assert got == step["expect_seq"]
        if op == "append":
            slots, copies = got
            if "expect_slots" in step:
                assert slots == step["expect_slots"]
            if "expect_slots_range" in step:
                a, b = step["expect_slots_range"]
                assert slots == list(range(a, b))
            assert [[c.src, c.dst, c.valid_tokens] for c in copies] == step["expect_copies"]


def test_golden_scripts():
    data = json.load(open(os.path.join(GOLDEN, "alloc_scripts.json")))
    for script in data["scripts"]:
        run_golden(lambda n, order: P.PoolModel(n, order=order), script)


def test_block_counts_closed_forms():
    # [P2] contiguous example lengths; [P3] 500 tokens -> 32 ids; 2000 tokens -> 125 blocks
    pool = P.PoolModel(1000)
    seqs = []
    for L in [300, 2000, 600, 4400]:
        s = pool.seq_create()
        pool.append(s, L)
        seqs.append(s)
    assert [len(pool.seq_blocks(s)) for s in seqs] == [19, 125, 38, 275]
    st = pool.stats()
    assert st["used_blocks"] == 457 and st["waste_tokens"] == 4 + 0 + 8 + 0
    s = pool.seq_create()
    pool.append(s, 500)
    assert len(pool.seq_blocks(s)) == 32


def test_kv_bytes_closed_forms():
    """Byte facts printed on the pages, from the size formula of [P3] 'KV cache
    memory math'.  Fixture values with citations in tests/golden/kv_bytes.json."""
    data = json.load(open(os.path.join(GOLDEN, "kv_bytes.json")))
    for case in data["cases"]:
        got = P.kv_bytes(case["tokens"], case["layers"], case["kv_heads"], case["head_dim"], case["bytes"])
        unit = {"B": 1, "MB": 1e6, "GB": 1e9, "MiB": 2**20, "GiB": 2**30}[case["unit"]]
        assert abs(got / unit - case["value"]) <= case["tol"], case


# ---------------------------------------------------------------------------
# invariants ([P2] 'PagedAttention - ...' and 'Sharing ...'; [P3] block management)


def snapshot(pool):
    return (list(pool.free_stack), list(pool.ref),
            {s: (list(q.blocks), q.length, q.swapped) for s, q in pool.seqs.items()}, pool.next_seq_id,
            pool.cow_count)


def check_invariants(pool, store_ok=True):
    N = pool.num_blocks
    # I1: refcounts equal the number of table entries pointing at each block
    count = [0] * N
    for q in pool.seqs.values():
        for b in q.blocks:
            count[b] += 1
    assert count == pool.ref
    # I2: free list + used blocks partition the pool, no duplicates
    assert len(set(pool.free_stack)) == len(pool.free_stack)
    assert all(pool.ref[b] == 0 for b in pool.free_stack)
    assert len(pool.free_stack) + sum(1 for r in pool.ref if r > 0) == N
    # I3: blocks = ceil(L / 16), so internal waste <= 15 tokens per sequence
    # (a swapped-out sequence holds no blocks and keeps its length)
    for q in pool.seqs.values():
        if q.swapped:
            assert q.blocks == []
            continue
        assert len(q.blocks) == -(-q.length // 16)
        assert len(q.blocks) * 16 - q.length <= 15


class Shadow:
    """Logical token streams and a TokenStore written through the slots (I5/I6)."""

    def __init__(self, n_blocks):
        import numpy as np

        self.np = np
        self.store = P.TokenStore(n_blocks, (), np.int64)
        self.streams = {}
        self.host = {}  # swapped-out sequences' tokens, read through their blocks at swap-out
        self.counter = 0

    def on_create(self, s):
        self.streams[s] = []

    def on_append(self, pool, s, n, slots, copies):
        for c in copies:
            # I5: the copy's source holds the sequence's valid tokens
            self.store.copy_block(c)
        vals = list(range(self.counter, self.counter + n))
        self.counter += n
        self.store.write(slots, vals)
        self.streams[s] += vals

    def on_swap_out(self, pool, s, ids):
        L = pool.seq_len(s)
        self.host[s] = list(self.store.gather(ids, L)) if L else []

    def on_swap_in(self, pool, s, ids):
        L = pool.seq_len(s)
        slots = [ids[t // 16] * 16 + t % 16 for t in range(L)]
        self.store.write(slots, self.host.pop(s))

    def check(self, pool):
        for s, stream in self.streams.items():
            if s not in pool.seqs or pool.seqs[s].swapped:
                continue
            row = pool.seq_blocks(s)
            got = list(self.store.gather(row, pool.seq_len(s))) if stream else []
            assert got == stream, s


def random_script_step(pool, shadow, rng):
    live = [s for s, q in pool.seqs.items() if not q.swapped]
    swapped = [s for s, q in pool.seqs.items() if q.swapped]
    kind = rng.choice(["create", "append", "append", "append", "fork", "share", "free", "swap_out", "swap_in"])
    before = snapshot(pool)
    try:
        if kind == "swap_in" and swapped:
            s = rng.choice(swapped)
            ids = pool.swap_in(s)
            assert len(ids) == -(-pool.seq_len(s) // 16) and all(pool.ref[b] == 1 for b in ids)
            shadow.on_swap_in(pool, s, ids)
        elif kind == "swap_out" and live:
            s = rng.choice(live)
            refs = {b: pool.ref[b] for b in pool.seq_blocks(s)}
            ids = pool.swap_out(s)
            assert ids == list(refs)
            for b in ids:  # one reference dropped from each block
                assert pool.ref[b] == refs[b] - 1
            shadow.on_swap_out(pool, s, ids)
        elif kind in ("create", "swap_in", "swap_out") or not live:
            s = pool.seq_create()
            shadow.on_create(s)
        elif kind == "append":
            s = rng.choice(live)
            n = rng.choice([0, 1, 3, 15, 16, 17, 40])
            old = [pool.ref[b] for b in pool.seq_blocks(s)]
            slots, copies = pool.append(s, n)
            for c in copies:
                # I5: a copy only happens for a shared partial block; old ref drops by one
                assert c.valid_tokens % 16 != 0
                assert pool.ref[c.dst] == 1
            shadow.on_append(pool, s, n, slots, copies)
            del old
        elif kind == "fork":
            p = rng.choice(live)
            c = pool.fork(p)
            shadow.streams[c] = list(shadow.streams[p])
            # I4: one physical copy, both tables point at it
            assert pool.seq_blocks(c) == pool.seq_blocks(p)
        elif kind == "share":
            p = rng.choice(live)
            n = (pool.seq_len(p) // 16) * 16
            c = pool.share_prefix(p, n)
            shadow.streams[c] = list(shadow.streams[p][:n])
            assert pool.seq_blocks(c) == pool.seq_blocks(p)[: n // 16]
        else:
            s = rng.choice(live + swapped)
            pool.seq_free(s)
            del shadow.streams[s]
            shadow.host.pop(s, None)
    except P.OutOfBlocks:
        # I7: an out-of-blocks error leaves every structure as it was
        assert snapshot(pool) == before


@pytest.mark.parametrize("seed", range(12))
def test_random_scripts_keep_invariants(seed):
    rng = random.Random(seed)
    n = rng.choice([4, 6, 9, 16, 33, 64])
    order = list(range(n))
    rng.shuffle(order)
    pool = P.PoolModel(n, order=order)
    shadow = Shadow(n)
    for _ in range(300):
        random_script_step(pool, shadow, rng)
        check_invariants(pool)
        shadow.check(pool)


def test_exhaustive_small_scripts():
    """Every script of up to 5 operations over a 5-block pool."""
    ops = [("create",), ("append", 0, 1), ("append", 0, 16), ("append", 0, 17), ("append", 1, 3),
           ("fork", 0), ("share", 0), ("free", 0), ("free", 1)]
    n_scripts = 0
    for depth in range(1, 6):
        for script in itertools.product(ops, repeat=depth):
            pool = P.PoolModel(5)
            shadow = Shadow(5)
            for op in script:
                live = sorted(pool.seqs)
                before = snapshot(pool)
                try:
                    if op[0] == "create":
                        shadow.on_create(pool.seq_create())
                    elif not live:
                        continue
                    elif op[0] == "append":
                        s = live[op[1] % len(live)]
                        slots, copies = pool.append(s, op[2])
                        shadow.on_append(pool, s, op[2], slots, copies)
                    elif op[0] == "fork":
                        p = live[0]
                        c = pool.fork(p)
                        shadow.streams[c] = list(shadow.streams[p])
                    elif op[0] == "share":
                        p = live[-1]
                        k = (pool.seq_len(p) // 16) * 16
                        c = pool.share_prefix(p, k)
                        shadow.streams[c] = list(shadow.streams[p][:k])
                    elif op[0] == "free":
                        s = live[op[1] % len(live)]
                        pool.seq_free(s)
                        del shadow.streams[s]
                except P.OutOfBlocks:
                    assert snapshot(pool) == before
                check_invariants(pool)
                shadow.check(pool)
            n_scripts += 1
    assert n_scripts == sum(len(ops) ** k for k in range(1, 6))


def test_swap_hand_worked():
    """A script worked out by hand from the documented policy: 6 blocks handed
    out in identity order, a fork sharing both blocks, a swap-out that frees
    only the unshared block, a swap-in into fresh blocks."""
    pool = P.PoolModel(6)
    a = pool.seq_create()
    pool.append(a, 20)                      # blocks 0, 1 (4 tokens in block 1)
    b = pool.fork(a)                        # both shared, refcount 2
    pool.append(b, 1)                       # b copies partial block 1 into block 2
    assert pool.seq_blocks(b) == [0, 2] and pool.ref == [2, 1, 1, 0, 0, 0]
    assert pool.swap_out(a) == [0, 1]       # drops a's references: block 1 is free again
    assert pool.ref == [1, 0, 1, 0, 0, 0] and pool.free_stack == [5, 4, 3, 1]
    assert pool.seq_len(a) == 20 and pool.stats()["swapped_seqs"] == 1
    assert pool.stats()["swapped_tokens"] == 20 and pool.stats()["tokens"] == 21
    for op in (lambda: pool.append(a, 1), lambda: pool.fork(a), lambda: pool.swap_out(a),
               lambda: pool.seq_blocks(a), lambda: pool.block_table([a], 4), lambda: pool.swap_in(b)):
        with pytest.raises(P.BadState):
            op()
    c = pool.seq_create()
    pool.append(c, 48)                      # takes 1, 3, 4 (last freed first)
    assert pool.seq_blocks(c) == [1, 3, 4]
    with pytest.raises(P.OutOfBlocks):      # a needs 2 blocks, 1 is free: nothing changes
        before = snapshot(pool)
        pool.swap_in(a)
    assert snapshot(pool) == before
    pool.seq_free(c)                        # pushes 1, 3, 4: free stack [5, 1, 3, 4]
    assert pool.swap_in(a) == [4, 3]        # private copies, refcount 1
    assert pool.ref == [1, 0, 1, 1, 1, 0] and pool.seq_blocks(a) == [4, 3]
    pool.seq_free(a)
    d = pool.seq_create()
    pool.append(d, 5)
    assert pool.swap_out(d) == [3]
    pool.seq_free(d)                        # a swapped-out sequence can be freed
    assert pool.stats()["swapped_seqs"] == 0 and pool.free_stack == [5, 1, 4, 3]


def test_errors():
    pool = P.PoolModel(4)
    with pytest.raises(P.InvalidArgument):
        P.PoolModel(4, block_size=32)
    with pytest.raises(P.InvalidArgument):
        P.PoolModel(3, order=[0, 1, 1])
    s = pool.seq_create()
    pool.append(s, 20)
    with pytest.raises(P.InvalidArgument):
        pool.append(s, -1)
    with pytest.raises(P.InvalidArgument):
        pool.share_prefix(s, 8)
    pool.seq_free(s)
    with pytest.raises(P.BadState):
        pool.seq_free(s)
    with pytest.raises(P.InvalidArgument):
        pool.seq_len(99)
    ids_ = pool.alloc(2)
    with pytest.raises(P.BadState):
        pool.free([ids_[0], ids_[0]])  # underflow on the second drop: nothing changes
    assert pool.ref[ids_[0]] == 1
    pool.free(ids_)
    with pytest.raises(P.OutOfBlocks):
        pool.alloc(5)
    assert pool.stats()["free_blocks"] == 4
