"""Block pool, free list, refcounts, block tables, sharing, copy-on-write.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain Python: lists and
ints, one step at a time, so that every rule can be checked against the pages
by eye.

What the pages fix:

* KV cache lives in fixed-size 16-token blocks; a table per request maps
  (request, logical block index) to a physical block; blocks are handed out on
  demand as the sequence grows and returned when the request completes
  ([P1] "PagedAttention: an OS idea, not an ML one"; [P2] "PagedAttention -
  operating-system virtual memory, applied to attention").
* Allocation takes a block from a pre-allocated free list in O(1) whenever a
  request needs a new block, i.e. every 16 tokens ([P3] "PagedAttention block
  management", item (c)).
* Shared blocks are reference counted: two requests sharing a prefix give the
  block refcount 2; a finished request decrements; at 0 the block goes back to
  the free pool ([P3] same section, item (e)).
* Identical prefixes are stored once and every sharer's table points at that
  one copy; a sequence that must write into a shared block first gets its own
  copy ([P2] "Sharing, and what makes a prefix reusable"; [P3] item (g)).
* Uniform blocks mean every free block fits every need, and the small block
  caps internal waste at 15 tokens per sequence ([P2] "PagedAttention - ...").
* When blocks run out the caller must be told, so that it can preempt or refuse
  admission ([P2] "When it runs out anyway"; [P3] item (f)).

What the pages leave open, and the reading taken here (the C++ allocator of the
library follows the same documented policy independently):

* Hand-out order.  The pool takes an optional permutation ``order`` of the
  block ids: at first, blocks are handed out in that order (identity if none).
  The free list is a stack: a freed block is the next one handed out (LIFO).
* A request for n blocks is all-or-nothing: if fewer than n are free, nothing
  changes and ``OutOfBlocks`` is raised.
* Sequence ids are 0, 1, 2, ... in creation order and are never reused.
* ``append`` first counts the blocks it will need (new blocks, plus one if the
  tail block is partial and shared); if short, nothing changes.  It then walks
  the new token positions t in order: at t % 16 == 0 it takes a new block; if
  instead the block holding t is shared (refcount > 1) it takes a new block,
  records a copy (src, dst, valid_tokens = t % 16), drops one reference to the
  old block and puts the new block in the table.  The slot of token t is
  table[t // 16] * 16 + t % 16.
* ``fork`` shares every block, the partial tail included (parallel sampling,
  [P3] item (g)); ``share_prefix`` shares the first n tokens, n a multiple of
  16 (prefix matching is block aligned, [P2] "Fast answers").
* ``free`` drops one reference to each block of the sequence, in logical order.
* Swapping to host memory ([P2] "When it runs out anyway": a preempted
  request's blocks move across the host link to CPU memory and return later;
  [P3] "M.65 Inference Serving": the same spill-and-reload of blocks).  ``swap_out`` returns the sequence's block ids
  in logical order (the caller copies those blocks to host memory before any
  of them is reused) and drops one reference to each, in that order; the
  sequence keeps its length and holds no blocks while swapped.  ``swap_in``
  takes ceil(length / 16) blocks off the free list (all or nothing) and
  returns them in logical order; the caller copies the host copy into them.
  A swapped sequence cannot be appended to, forked, shared, swapped out again
  or put in a block table; it can be freed.  Blocks that were shared when the
  sequence left come back as private copies.
* Prefix caching with retention ([P1] "PagedAttention ...": hash a shared
  prefix and reuse its KV blocks; [P2] "Sharing, and what makes a prefix
  reusable": keep a finished request's cache and match new requests against
  it, on exact token ids, block-aligned, from the very start; [P2] "The
  isolation question": key the cache per tenant).  Readings:
  - A full block (16 tokens) is keyed by a chain: key_j = FNV-1a-64 over the
    bytes of key_{j-1} (8 bytes little-endian; 0 before the first block), the
    tenant (4 bytes) and the block's 16 token ids (4 bytes each), all
    little-endian.  An entry records the key, the block, the parent key, the
    tenant and the 16 ids; a lookup matches only when all of them agree, so a
    hash collision cannot produce a wrong match.
  - ``create_cached(tenant, tokens)`` starts a sequence with as many leading
    full blocks of ``tokens`` as the cache holds, at most len(tokens) - 1
    tokens (one token is always left to compute).  A matched block gains a
    reference; if it was retained with no reference it leaves the evictable
    list.  The sequence records the tenant and the keys of its blocks.
  - ``cache_tokens(s, start, tokens)`` registers the sequence's full blocks
    holding positions start .. start + len - 1; ``start`` must equal 16 x the
    blocks already keyed (matched or registered), and the positions must be
    written.  A block whose key is already in the cache (same content keyed
    earlier by another block) stays unregistered.
  - A registered block whose last reference drops is retained: it goes to the
    evictable list (least recently used first) instead of the free stack.
    When a sequence drops several at once (free, swap-out), the deeper blocks
    are listed as older, so a chain is evicted from its leaves back to its root.
  - Taking a block uses the free stack first; when it is empty, the oldest
    evictable block is reused and its cache entry removed.  Every
    all-or-nothing check counts free plus evictable blocks.
  - fork and share_prefix carry the tenant and the keys of the shared blocks.
    A swapped-out sequence forgets its keys: its blocks come back private and
    unregistered.
"""

from __future__ import annotations

import struct
from dataclasses import dataclass, field

BLOCK = 16


class PoolError(Exception):
    """Base class; ``code`` matches the library's status names."""

    code = "INVALID"


class InvalidArgument(PoolError):
    code = "INVALID"


class OutOfBlocks(PoolError):
    code = "OOM"


class BadState(PoolError):
    """Double free, refcount underflow, use of a freed sequence."""

    code = "STATE"


@dataclass
class CopyOp:
    """A copy-on-write the caller must run before writing the token."""

    src: int
    dst: int
    valid_tokens: int


@dataclass
class Seq:
    blocks: list = field(default_factory=list)
    length: int = 0
    swapped: bool = False
    tenant: int = 0
    keys: list = field(default_factory=list)  # chain key of each leading keyed block


FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a (Fowler, Noll, Vo): xor each byte in, then multiply."""
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def block_key(parent_key: int, tenant: int, token_ids) -> int:
    """Chain key of one full block (see the module docstring)."""
    ids = [int(t) for t in token_ids]
    assert len(ids) == BLOCK
    data = struct.pack("<QI", parent_key, tenant & 0xFFFFFFFF) + struct.pack(f"<{BLOCK}i", *ids)
    return fnv1a64(data)


@dataclass
class CacheEntry:
    block: int
    parent_key: int
    tenant: int
    tokens: tuple


class PoolModel:
    """Host model of the block pool and every sequence's block table."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK, order=None):
        if block_size != BLOCK:
            raise InvalidArgument("block size is fixed at 16 tokens")
        if num_blocks <= 0:
            raise InvalidArgument("num_blocks must be positive")
        if order is None:
            order = list(range(num_blocks))
        order = [int(b) for b in order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArgument("order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        # The stack's top is its last element; order[0] must come out first.
        self.free_stack = list(reversed(order))
        self.ref = [0] * num_blocks
        self.seqs: dict[int, Seq] = {}
        self.next_seq_id = 0
        self.cow_count = 0
        self.cache: dict[int, CacheEntry] = {}  # key -> entry
        self.key_of: dict[int, int] = {}        # registered block -> key
        self.evictable: list = []               # retained blocks, least recently used first
        self.matched_tokens = 0

    # -- raw blocks -------------------------------------------------------
    def available(self) -> int:
        """Blocks a request can take: the free stack plus the evictable list."""
        return len(self.free_stack) + len(self.evictable)

    def _pop(self) -> int:
        if self.free_stack:
            b = self.free_stack.pop()
        else:  # reuse the least recently used retained block; its entry goes
            b = self.evictable.pop(0)
            del self.cache[self.key_of.pop(b)]
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _decref(self, b: int, retained=None) -> None:
        """Drop one reference; at 0 a registered block is retained (appended
        to ``retained`` if given, else straight to the evictable list) and any
        other block goes back on the free stack."""
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                if retained is None:
                    self.evictable.append(b)
                else:
                    retained.append(b)
            else:
                self.free_stack.append(b)

    def _drop_all(self, blocks) -> None:
        """Drop one reference from each block in logical order; the ones that
        become retained join the evictable list deepest first (oldest)."""
        retained = []
        for b in blocks:
            self._decref(b, retained)
        self.evictable.extend(reversed(retained))

    def alloc(self, n: int) -> list:
        if n < 0:
            raise InvalidArgument("negative count")
        if self.available() < n:
            raise OutOfBlocks(f"need {n}, available {self.available()}")
        return [self._pop() for _ in range(n)]

    def _check_ids(self, ids) -> list:
        ids = [int(b) for b in ids]
        for b in ids:
            if not 0 <= b < self.num_blocks:
                raise InvalidArgument(f"block id {b} out of range")
        return ids

    def incref(self, ids) -> None:
        ids = self._check_ids(ids)
        for b in ids:
            if self.ref[b] == 0:
                raise BadState(f"incref of free block {b}")
        for b in ids:
            self.ref[b] += 1

    def free(self, ids) -> None:
        ids = self._check_ids(ids)
        # Validate the whole list first, so that an error changes nothing.
        drops: dict[int, int] = {}
        for b in ids:
            drops[b] = drops.get(b, 0) + 1
        for b, k in drops.items():
            if self.ref[b] < k:
                raise BadState(f"refcount underflow on block {b}")
        for b in ids:
            self._decref(b)

    # -- sequences --------------------------------------------------------
    def _seq(self, s: int) -> Seq:
        if s not in self.seqs:
            if 0 <= s < self.next_seq_id:
                raise BadState(f"sequence {s} was freed")
            raise InvalidArgument(f"no sequence {s}")
        return self.seqs[s]

    def seq_create(self) -> int:
        s = self.next_seq_id
        self.next_seq_id += 1
        self.seqs[s] = Seq()
        return s

    def _resident(self, s: int) -> Seq:
        q = self._seq(s)
        if q.swapped:
            raise BadState(f"sequence {s} is swapped out")
        return q

    def seq_len(self, s: int) -> int:
        return self._seq(s).length

    def seq_blocks(self, s: int) -> list:
        return list(self._resident(s).blocks)

    def append(self, s: int, n: int):
        """Grow sequence ``s`` by ``n`` tokens; returns (slots, copies)."""
        if n < 0:  # a bad argument is reported before the sequence's state
            raise InvalidArgument("negative token count")
        q = self._resident(s)
        L = q.length
        have = -(-L // BLOCK)
        want = -(-(L + n) // BLOCK)
        need = want - have
        if n > 0 and L % BLOCK != 0 and self.ref[q.blocks[L // BLOCK]] > 1:
            need += 1
        if self.available() < need:
            raise OutOfBlocks(f"append needs {need} blocks, available {self.available()}")
        slots, copies = [], []
        for t in range(L, L + n):
            j, o = divmod(t, BLOCK)
            if o == 0:
                q.blocks.append(self._pop())
            elif self.ref[q.blocks[j]] > 1:
                old = q.blocks[j]
                new = self._pop()
                copies.append(CopyOp(src=old, dst=new, valid_tokens=o))
                self._decref(old)
                q.blocks[j] = new
                self.cow_count += 1
            slots.append(q.blocks[j] * BLOCK + o)
        q.length = L + n
        return slots, copies

    def fork(self, parent: int) -> int:
        p = self._resident(parent)
        for b in p.blocks:
            self.ref[b] += 1
        c = self.seq_create()
        self.seqs[c].blocks = list(p.blocks)
        self.seqs[c].length = p.length
        self.seqs[c].tenant = p.tenant
        self.seqs[c].keys = list(p.keys)
        return c

    def share_prefix(self, src: int, n_tokens: int) -> int:
        p = self._resident(src)
        if n_tokens < 0 or n_tokens % BLOCK != 0 or n_tokens > p.length:
            raise InvalidArgument("shared prefix must be block aligned and within the source")
        shared = p.blocks[: n_tokens // BLOCK]
        for b in shared:
            self.ref[b] += 1
        c = self.seq_create()
        self.seqs[c].blocks = list(shared)
        self.seqs[c].length = n_tokens
        self.seqs[c].tenant = p.tenant
        self.seqs[c].keys = p.keys[: n_tokens // BLOCK]
        return c

    def seq_free(self, s: int) -> None:
        q = self._seq(s)
        self._drop_all(q.blocks)
        del self.seqs[s]

    def swap_out(self, s: int) -> list:
        """Block ids of ``s`` in logical order; then one reference dropped from
        each, and ``s`` swapped out with its length kept."""
        q = self._resident(s)
        ids = list(q.blocks)
        self._drop_all(ids)
        q.blocks = []
        q.keys = []
        q.swapped = True
        return ids

    def swap_in(self, s: int) -> list:
        """Fresh blocks for swapped-out ``s`` (all or nothing), in logical order."""
        q = self._seq(s)
        if not q.swapped:
            raise BadState(f"sequence {s} is not swapped out")
        n = -(-q.length // BLOCK)
        if self.available() < n:
            raise OutOfBlocks(f"swap in needs {n} blocks, available {self.available()}")
        q.blocks = [self._pop() for _ in range(n)]
        q.swapped = False
        return list(q.blocks)

    # -- prefix cache ---------------------------------------------------------
    def create_cached(self, tenant: int, tokens) -> tuple:
        """New sequence holding the longest cached run of leading full blocks
        of ``tokens`` (at most len(tokens) - 1 tokens); returns (seq, tokens
        matched)."""
        tokens = [int(t) for t in tokens]
        blocks, keys = [], []
        parent = 0
        for j in range(max(0, len(tokens) - 1) // BLOCK):
            ids = tuple(tokens[BLOCK * j: BLOCK * (j + 1)])
            key = block_key(parent, tenant, ids)
            e = self.cache.get(key)
            if e is None or e.parent_key != parent or e.tenant != tenant or e.tokens != ids:
                break
            blocks.append(e.block)
            keys.append(key)
            parent = key
        for b in blocks:
            if self.ref[b] == 0:
                self.evictable.remove(b)
            self.ref[b] += 1
        s = self.seq_create()
        q = self.seqs[s]
        q.blocks, q.keys, q.length, q.tenant = blocks, keys, BLOCK * len(blocks), tenant
        self.matched_tokens += BLOCK * len(blocks)
        return s, BLOCK * len(blocks)

    def cache_tokens(self, s: int, start: int, tokens) -> int:
        """Key and register the full blocks of ``s`` covering positions start
        .. start + len(tokens) - 1; returns how many blocks were keyed."""
        q = self._resident(s)
        tokens = [int(t) for t in tokens]
        if start != BLOCK * len(q.keys) or start + len(tokens) > q.length:
            raise InvalidArgument("tokens must start at the first unkeyed block and lie inside the sequence")
        parent = q.keys[-1] if q.keys else 0
        n_full = len(tokens) // BLOCK
        for j in range(n_full):
            ids = tuple(tokens[BLOCK * j: BLOCK * (j + 1)])
            key = block_key(parent, q.tenant, ids)
            b = q.blocks[len(q.keys)]
            if key not in self.cache and b not in self.key_of:
                self.cache[key] = CacheEntry(b, parent, q.tenant, ids)
                self.key_of[b] = key
            q.keys.append(key)
            parent = key
        return n_full

    def block_table(self, seq_ids, max_blocks: int):
        """Rows of physical block ids padded with -1, and the lengths."""
        rows, lens = [], []
        for s in seq_ids:
            q = self._resident(int(s))
            if len(q.blocks) > max_blocks:
                raise InvalidArgument("sequence has more blocks than max_blocks")
            rows.append(list(q.blocks) + [-1] * (max_blocks - len(q.blocks)))
            lens.append(q.length)
        return rows, lens

    def stats(self) -> dict:
        used = sum(1 for r in self.ref if r > 0)
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free_stack),
            "used_blocks": used,
            "shared_blocks": sum(1 for r in self.ref if r > 1),
            "refcount_sum": sum(self.ref),
            "cow_count": self.cow_count,
            "num_seqs": len(self.seqs),
            "tokens": sum(q.length for q in self.seqs.values() if not q.swapped),
            "waste_tokens": sum(len(q.blocks) * BLOCK - q.length for q in self.seqs.values() if not q.swapped),
            "swapped_seqs": sum(1 for q in self.seqs.values() if q.swapped),
            "swapped_tokens": sum(q.length for q in self.seqs.values() if q.swapped),
            "cached_blocks": len(self.cache),
            "evictable_blocks": len(self.evictable),
            "matched_tokens": self.matched_tokens,
        }


class TokenStore:
    """Host storage written and read through the pool's slots.

    Its own layout, ``data[block][token_in_block][...]``, is unrelated to the
    device layout of the library: what it models is that paging is a change of
    where tokens live, never of what attention reads ([P2] "PagedAttention -
    ...": results are bit-for-bit identical).
    """

    def __init__(self, num_blocks: int, token_shape, dtype):
        import numpy as np

        self.data = np.zeros((num_blocks, BLOCK) + tuple(token_shape), dtype=dtype)

    def write(self, slots, values) -> None:
        for i, slot in enumerate(slots):
            b, o = divmod(int(slot), BLOCK)
            self.data[b, o] = values[i]

    def copy_block(self, op: CopyOp) -> None:
        self.data[op.dst] = self.data[op.src]

    def gather(self, table_row, length: int):
        """Token rows 0..length-1 of one sequence, read through its table."""
        import numpy as np

        out = np.empty((length,) + self.data.shape[2:], dtype=self.data.dtype)
        for t in range(length):
            b = int(table_row[t // BLOCK])
            out[t] = self.data[b, t % BLOCK]
        return out


def kv_bytes(tokens: int, layers: int, kv_heads: int, head_dim: int, bytes_per_elt: float) -> float:
    """Bytes of K and V for ``tokens`` cached tokens: 2 (K and V) x layers x
    heads x head_dim x tokens x bytes per element ([P3] "KV cache memory math";
    with grouped-query attention, heads are the kv heads)."""
    return 2 * layers * kv_heads * head_dim * tokens * bytes_per_elt
