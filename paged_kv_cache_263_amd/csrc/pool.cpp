// Host block allocator: free list, refcounts, per-sequence block tables,
// sharing and copy-on-write planning.
//
// Mechanism from the pages: fixed 16-token blocks handed out on demand from a
// pre-allocated free list and returned when a request completes ([P1]
// "PagedAttention: an OS idea, not an ML one"; [P3] "PagedAttention block
// management" items (b), (c)); reference-counted sharing, a block going back to
// the pool when its count reaches 0 ([P3] item (e)); one physical copy of a
// shared prefix, and a private copy before writing into a shared block ([P2]
// "Sharing, and what makes a prefix reusable"; [P3] item (g)).
//
// Policy where the pages are silent (documented in pagedkv.h): blocks are
// first handed out in the caller's order, then last-freed-first; every
// request is all-or-nothing, so an out-of-blocks error changes nothing.
//
// Prefix caching with retention ([P1] "PagedAttention ...": hash a shared
// prefix and reuse its blocks; [P2] "Sharing, and what makes a prefix
// reusable": keep a finished request's cache, match new requests on exact
// token ids, block-aligned, from the start; [P2] "The isolation question": key
// per tenant).  Full blocks are keyed by an FNV-1a-64 chain over (parent key,
// tenant, 16 token ids); a registered block whose last reference drops is
// retained on an LRU list and reused only when the free stack is empty.
#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "internal.h"

using pkv::fail;

namespace {

constexpr int32_t kBlock = PKV_BLOCK_SIZE;

struct Sequence {
    std::vector<int32_t> blocks;  // logical block index -> physical block id
    int32_t len = 0;
    bool live = false;
    bool swapped = false;         // blocks are in host memory; the table is empty
    int32_t tenant = 0;
    std::vector<uint64_t> keys;   // chain key of each leading keyed block
};

inline int32_t blocks_for(int64_t tokens) { return static_cast<int32_t>((tokens + kBlock - 1) / kBlock); }

// 64-bit FNV-1a (Fowler, Noll, Vo) over the little-endian bytes of
// (parent key, tenant, the block's 16 token ids).
uint64_t block_key(uint64_t parent, int32_t tenant, const int32_t* ids) {
    unsigned char buf[8 + 4 + 4 * kBlock];
    for (int i = 0; i < 8; ++i) buf[i] = static_cast<unsigned char>(parent >> (8 * i));
    const uint32_t t = static_cast<uint32_t>(tenant);
    for (int i = 0; i < 4; ++i) buf[8 + i] = static_cast<unsigned char>(t >> (8 * i));
    for (int k = 0; k < kBlock; ++k) {
        const uint32_t v = static_cast<uint32_t>(ids[k]);
        for (int i = 0; i < 4; ++i) buf[12 + 4 * k + i] = static_cast<unsigned char>(v >> (8 * i));
    }
    uint64_t h = 0xCBF29CE484222325ull;
    for (unsigned char c : buf) {
        h ^= c;
        h *= 0x100000001B3ull;
    }
    return h;
}

struct CacheEntry {
    int32_t block;
    uint64_t parent;
    int32_t tenant;
    int32_t ids[kBlock];
};

}  // namespace

struct pkv_pool {
    int32_t num_blocks = 0;
    std::vector<int32_t> free_stack;  // back() is handed out next
    std::vector<int32_t> ref;
    std::vector<Sequence> seqs;       // index = sequence id
    int64_t cow_count = 0;
    int64_t live_seqs = 0;
    // prefix cache
    std::unordered_map<uint64_t, CacheEntry> cache;  // key -> entry
    std::vector<uint64_t> key_of;                    // registered block -> its key
    std::vector<uint8_t> registered;
    // evictable list (least recently used at the head), linked through the block ids
    std::vector<int32_t> ev_prev, ev_next;
    int32_t ev_head = -1, ev_tail = -1;
    int64_t ev_count = 0;
    int64_t matched_tokens = 0;

    int64_t available() const { return static_cast<int64_t>(free_stack.size()) + ev_count; }
    void ev_push_back(int32_t b) {
        ev_prev[b] = ev_tail;
        ev_next[b] = -1;
        if (ev_tail >= 0) ev_next[ev_tail] = b; else ev_head = b;
        ev_tail = b;
        ev_count += 1;
    }
    void ev_remove(int32_t b) {
        if (ev_prev[b] >= 0) ev_next[ev_prev[b]] = ev_next[b]; else ev_head = ev_next[b];
        if (ev_next[b] >= 0) ev_prev[ev_next[b]] = ev_prev[b]; else ev_tail = ev_prev[b];
        ev_prev[b] = ev_next[b] = -1;
        ev_count -= 1;
    }
    // A block off the free stack, else the least recently used retained block
    // (its cache entry is removed).  The caller has checked available().
    int32_t take() {
        int32_t b;
        if (!free_stack.empty()) {
            b = free_stack.back();
            free_stack.pop_back();
        } else {
            b = ev_head;
            ev_remove(b);
            cache.erase(key_of[b]);
            registered[b] = 0;
        }
        ref[b] = 1;
        return b;
    }
    // Drop one reference; at 0 a registered block is retained (into *retained
    // if given, else onto the evictable list) and any other block is freed.
    void drop(int32_t b, std::vector<int32_t>* retained = nullptr) {
        if (--ref[b] != 0) return;
        if (registered[b]) {
            if (retained) retained->push_back(b); else ev_push_back(b);
        } else {
            free_stack.push_back(b);
        }
    }
    // Drop one reference from each block in logical order; blocks that become
    // retained join the evictable list deepest first (evicted first).
    void drop_all(const std::vector<int32_t>& blocks) {
        std::vector<int32_t> retained;
        for (int32_t b : blocks) drop(b, &retained);
        for (auto it = retained.rbegin(); it != retained.rend(); ++it) ev_push_back(*it);
    }
    Sequence* find(int32_t s, int* status) {
        if (s < 0 || s >= static_cast<int32_t>(seqs.size())) {
            *status = fail(PKV_ERR_INVALID, "no sequence %d", s);
            return nullptr;
        }
        if (!seqs[s].live) {
            *status = fail(PKV_ERR_STATE, "sequence %d was freed", s);
            return nullptr;
        }
        return &seqs[s];
    }
    // A live sequence that holds its blocks (not swapped out).
    Sequence* resident(int32_t s, int* status) {
        Sequence* q = find(s, status);
        if (q && q->swapped) {
            *status = fail(PKV_ERR_STATE, "sequence %d is swapped out", s);
            return nullptr;
        }
        return q;
    }
    // Blocks one append of n tokens to q will take (new blocks, plus one if the
    // partial tail block is shared and must be copied first).
    int64_t blocks_needed(const Sequence& q, int32_t n) const {
        int64_t need = blocks_for(static_cast<int64_t>(q.len) + n) - blocks_for(q.len);
        if (n > 0 && q.len % kBlock != 0 && ref[q.blocks[q.len / kBlock]] > 1) need += 1;
        return need;
    }
    // Perform an append already checked to fit.
    void do_append(Sequence& q, int32_t n, int32_t* slots, pkv_copy* copy, int32_t* n_copy) {
        *n_copy = 0;
        for (int32_t i = 0; i < n; ++i) {
            const int32_t t = q.len + i;
            const int32_t j = t / kBlock;
            const int32_t o = t % kBlock;
            if (o == 0) {
                q.blocks.push_back(take());
            } else if (ref[q.blocks[j]] > 1) {
                const int32_t old = q.blocks[j];
                const int32_t fresh = take();
                copy[*n_copy] = pkv_copy{old, fresh, o};
                *n_copy += 1;
                drop(old);
                q.blocks[j] = fresh;
                cow_count += 1;
            }
            slots[i] = q.blocks[j] * kBlock + o;
        }
        q.len += n;
    }
    int32_t new_seq() {
        seqs.emplace_back();
        seqs.back().live = true;
        live_seqs += 1;
        return static_cast<int32_t>(seqs.size() - 1);
    }
};

extern "C" {

int kv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* order, pkv_pool** out) {
    if (!out) return fail(PKV_ERR_INVALID, "kv_pool_create: null output");
    *out = nullptr;
    if (block_size != kBlock) return fail(PKV_ERR_UNSUPPORTED, "block size must be %d", kBlock);
    if (num_blocks <= 0 || num_blocks > (INT32_MAX / kBlock)) return fail(PKV_ERR_INVALID, "bad num_blocks %d", num_blocks);
    pkv_pool* p = new (std::nothrow) pkv_pool();
    if (!p) return fail(PKV_ERR_INVALID, "host allocation failed");
    p->num_blocks = num_blocks;
    p->ref.assign(num_blocks, 0);
    p->key_of.assign(num_blocks, 0);
    p->registered.assign(num_blocks, 0);
    p->ev_prev.assign(num_blocks, -1);
    p->ev_next.assign(num_blocks, -1);
    p->free_stack.resize(num_blocks);
    if (order) {
        std::vector<char> seen(num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            const int32_t b = order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete p;
                return fail(PKV_ERR_INVALID, "order is not a permutation (entry %d = %d)", i, b);
            }
            seen[b] = 1;
            p->free_stack[num_blocks - 1 - i] = b;  // order[0] on top
        }
    } else {
        for (int32_t i = 0; i < num_blocks; ++i) p->free_stack[num_blocks - 1 - i] = i;
    }
    *out = p;
    return PKV_OK;
}

void kv_pool_destroy(pkv_pool* pool) { delete pool; }

int kv_pool_alloc(pkv_pool* p, int32_t n, int32_t* out_ids) {
    if (!p || n < 0 || (n > 0 && !out_ids)) return fail(PKV_ERR_INVALID, "kv_pool_alloc: bad arguments");
    if (n > p->available())
        return fail(PKV_ERR_OOM, "kv_pool_alloc: need %d blocks, %lld available", n, static_cast<long long>(p->available()));
    for (int32_t i = 0; i < n; ++i) out_ids[i] = p->take();
    return PKV_OK;
}

static int check_ids(const pkv_pool* p, const int32_t* ids, int32_t n) {
    if (!p || n < 0 || (n > 0 && !ids)) return fail(PKV_ERR_INVALID, "bad block id list");
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= p->num_blocks) return fail(PKV_ERR_INVALID, "block id %d out of range", ids[i]);
    return PKV_OK;
}

int kv_pool_incref(pkv_pool* p, const int32_t* ids, int32_t n) {
    int st = check_ids(p, ids, n);
    if (st) return st;
    for (int32_t i = 0; i < n; ++i)
        if (p->ref[ids[i]] == 0) return fail(PKV_ERR_STATE, "incref of free block %d", ids[i]);
    for (int32_t i = 0; i < n; ++i) p->ref[ids[i]] += 1;
    return PKV_OK;
}

int kv_pool_free(pkv_pool* p, const int32_t* ids, int32_t n) {
    int st = check_ids(p, ids, n);
    if (st) return st;
    // Check the whole list first (a block may appear more than once).
    std::vector<int32_t> sorted(ids, ids + n);
    std::sort(sorted.begin(), sorted.end());
    for (int32_t i = 0; i < n;) {
        int32_t k = i;
        while (k < n && sorted[k] == sorted[i]) ++k;
        if (p->ref[sorted[i]] < k - i) return fail(PKV_ERR_STATE, "refcount underflow on block %d", sorted[i]);
        i = k;
    }
    for (int32_t i = 0; i < n; ++i) p->drop(ids[i]);
    return PKV_OK;
}

int kv_pool_refcount(const pkv_pool* p, int32_t block, int32_t* out) {
    if (!p || !out || block < 0 || block >= p->num_blocks) return fail(PKV_ERR_INVALID, "kv_pool_refcount: bad arguments");
    *out = p->ref[block];
    return PKV_OK;
}

int kv_pool_stats(const pkv_pool* p, pkv_stats* s) {
    if (!p || !s) return fail(PKV_ERR_INVALID, "kv_pool_stats: null argument");
    pkv_stats r{};
    r.num_blocks = p->num_blocks;
    r.free_blocks = static_cast<int32_t>(p->free_stack.size());
    for (int32_t c : p->ref) {
        r.used_blocks += c > 0;
        r.shared_blocks += c > 1;
        r.refcount_sum += c;
    }
    r.cow_count = p->cow_count;
    r.num_seqs = p->live_seqs;
    r.cached_blocks = static_cast<int64_t>(p->cache.size());
    r.evictable_blocks = p->ev_count;
    r.matched_tokens = p->matched_tokens;
    for (const Sequence& q : p->seqs) {
        if (!q.live) continue;
        if (q.swapped) {
            r.swapped_seqs += 1;
            r.swapped_tokens += q.len;
            continue;
        }
        r.tokens += q.len;
        r.waste_tokens += static_cast<int64_t>(q.blocks.size()) * kBlock - q.len;
    }
    *s = r;
    return PKV_OK;
}

int kv_pool_free_list(const pkv_pool* p, int32_t* out, int32_t cap, int32_t* n) {
    if (!p || !n || cap < 0 || (cap > 0 && !out)) return fail(PKV_ERR_INVALID, "kv_pool_free_list: bad arguments");
    *n = static_cast<int32_t>(p->free_stack.size());
    if (*n > cap) return fail(PKV_ERR_INVALID, "kv_pool_free_list: capacity %d < %d", cap, *n);
    std::copy(p->free_stack.begin(), p->free_stack.end(), out);
    return PKV_OK;
}

int kv_pool_evictable_list(const pkv_pool* p, int32_t* out, int32_t cap, int32_t* n) {
    if (!p || !n || cap < 0 || (cap > 0 && !out)) return fail(PKV_ERR_INVALID, "kv_pool_evictable_list: bad arguments");
    *n = static_cast<int32_t>(p->ev_count);
    if (*n > cap) return fail(PKV_ERR_INVALID, "kv_pool_evictable_list: capacity %d < %d", cap, *n);
    int32_t i = 0;
    for (int32_t b = p->ev_head; b >= 0; b = p->ev_next[b]) out[i++] = b;
    return PKV_OK;
}

int seq_create(pkv_pool* p, int32_t* out_seq) {
    if (!p || !out_seq) return fail(PKV_ERR_INVALID, "seq_create: null argument");
    if (p->seqs.size() >= static_cast<size_t>(INT32_MAX)) return fail(PKV_ERR_INVALID, "too many sequences");
    *out_seq = p->new_seq();
    return PKV_OK;
}

int seq_append(pkv_pool* p, int32_t s, int32_t n, int32_t* out_slots, pkv_copy* out_copy, int32_t* n_copy) {
    if (!p || n < 0 || (n > 0 && !out_slots) || !out_copy || !n_copy)
        return fail(PKV_ERR_INVALID, "seq_append: bad arguments");
    int st = PKV_OK;
    Sequence* q = p->resident(s, &st);
    if (!q) return st;
    if (static_cast<int64_t>(q->len) + n > static_cast<int64_t>(INT32_MAX) - kBlock)
        return fail(PKV_ERR_INVALID, "seq_append: length overflow");
    const int64_t need = p->blocks_needed(*q, n);
    if (need > p->available())
        return fail(PKV_ERR_OOM, "seq_append: need %lld blocks, %lld available", static_cast<long long>(need),
                    static_cast<long long>(p->available()));
    p->do_append(*q, n, out_slots, out_copy, n_copy);
    return PKV_OK;
}

int seq_append_batch(pkv_pool* p, const int32_t* seqs, const int32_t* n_tokens, int32_t n, int32_t* out_slots,
                     pkv_copy* out_copies, int32_t* n_copies) {
    if (!p || n < 0 || (n > 0 && (!seqs || !n_tokens || !out_copies)) || !n_copies)
        return fail(PKV_ERR_INVALID, "seq_append_batch: bad arguments");
    std::vector<int32_t> ids(seqs, seqs + n);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
        return fail(PKV_ERR_INVALID, "seq_append_batch: a sequence is listed twice");
    int64_t need = 0, total = 0;
    for (int32_t i = 0; i < n; ++i) {
        int st = PKV_OK;
        Sequence* q = p->resident(seqs[i], &st);
        if (!q) return st;
        if (n_tokens[i] < 0 || static_cast<int64_t>(q->len) + n_tokens[i] > static_cast<int64_t>(INT32_MAX) - kBlock)
            return fail(PKV_ERR_INVALID, "seq_append_batch: bad token count %d", n_tokens[i]);
        need += p->blocks_needed(*q, n_tokens[i]);
        total += n_tokens[i];
    }
    if (total > 0 && !out_slots) return fail(PKV_ERR_INVALID, "seq_append_batch: null slots");
    if (need > p->available())
        return fail(PKV_ERR_OOM, "seq_append_batch: need %lld blocks, %lld available", static_cast<long long>(need),
                    static_cast<long long>(p->available()));
    int64_t off = 0;
    *n_copies = 0;
    for (int32_t i = 0; i < n; ++i) {
        int32_t c = 0;
        p->do_append(p->seqs[seqs[i]], n_tokens[i], out_slots + off, out_copies + *n_copies, &c);
        *n_copies += c;
        off += n_tokens[i];
    }
    return PKV_OK;
}

int seq_fork(pkv_pool* p, int32_t parent, int32_t* out_child) {
    if (!p || !out_child) return fail(PKV_ERR_INVALID, "seq_fork: null argument");
    int st = PKV_OK;
    if (!p->resident(parent, &st)) return st;
    const int32_t c = p->new_seq();  // may move the vector: index afresh below
    Sequence& src = p->seqs[parent];
    for (int32_t b : src.blocks) p->ref[b] += 1;
    p->seqs[c].blocks = src.blocks;
    p->seqs[c].len = src.len;
    p->seqs[c].tenant = src.tenant;
    p->seqs[c].keys = src.keys;
    *out_child = c;
    return PKV_OK;
}

int seq_share_prefix(pkv_pool* p, int32_t src, int32_t n_tokens, int32_t* out_seq) {
    if (!p || !out_seq) return fail(PKV_ERR_INVALID, "seq_share_prefix: null argument");
    int st = PKV_OK;
    Sequence* q = p->resident(src, &st);
    if (!q) return st;
    if (n_tokens < 0 || n_tokens % kBlock != 0 || n_tokens > q->len)
        return fail(PKV_ERR_INVALID, "seq_share_prefix: %d tokens is not a block-aligned prefix of %d", n_tokens, q->len);
    const int32_t c = p->new_seq();
    Sequence& s = p->seqs[src];
    const int32_t nb = n_tokens / kBlock;
    p->seqs[c].blocks.assign(s.blocks.begin(), s.blocks.begin() + nb);
    for (int32_t i = 0; i < nb; ++i) p->ref[s.blocks[i]] += 1;
    p->seqs[c].len = n_tokens;
    p->seqs[c].tenant = s.tenant;
    p->seqs[c].keys.assign(s.keys.begin(), s.keys.begin() + std::min<size_t>(nb, s.keys.size()));
    *out_seq = c;
    return PKV_OK;
}

int seq_free(pkv_pool* p, int32_t s) {
    if (!p) return fail(PKV_ERR_INVALID, "seq_free: null pool");
    int st = PKV_OK;
    Sequence* q = p->find(s, &st);
    if (!q) return st;
    p->drop_all(q->blocks);
    q->blocks.clear();
    q->blocks.shrink_to_fit();
    q->keys.clear();
    q->keys.shrink_to_fit();
    q->len = 0;
    q->live = false;
    q->swapped = false;
    p->live_seqs -= 1;
    return PKV_OK;
}

int seq_swap_out(pkv_pool* p, int32_t s, int32_t* out_ids, int32_t cap, int32_t* n_out) {
    if (!p || !n_out || cap < 0 || (cap > 0 && !out_ids)) return fail(PKV_ERR_INVALID, "seq_swap_out: bad arguments");
    int st = PKV_OK;
    Sequence* q = p->resident(s, &st);
    if (!q) return st;
    const int32_t n = static_cast<int32_t>(q->blocks.size());
    if (n > cap) return fail(PKV_ERR_INVALID, "seq_swap_out: capacity %d < %d blocks", cap, n);
    std::copy(q->blocks.begin(), q->blocks.end(), out_ids);
    p->drop_all(q->blocks);
    q->blocks.clear();
    q->keys.clear();
    q->swapped = true;
    *n_out = n;
    return PKV_OK;
}

int seq_swap_in(pkv_pool* p, int32_t s, int32_t* out_ids, int32_t cap, int32_t* n_out) {
    if (!p || !n_out || cap < 0 || (cap > 0 && !out_ids)) return fail(PKV_ERR_INVALID, "seq_swap_in: bad arguments");
    int st = PKV_OK;
    Sequence* q = p->find(s, &st);
    if (!q) return st;
    if (!q->swapped) return fail(PKV_ERR_STATE, "sequence %d is not swapped out", s);
    const int32_t n = blocks_for(q->len);
    if (n > cap) return fail(PKV_ERR_INVALID, "seq_swap_in: capacity %d < %d blocks", cap, n);
    if (n > p->available())
        return fail(PKV_ERR_OOM, "seq_swap_in: need %d blocks, %lld available", n, static_cast<long long>(p->available()));
    q->blocks.resize(n);
    for (int32_t j = 0; j < n; ++j) q->blocks[j] = p->take();
    std::copy(q->blocks.begin(), q->blocks.end(), out_ids);
    q->swapped = false;
    *n_out = n;
    return PKV_OK;
}

int seq_create_cached(pkv_pool* p, int32_t tenant, const int32_t* tokens, int32_t n, int32_t* out_seq,
                      int32_t* out_matched) {
    if (!p || !out_seq || !out_matched || n < 0 || (n > 0 && !tokens))
        return fail(PKV_ERR_INVALID, "seq_create_cached: bad arguments");
    if (p->seqs.size() >= static_cast<size_t>(INT32_MAX)) return fail(PKV_ERR_INVALID, "too many sequences");
    std::vector<int32_t> blocks;
    std::vector<uint64_t> keys;
    uint64_t parent = 0;
    const int32_t max_blocks = n > 0 ? (n - 1) / kBlock : 0;  // one token is always left to compute
    for (int32_t j = 0; j < max_blocks; ++j) {
        const int32_t* ids = tokens + static_cast<int64_t>(j) * kBlock;
        const uint64_t key = block_key(parent, tenant, ids);
        auto it = p->cache.find(key);
        if (it == p->cache.end()) break;
        const CacheEntry& e = it->second;
        if (e.parent != parent || e.tenant != tenant || std::memcmp(e.ids, ids, sizeof(e.ids)) != 0) break;
        blocks.push_back(e.block);
        keys.push_back(key);
        parent = key;
    }
    for (int32_t b : blocks) {
        if (p->ref[b] == 0) p->ev_remove(b);
        p->ref[b] += 1;
    }
    const int32_t s = p->new_seq();
    Sequence& q = p->seqs[s];
    q.len = static_cast<int32_t>(blocks.size()) * kBlock;
    q.blocks = std::move(blocks);
    q.keys = std::move(keys);
    q.tenant = tenant;
    p->matched_tokens += q.len;
    *out_seq = s;
    *out_matched = q.len;
    return PKV_OK;
}

int seq_cache_tokens(pkv_pool* p, int32_t s, int32_t start, const int32_t* tokens, int32_t n, int32_t* out_keyed) {
    if (!p || !out_keyed || n < 0 || (n > 0 && !tokens)) return fail(PKV_ERR_INVALID, "seq_cache_tokens: bad arguments");
    int st = PKV_OK;
    Sequence* q = p->resident(s, &st);
    if (!q) return st;
    if (static_cast<int64_t>(start) != static_cast<int64_t>(q->keys.size()) * kBlock ||
        static_cast<int64_t>(start) + n > q->len)
        return fail(PKV_ERR_INVALID, "seq_cache_tokens: tokens must start at position %zu (the first unkeyed block) "
                    "and lie inside the sequence's %d tokens", q->keys.size() * kBlock, q->len);
    uint64_t parent = q->keys.empty() ? 0 : q->keys.back();
    const int32_t n_full = n / kBlock;
    for (int32_t j = 0; j < n_full; ++j) {
        const int32_t* ids = tokens + static_cast<int64_t>(j) * kBlock;
        const uint64_t key = block_key(parent, q->tenant, ids);
        const int32_t b = q->blocks[q->keys.size()];
        if (!p->registered[b] && p->cache.find(key) == p->cache.end()) {
            CacheEntry e;
            e.block = b;
            e.parent = parent;
            e.tenant = q->tenant;
            std::memcpy(e.ids, ids, sizeof(e.ids));
            p->cache.emplace(key, e);
            p->key_of[b] = key;
            p->registered[b] = 1;
        }
        q->keys.push_back(key);
        parent = key;
    }
    *out_keyed = n_full;
    return PKV_OK;
}

int seq_len(const pkv_pool* p, int32_t s, int32_t* out_len) {
    if (!p || !out_len) return fail(PKV_ERR_INVALID, "seq_len: null argument");
    int st = PKV_OK;
    const Sequence* q = const_cast<pkv_pool*>(p)->find(s, &st);
    if (!q) return st;
    *out_len = q->len;
    return PKV_OK;
}

int seq_num_blocks(const pkv_pool* p, int32_t s, int32_t* out_n) {
    if (!p || !out_n) return fail(PKV_ERR_INVALID, "seq_num_blocks: null argument");
    int st = PKV_OK;
    const Sequence* q = const_cast<pkv_pool*>(p)->resident(s, &st);
    if (!q) return st;
    *out_n = static_cast<int32_t>(q->blocks.size());
    return PKV_OK;
}

int block_table_build(const pkv_pool* p, const int32_t* seqs, int32_t n, int32_t max_blocks, int32_t* out_table,
                      int32_t* out_lens) {
    if (!p || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !out_lens || (max_blocks > 0 && !out_table))))
        return fail(PKV_ERR_INVALID, "block_table_build: bad arguments");
    for (int32_t i = 0; i < n; ++i) {
        int st = PKV_OK;
        const Sequence* q = const_cast<pkv_pool*>(p)->resident(seqs[i], &st);
        if (!q) return st;
        if (static_cast<int64_t>(q->blocks.size()) > max_blocks)
            return fail(PKV_ERR_INVALID, "sequence %d has %zu blocks > max_blocks %d", seqs[i], q->blocks.size(), max_blocks);
    }
    for (int32_t i = 0; i < n; ++i) {
        const Sequence& q = p->seqs[seqs[i]];
        int32_t* row = out_table + static_cast<int64_t>(i) * max_blocks;
        std::copy(q.blocks.begin(), q.blocks.end(), row);
        std::fill(row + q.blocks.size(), row + max_blocks, -1);
        out_lens[i] = q.len;
    }
    return PKV_OK;
}

}  // extern "C"
