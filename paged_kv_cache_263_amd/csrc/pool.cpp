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
#include <algorithm>
#include <new>
#include <vector>

#include "internal.h"

using pkv::fail;

namespace {

constexpr int32_t kBlock = PKV_BLOCK_SIZE;

struct Sequence {
    std::vector<int32_t> blocks;  // logical block index -> physical block id
    int32_t len = 0;
    bool live = false;
    bool swapped = false;  // blocks are in host memory; the table is empty
};

inline int32_t blocks_for(int64_t tokens) { return static_cast<int32_t>((tokens + kBlock - 1) / kBlock); }

}  // namespace

struct pkv_pool {
    int32_t num_blocks = 0;
    std::vector<int32_t> free_stack;  // back() is handed out next
    std::vector<int32_t> ref;
    std::vector<Sequence> seqs;       // index = sequence id
    int64_t cow_count = 0;
    int64_t live_seqs = 0;

    int32_t take() {
        int32_t b = free_stack.back();
        free_stack.pop_back();
        ref[b] = 1;
        return b;
    }
    void drop(int32_t b) {
        if (--ref[b] == 0) free_stack.push_back(b);
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
    if (static_cast<size_t>(n) > p->free_stack.size())
        return fail(PKV_ERR_OOM, "kv_pool_alloc: need %d blocks, %zu free", n, p->free_stack.size());
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
    if (need > static_cast<int64_t>(p->free_stack.size()))
        return fail(PKV_ERR_OOM, "seq_append: need %lld blocks, %zu free", static_cast<long long>(need), p->free_stack.size());
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
    if (need > static_cast<int64_t>(p->free_stack.size()))
        return fail(PKV_ERR_OOM, "seq_append_batch: need %lld blocks, %zu free", static_cast<long long>(need),
                    p->free_stack.size());
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
    *out_seq = c;
    return PKV_OK;
}

int seq_free(pkv_pool* p, int32_t s) {
    if (!p) return fail(PKV_ERR_INVALID, "seq_free: null pool");
    int st = PKV_OK;
    Sequence* q = p->find(s, &st);
    if (!q) return st;
    for (int32_t b : q->blocks) p->drop(b);
    q->blocks.clear();
    q->blocks.shrink_to_fit();
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
    for (int32_t b : q->blocks) p->drop(b);
    q->blocks.clear();
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
    if (static_cast<size_t>(n) > p->free_stack.size())
        return fail(PKV_ERR_OOM, "seq_swap_in: need %d blocks, %zu free", n, p->free_stack.size());
    q->blocks.resize(n);
    for (int32_t j = 0; j < n; ++j) q->blocks[j] = p->take();
    std::copy(q->blocks.begin(), q->blocks.end(), out_ids);
    q->swapped = false;
    *n_out = n;
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
