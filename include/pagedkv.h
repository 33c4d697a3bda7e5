/*
 * pagedkv.h - C ABI of a paged KV-cache attention library for AMD MI355X (gfx950).
 *
 * What the library does comes from three pages on paged KV caches:
 *   [P1] "PagedAttention, chunked prefill, and the launch that cascades" (deepnotes.pages.dev)
 *   [P2] "Waste, and three ways to reclaim it" (runbooks.in, LLM Inference Runbook, document 10)
 *   [P3] "M.65 Inference Serving" (systemdesigntutorial.com)
 *
 * The KV cache lives in fixed 16-token blocks scattered through a pool; each
 * sequence reaches its blocks through a block table; blocks are reference
 * counted so that identical prefixes are stored once, and a sequence that must
 * write into a shared block gets its own copy first.  Attention reads K/V
 * through the table ([P2] "PagedAttention - operating-system virtual memory,
 * applied to attention"; [P3] "PagedAttention block management").
 *
 * Conventions for every function:
 *  - The return value is a status: PKV_OK (0) or a negative PKV_ERR_* code.
 *    Nothing throws across this ABI.  pkv_last_error() returns a message for
 *    the last failing call on the calling thread.
 *  - "host" pointers are ordinary CPU memory; "device" pointers are GPU memory
 *    allocated by the caller.  The library never allocates or frees device
 *    memory and never synchronises a stream: kernels and copies are enqueued
 *    on the caller's stream (a hipStream_t passed as void*, NULL = the null
 *    stream).  Faults inside kernels surface when the caller synchronises.
 *  - A pkv_pool holds host metadata only (free list, refcounts, tables).  It
 *    is not thread safe: the caller serialises calls on one pool.
 *  - The block size is fixed at 16 tokens ([P3] item (a): fixed at compile
 *    time, 16 by default) and the head dimension at 128.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_BLOCK_SIZE 16
#define PKV_HEAD_DIM 128

enum {
    PKV_OK = 0,
    PKV_ERR_INVALID = -1,     /* bad argument: null pointer, size out of range, unknown id */
    PKV_ERR_OOM = -2,         /* not enough free blocks; nothing was changed */
    PKV_ERR_STATE = -3,       /* double free, refcount underflow, use of a freed sequence */
    PKV_ERR_UNSUPPORTED = -4, /* block size != 16, head_dim != 128, dtype combination */
    PKV_ERR_HIP = -5,         /* a HIP runtime call (launch, copy) failed */
    PKV_ERR_WORKSPACE = -6    /* workspace missing or smaller than paged_attn_workspace_size() */
};

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2, PKV_INT8 = 3 } pkv_dtype;

/* ------------------------------------------------------------------------
 * Host block allocator, sequences and block tables
 * ([P1] "PagedAttention: an OS idea, not an ML one"; [P3] "PagedAttention
 * block management" items (b) table per request, (c) a block from the free
 * list every 16 tokens, returned when the request completes, (e) refcounts,
 * (g) copy-on-write; [P2] "Sharing, and what makes a prefix reusable").
 *
 * Policy (the pages leave it open): at first blocks are handed out in the
 * order given to kv_pool_create (identity if NULL); the free list is a stack,
 * so a freed block is the next one handed out.  Every request for blocks is
 * all-or-nothing: PKV_ERR_OOM leaves the pool exactly as it was, so that the
 * caller can preempt or refuse admission ([P2] "When it runs out anyway").
 * ------------------------------------------------------------------------ */

typedef struct pkv_pool pkv_pool; /* opaque */

/* A copy the caller must perform (kv_copy_blocks) before writing the token
 * that caused it: block src's contents go to block dst.  valid_tokens is the
 * number of tokens of src in use (the rest of the block is unwritten). */
typedef struct {
    int32_t src;
    int32_t dst;
    int32_t valid_tokens;
} pkv_copy;

typedef struct {
    int32_t num_blocks;
    int32_t free_blocks;
    int32_t used_blocks;   /* refcount > 0 */
    int32_t shared_blocks; /* refcount > 1 */
    int64_t refcount_sum;
    int64_t cow_count;     /* copies planned so far */
    int64_t num_seqs;      /* live sequences */
    int64_t tokens;        /* sum of live sequence lengths */
    int64_t waste_tokens;  /* sum over resident sequences of blocks*16 - length (each <= 15) */
    int64_t swapped_seqs;  /* live sequences swapped out to host memory */
    int64_t swapped_tokens;/* their lengths (tokens counts resident sequences only) */
    int64_t cached_blocks; /* blocks registered in the prefix cache */
    int64_t evictable_blocks; /* registered blocks with no reference, kept for reuse */
    int64_t matched_tokens;/* tokens matched by seq_create_cached so far */
} pkv_stats;

/* Create a pool of num_blocks blocks (block_size must be 16).  order: host,
 * NULL or a permutation of 0..num_blocks-1 giving the order in which blocks
 * are first handed out.  *out receives the handle (free with kv_pool_destroy). */
int kv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* order, pkv_pool** out);
void kv_pool_destroy(pkv_pool* pool);

/* Take n blocks off the free list (all or nothing); each gets refcount 1.
 * out_ids: host [n], ids in the order taken. */
int kv_pool_alloc(pkv_pool* pool, int32_t n, int32_t* out_ids);
/* Add one reference to each listed block (each must be in use). */
int kv_pool_incref(pkv_pool* pool, const int32_t* ids, int32_t n);
/* Drop one reference from each listed block; a block reaching 0 goes back on
 * the free list, in list order.  Checked first: an underflow changes nothing
 * and returns PKV_ERR_STATE. */
int kv_pool_free(pkv_pool* pool, const int32_t* ids, int32_t n);
int kv_pool_refcount(const pkv_pool* pool, int32_t block, int32_t* out);
int kv_pool_stats(const pkv_pool* pool, pkv_stats* out);
/* Copy the free list, bottom to top (the top is handed out next), into
 * out[cap]; *n receives its length (PKV_ERR_INVALID if cap is too small). */
int kv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n);
/* Copy the evictable list (retained prefix-cache blocks with no reference),
 * least recently used first, into out[cap]; *n receives its length. */
int kv_pool_evictable_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n);

/* Sequence ids are 0, 1, 2, ... in creation order and are never reused. */
int seq_create(pkv_pool* pool, int32_t* out_seq);
/* Grow sequence seq by n_tokens (>= 0).  Blocks are taken on demand, one each
 * time a token starts a new block.  If the sequence's partial last block is
 * shared (refcount > 1) it is first replaced by a fresh block and the copy is
 * reported in out_copy[0] (*n_copy = 1; at most one per call), else
 * *n_copy = 0.  out_slots: host [n_tokens]; slot of token t = block*16 + t%16.
 * All or nothing: PKV_ERR_OOM changes nothing. */
int seq_append(pkv_pool* pool, int32_t seq, int32_t n_tokens, int32_t* out_slots,
               pkv_copy* out_copy, int32_t* n_copy);
/* seq_append for n distinct sequences at once (all or nothing over the whole
 * batch).  n_tokens: host [n]; out_slots: host [sum n_tokens], grouped by
 * sequence in list order; out_copies: host [n]; *n_copies receives how many. */
int seq_append_batch(pkv_pool* pool, const int32_t* seqs, const int32_t* n_tokens, int32_t n,
                     int32_t* out_slots, pkv_copy* out_copies, int32_t* n_copies);
/* New sequence sharing every block of parent, the partial last one included
 * (parallel sampling, [P3] item (g)). */
int seq_fork(pkv_pool* pool, int32_t parent, int32_t* out_child);
/* New sequence sharing the first n_tokens of src; n_tokens must be a multiple
 * of 16 (prefix matching is block aligned, [P2] "Fast answers"). */
int seq_share_prefix(pkv_pool* pool, int32_t src, int32_t n_tokens, int32_t* out_seq);
/* Drop one reference to each block of seq, in logical order; seq is gone
 * (a swapped-out sequence holds no blocks and is simply removed). */
int seq_free(pkv_pool* pool, int32_t seq);
int seq_len(const pkv_pool* pool, int32_t seq, int32_t* out_len);
int seq_num_blocks(const pkv_pool* pool, int32_t seq, int32_t* out_n);

/* Swapping a sequence to host memory when blocks run out ([P2] "When it runs
 * out anyway": a preempted request's blocks move across the host link to CPU
 * memory and come back later; [P3] "M.65 Inference Serving": the same
 * spill-and-reload of blocks).
 * seq_swap_out: out_ids host [cap] receives seq's block ids in logical order
 * (*n_out = ceil(len / 16)); then one reference is dropped from each, in that
 * order, and seq is swapped out: it keeps its length and holds no blocks.
 * Copy those blocks to host memory (kv_swap_out) on the stream before any of
 * them can be written again.  seq_swap_in: takes ceil(len / 16) blocks (all
 * or nothing: PKV_ERR_OOM changes nothing) and returns them in logical order
 * in out_ids; copy the host copy into them with kv_swap_in.  A swapped-out
 * sequence cannot be appended to, forked, shared, swapped out again, counted
 * by seq_num_blocks or put in a block table (PKV_ERR_STATE); seq_len and
 * seq_free work.  Blocks that were shared when it left come back as private
 * copies.  cap smaller than the block count is PKV_ERR_INVALID (nothing
 * changes). */
int seq_swap_out(pkv_pool* pool, int32_t seq, int32_t* out_ids, int32_t cap, int32_t* n_out);
int seq_swap_in(pkv_pool* pool, int32_t seq, int32_t* out_ids, int32_t cap, int32_t* n_out);

/* Prefix caching with retention ([P1] "PagedAttention ...": hash a shared
 * prefix and reuse its blocks instead of recomputing them; [P2] "Sharing, and
 * what makes a prefix reusable": a finished request's cache is kept and new
 * requests match against it on exact token ids, block-aligned, from the very
 * start; [P2] "The isolation question": key the cache per tenant).
 *   Keys: full block j of a sequence has key_j = FNV-1a-64 over the
 *   little-endian bytes of key_{j-1} (8 bytes; 0 for the first block), the
 *   tenant (4 bytes) and its 16 token ids (4 bytes each).  An entry keeps the
 *   key, block, parent key, tenant and ids; a match needs all of them equal,
 *   so a hash collision cannot match wrong content.
 *   Retention: a registered block whose last reference drops goes to the
 *   evictable list instead of the free list (a sequence dropping several at
 *   once lists its deeper blocks as older).  Blocks are taken from the free
 *   list first, then from the evictable list, least recently used first, which
 *   removes the block's entry; every all-or-nothing check counts both lists.
 *   fork and seq_share_prefix carry the tenant and keys of the shared blocks;
 *   seq_swap_out forgets them (blocks come back private and unregistered).
 * seq_create_cached: a new sequence of the given tenant holding the longest
 * run of leading full blocks of tokens[0..n) found in the cache, at most n - 1
 * tokens (one token is always left to compute); *out_matched receives its
 * length (a multiple of 16).  Matched blocks gain a reference (and leave the
 * evictable list).  Append the remaining tokens with seq_append.
 * seq_cache_tokens: key and register the full blocks of seq covering
 * positions start .. start + n - 1, whose token ids are tokens[0..n); start
 * must be 16 x the blocks already keyed (seq_create_cached's *out_matched, then
 * advancing by 16 x *out_keyed) and the positions must lie inside the sequence
 * (PKV_ERR_INVALID otherwise).  A block whose key is already registered to
 * another block stays unregistered.  *out_keyed = n / 16. */
int seq_create_cached(pkv_pool* pool, int32_t tenant, const int32_t* tokens, int32_t n, int32_t* out_seq,
                      int32_t* out_matched);
int seq_cache_tokens(pkv_pool* pool, int32_t seq, int32_t start, const int32_t* tokens, int32_t n,
                     int32_t* out_keyed);

/* Block table rows for n sequences: out_table host [n][max_blocks] (physical
 * block ids, padded with -1), out_lens host [n].  A sequence with more than
 * max_blocks blocks is PKV_ERR_INVALID.  The caller uploads both. */
int block_table_build(const pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                      int32_t* out_table, int32_t* out_lens);

/* ------------------------------------------------------------------------
 * Device cache and kernels
 * ------------------------------------------------------------------------ */

/* Device KV cache, owned by the caller.  One block id addresses every layer.
 *   k_pool: [num_layers][num_blocks][num_kv_heads][16 tokens][head_dim]
 *   v_pool: [num_layers][num_blocks][num_kv_heads][head_dim][16 tokens]
 * (V is stored token-minor inside a block so that the P.V contraction over
 * tokens reads contiguous memory.)  One-byte V tiles (fp8 and int8: 16 x 128
 * codes, 2 KiB) keep (d, token) at byte (token / 4) * 512 + (d / 64) * 256 +
 * (d % 16) * 16 + ((d / 16) % 4) * 4 + token % 4, so the decode kernel reads
 * them with 16-byte loads that cover whole 256-byte runs.  bf16 tiles (4 KiB)
 * keep K (token, d) at element (d / 8) * 128 + token * 8 + d % 8 and V
 * (d, token) at element (d / 32) * 512 + ((token / 4) * 16 + d % 16) * 8 +
 * ((d / 16) % 2) * 4 + token % 4, so every load instruction of the decode
 * kernel reads 1 KiB contiguously.  fp32 tiles keep the plain orders above.
 * Only the library's kernels read or write inside a tile.  Elements are kv_dtype.  Stored value = e4m3(code) * scale for fp8
 * ([P2] "Quantising the cache") and code * scale for int8 (a signed byte in
 * -127..127; [P3] "M.65 Inference Serving", quantisation of the KV cache),
 * with one fp32 scale per (layer, kv head) for K (k_scale [num_layers]
 * [num_kv_heads]) and for V (v_scale); NULL for f32 and bf16. */
typedef struct {
    int32_t kv_dtype;     /* pkv_dtype */
    int32_t num_layers;
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t head_dim;     /* must be 128 */
    int32_t block_size;   /* must be 16 */
    void* k_pool;
    void* v_pool;
    const float* k_scale;
    const float* v_scale;
} pkv_cache;

/* Arguments of an attention call.  Supported (q_dtype, kv_dtype) pairs:
 * (F32, F32), (BF16, BF16), (BF16, FP8_E4M3), (BF16, INT8).  out has q's
 * dtype and shape.
 * GQA: query head h reads kv head h / (num_q_heads / num_kv_heads). */
typedef struct {
    int32_t layer;
    int32_t q_dtype;
    int32_t num_seqs;            /* batch rows */
    int32_t num_q_heads;         /* multiple of num_kv_heads, at most 16 per kv head */
    const void* q;               /* device [total_q][num_q_heads][head_dim] */
    void* out;                   /* device, same shape and dtype as q */
    const int32_t* block_table;  /* device [num_seqs][max_blocks], row i for batch row i */
    int32_t max_blocks;
    const int32_t* kv_lens;      /* device [num_seqs]: cached tokens per row, >= 1 */
    int32_t max_kv_len;          /* host: upper bound on kv_lens (sizes the launch); num_seqs x ceil(max_kv_len / 16) must be below 2^31 (PKV_ERR_INVALID otherwise) */
    /* prefill only (paged_attn_prefill_chunk): */
    const int32_t* cu_q;         /* device [num_seqs + 1]: row i's queries are cu_q[i]..cu_q[i+1]-1 */
    int32_t num_decode;          /* rows 0..num_decode-1 have exactly one query (cu_q[i] = i) */
    int32_t max_decode_kv_len;   /* host: bound on the decode rows' kv_lens (0 = max_kv_len) */
    int32_t max_q_len;           /* host: upper bound on the other rows' query counts (a chunk row
                                    with more queries is invalid: all its outputs are NaN) */
    int32_t total_q;             /* host: cu_q[num_seqs] */
    /* tuning and scratch: */
    int32_t decode_parts;        /* decode: the blocks of each kv head are divided evenly among this
                                    many wavefronts (<= 4096, and at most one per 8 blocks of the
                                    head's work); 0 = auto (8 per compute unit in all, 12 for a
                                    one-byte cache) */
    int32_t prefill_parts;       /* prefill: key ranges each tile of query rows is split into
                                    (1..8; their states are merged by a second kernel);
                                    0 = auto (enough workgroups for one per compute unit) */
    int32_t shared_prefix_blocks;/* decode only: the caller promises that the first
                                    shared_prefix_blocks entries of every row's block table are the
                                    same block ids (a prefix all rows share); the call then computes
                                    attention over those blocks once for all rows and continues each
                                    row from there.  Each row's kv_lens must be at least 16 times
                                    this (else the row is invalid).  The promise is checked on the
                                    device: a row whose first shared_prefix_blocks ids differ from
                                    row 0's gets NaN output, the other rows are unaffected.
                                    0 = no promise. */
    void* workspace;             /* device scratch: row plan and partial results */
    size_t workspace_bytes;
    /* optional profiling: hipEvent_t handles (NULL entries are skipped) that
     * the call records on its stream: [0] just before the decode kernel (after
     * the plan kernel that batches of more than 1024 rows need; with a shared
     * prefix, before the one launch that runs the shared-prefix pass and the
     * decode), [1] after it, [2] after the decode merge kernel, [3] after the
     * prefill kernel.  The caller owns the events. */
    void* events[4];
} pkv_attn_args;

/* Bytes of workspace paged_attn_decode / paged_attn_prefill_chunk need for
 * these arguments (0 if none). */
int paged_attn_workspace_size(const pkv_cache* cache, const pkv_attn_args* args, size_t* bytes);

/* Decode: one query per row over its kv_lens[i] cached tokens, read through
 * the block table ([P3] item (d): the attention kernel reads K/V from
 * non-contiguous blocks through the table); softmax(q K^T / sqrt(d)) V with a
 * running max and normaliser over blocks ([P1] "FlashAttention: why the
 * mechanism this whole layer runs on isn't compute-bound").  The blocks of
 * all rows are divided evenly among decode_parts wavefronts per kv head; rows
 * cut between wavefronts are merged by a second kernel.  The arithmetic order
 * depends on logical positions only, so any placement of the blocks gives
 * bit-identical output.  A row with an invalid length or an out-of-range
 * block id gets NaN output. */
/* With shared_prefix_blocks = S > 0 (the rows' tables all start with the same
 * S block ids: a shared prefix, [P2] "Sharing, and what makes a prefix
 * reusable"), the call computes, on the matrix cores, every row's attention
 * state (running max, normaliser, unnormalised output) over the 16 S prefix
 * tokens, reading those blocks once per kv head instead of once per row, in
 * the same launch as the decode over each row's remaining blocks; the merge
 * kernel combines the two states.  The result is the same attention (a
 * different summation order); it is still independent of where the blocks
 * sit. */
int paged_attn_decode(const pkv_cache* cache, const pkv_attn_args* args, void* stream);

/* paged_attn_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops and harnesses that forbid hipMalloc):
 * the same kernels and result, with the workspace taken from a fixed array of
 * PKV_NOALLOC_SCRATCH_BYTES in device memory that the library holds on each
 * GPU it runs on until the process ends.  args->workspace must be NULL and
 * workspace_bytes 0.  A call whose paged_attn_workspace_size exceeds
 * PKV_NOALLOC_SCRATCH_BYTES is PKV_ERR_WORKSPACE (nothing launched).  The
 * call allocates nothing.  stream must belong to the current device.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams with no ordering between them) race; calls on one stream
 * are safe. */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int paged_attn_decode_noalloc(const pkv_cache* cache, const pkv_attn_args* args, void* stream);

/* Chunked prefill batched with decode rows ([P1] "Serving systems: the layer
 * that survives real traffic"; [P3] "prefill vs decode phase separation",
 * item (e)).  Rows 0..num_decode-1 are decode rows; each other row i holds
 * C_i = cu_q[i+1]-cu_q[i] queries that are the last C_i of its kv_lens[i]
 * cached tokens (their K/V already written), and query j attends keys
 * 0..kv_lens[i]-C_i+j (causal, bottom-right aligned).  Chunk rows need a
 * bf16, fp8 or int8 cache (PKV_ERR_UNSUPPORTED for fp32).  A chunk row with an
 * invalid length or block id, or with more queries than max_q_len, gets NaN
 * output.  The kernels trust cu_q to be non-decreasing and within
 * 0..total_q: a row whose cu_q entries are not is left unwritten (its output
 * place is unknown). */
int paged_attn_prefill_chunk(const pkv_cache* cache, const pkv_attn_args* args, void* stream);

/* Write n_tokens new tokens' K and V into the cache at their slots (fp8:
 * code = e4m3 round-to-nearest-even of fp32(x / scale), saturating at +-448;
 * int8: code = fp32(x / scale) rounded half to even, clamped to +-127).
 *   k_new, v_new: device [n_tokens][num_kv_heads][head_dim] of val_dtype
 *                 (F32 for an F32 cache, BF16 for BF16, FP8 and INT8 caches)
 *   slots:        [n_tokens], slot = block*16 + offset (from seq_append)
 * slots, rows and positions may be device memory or pinned host memory mapped
 * for the device (hipHostMalloc); the kernel then reads them over the host
 * link, and the host must not change them until the call has run.
 * A slot outside the pool is skipped (the kernel cannot report it).
 * Optional device block-table upkeep (pass NULL block_table to skip): token i
 * belongs to batch row rows[i] (0 <= rows[i] < num_rows; block_table is
 * [num_rows][max_blocks], kv_lens [num_rows]) at position positions[i]; the
 * call sets
 * block_table[rows[i]][positions[i]/16] = slots[i]/16 and, for the last token
 * of each row (tokens of one row must be consecutive and increasing),
 * kv_lens[rows[i]] = positions[i] + 1. */
int kv_cache_write(const pkv_cache* cache, int32_t layer, int32_t n_tokens, int32_t val_dtype,
                   const void* k_new, const void* v_new, const int32_t* slots,
                   const int32_t* rows, const int32_t* positions, int32_t num_rows,
                   int32_t* block_table, int32_t max_blocks, int32_t* kv_lens, void* stream);

/* Copy whole blocks (all layers, K and V) for the copy-on-write operations
 * reported by seq_append.  copies: host [n]; enqueued on stream. */
int kv_copy_blocks(const pkv_cache* cache, const pkv_copy* copies, int32_t n, void* stream);

/* Bytes one block takes in a swap buffer: num_layers * 2 (K, V) *
 * num_kv_heads * 16 * head_dim * element size. */
int kv_swap_block_bytes(const pkv_cache* cache, size_t* out_bytes);
/* Move n whole blocks (all layers, K and V) between the device cache and a
 * host swap buffer over the host link ([P2] "When it runs out anyway").
 *   ids:  host [n], block ids (each in range; they need not be distinct for
 *         kv_swap_out, must be for kv_swap_in)
 *   host: pinned host memory (hipHostMalloc or torch pin_memory) of n *
 *         kv_swap_block_bytes; block i occupies bytes [i * B, (i + 1) * B) as
 *         [layer][K, V][kv head][the cache's own tile bytes].  Memory that is
 *         not pinned is PKV_ERR_INVALID.
 * kv_swap_out copies blocks ids[i] -> host slot i; kv_swap_in copies host
 * slot i -> block ids[i].  Both are kernels on stream that read or write the
 * host memory directly; the host must not touch the buffer until the stream
 * has passed them. */
int kv_swap_out(const pkv_cache* cache, const int32_t* ids, int32_t n, void* host, void* stream);
int kv_swap_in(const pkv_cache* cache, const void* host, const int32_t* ids, int32_t n, void* stream);

/* Messages. */
const char* pkv_strerror(int status);
const char* pkv_last_error(void);
int pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
