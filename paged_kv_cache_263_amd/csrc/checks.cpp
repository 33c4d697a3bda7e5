// Host-side validation of the device entry points' arguments.
#include "internal.h"

namespace pkv {

int check_cache(const pkv_cache* c) {
    if (!c) return fail(PKV_ERR_INVALID, "null cache descriptor");
    if (c->block_size != PKV_BLOCK_SIZE) return fail(PKV_ERR_UNSUPPORTED, "block size %d (only 16)", c->block_size);
    if (c->head_dim != PKV_HEAD_DIM) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (only 128)", c->head_dim);
    if (c->kv_dtype != PKV_F32 && c->kv_dtype != PKV_BF16 && c->kv_dtype != PKV_FP8_E4M3)
        return fail(PKV_ERR_INVALID, "unknown kv dtype %d", c->kv_dtype);
    if (c->num_layers <= 0 || c->num_blocks <= 0 || c->num_kv_heads <= 0)
        return fail(PKV_ERR_INVALID, "bad cache shape (layers %d, blocks %d, kv heads %d)", c->num_layers,
                    c->num_blocks, c->num_kv_heads);
    if (static_cast<int64_t>(c->num_blocks) * PKV_BLOCK_SIZE > INT32_MAX)
        return fail(PKV_ERR_INVALID, "too many blocks for int32 slots");
    if (!c->k_pool || !c->v_pool) return fail(PKV_ERR_INVALID, "null K or V pool");
    if (c->kv_dtype == PKV_FP8_E4M3 && (!c->k_scale || !c->v_scale))
        return fail(PKV_ERR_INVALID, "fp8 cache needs k_scale and v_scale");
    return PKV_OK;
}

int check_attn(const pkv_cache* c, const pkv_attn_args* a) {
    int st = check_cache(c);
    if (st) return st;
    if (!a) return fail(PKV_ERR_INVALID, "null attention arguments");
    if (a->layer < 0 || a->layer >= c->num_layers) return fail(PKV_ERR_INVALID, "layer %d out of range", a->layer);
    const bool ok = (a->q_dtype == PKV_F32 && c->kv_dtype == PKV_F32) ||
                    (a->q_dtype == PKV_BF16 && (c->kv_dtype == PKV_BF16 || c->kv_dtype == PKV_FP8_E4M3));
    if (!ok) return fail(PKV_ERR_UNSUPPORTED, "q dtype %d with kv dtype %d", a->q_dtype, c->kv_dtype);
    if (a->num_q_heads <= 0 || a->num_q_heads % c->num_kv_heads != 0)
        return fail(PKV_ERR_INVALID, "%d query heads is not a multiple of %d kv heads", a->num_q_heads, c->num_kv_heads);
    if (a->num_q_heads / c->num_kv_heads > 16)
        return fail(PKV_ERR_UNSUPPORTED, "more than 16 query heads per kv head");
    if (a->num_seqs < 0) return fail(PKV_ERR_INVALID, "negative num_seqs");
    if (a->num_seqs == 0) return PKV_OK;
    if (!a->q || !a->out || !a->block_table || !a->kv_lens) return fail(PKV_ERR_INVALID, "null q/out/table/kv_lens");
    if (a->max_blocks <= 0 || a->max_kv_len <= 0)
        return fail(PKV_ERR_INVALID, "max_blocks %d / max_kv_len %d must be positive", a->max_blocks, a->max_kv_len);
    if (static_cast<int64_t>(a->max_kv_len) > static_cast<int64_t>(a->max_blocks) * PKV_BLOCK_SIZE)
        return fail(PKV_ERR_INVALID, "max_kv_len %d exceeds max_blocks * 16", a->max_kv_len);
    if (a->split_tokens != 0 && (a->split_tokens % PKV_BLOCK_SIZE != 0 || a->split_tokens < 16 || a->split_tokens > 1024))
        return fail(PKV_ERR_INVALID, "split_tokens %d must be 0 or a multiple of 16 in [16, 1024]", a->split_tokens);
    const uintptr_t align = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->out) |
                            reinterpret_cast<uintptr_t>(c->k_pool) | reinterpret_cast<uintptr_t>(c->v_pool) |
                            reinterpret_cast<uintptr_t>(a->workspace);
    if (align & 15u) return fail(PKV_ERR_INVALID, "q, out, pools and workspace must be 16-byte aligned");
    return PKV_OK;
}

int32_t decode_split_tokens(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, int32_t max_kv_len) {
    if (a->split_tokens) return a->split_tokens;
    // The largest chunk that still gives ~8K work items (32 per CU): long rows
    // get long chunks (fewer partial results to write and merge), short
    // batches get short ones (enough work items to fill 256 CUs).
    const int64_t pairs = static_cast<int64_t>(rows) * c->num_kv_heads;
    for (int32_t st : {1024, 512, 256, 128}) {
        if (pairs * ((max_kv_len + st - 1) / st) >= 8192) return st;
    }
    return 64;
}

size_t decode_workspace_bytes(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, int32_t max_kv_len) {
    if (rows <= 0) return 0;
    const int32_t st = decode_split_tokens(c, a, rows, max_kv_len);
    const int64_t splits = (max_kv_len + st - 1) / st;
    if (splits <= 1) return 0;
    return static_cast<size_t>(rows) * a->num_q_heads * splits * (PKV_HEAD_DIM + 2) * sizeof(float);
}

}  // namespace pkv
