// Host-side validation of the device entry points' arguments.
#include "internal.h"

namespace pkv {

int check_cache(const pkv_cache* c) {
    if (!c) return fail(PKV_ERR_INVALID, "null cache descriptor");
    if (c->block_size != PKV_BLOCK_SIZE) return fail(PKV_ERR_UNSUPPORTED, "block size %d (only 16)", c->block_size);
    if (c->head_dim != PKV_HEAD_DIM) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (only 128)", c->head_dim);
    if (c->kv_dtype != PKV_F32 && c->kv_dtype != PKV_BF16 && c->kv_dtype != PKV_FP8_E4M3 && c->kv_dtype != PKV_INT8)
        return fail(PKV_ERR_INVALID, "unknown kv dtype %d", c->kv_dtype);
    if (c->num_layers <= 0 || c->num_blocks <= 0 || c->num_kv_heads <= 0)
        return fail(PKV_ERR_INVALID, "bad cache shape (layers %d, blocks %d, kv heads %d)", c->num_layers,
                    c->num_blocks, c->num_kv_heads);
    if (static_cast<int64_t>(c->num_blocks) * PKV_BLOCK_SIZE > INT32_MAX)
        return fail(PKV_ERR_INVALID, "too many blocks for int32 slots");
    if (!c->k_pool || !c->v_pool) return fail(PKV_ERR_INVALID, "null K or V pool");
    if ((c->kv_dtype == PKV_FP8_E4M3 || c->kv_dtype == PKV_INT8) && (!c->k_scale || !c->v_scale))
        return fail(PKV_ERR_INVALID, "fp8 and int8 caches need k_scale and v_scale");
    return PKV_OK;
}

int check_attn(const pkv_cache* c, const pkv_attn_args* a) {
    int st = check_cache(c);
    if (st) return st;
    if (!a) return fail(PKV_ERR_INVALID, "null attention arguments");
    if (a->layer < 0 || a->layer >= c->num_layers) return fail(PKV_ERR_INVALID, "layer %d out of range", a->layer);
    const bool ok = (a->q_dtype == PKV_F32 && c->kv_dtype == PKV_F32) ||
                    (a->q_dtype == PKV_BF16 && (c->kv_dtype == PKV_BF16 || c->kv_dtype == PKV_FP8_E4M3 ||
                                                c->kv_dtype == PKV_INT8));
    if (!ok) return fail(PKV_ERR_UNSUPPORTED, "q dtype %d with kv dtype %d", a->q_dtype, c->kv_dtype);
    if (a->num_q_heads <= 0 || a->num_q_heads % c->num_kv_heads != 0)
        return fail(PKV_ERR_INVALID, "%d query heads is not a multiple of %d kv heads", a->num_q_heads, c->num_kv_heads);
    if (a->num_q_heads / c->num_kv_heads > 16)
        return fail(PKV_ERR_UNSUPPORTED, "more than 16 query heads per kv head");
    if (a->num_seqs < 0) return fail(PKV_ERR_INVALID, "negative num_seqs");
    if (a->shared_prefix_blocks < 0 || a->shared_prefix_blocks > a->max_blocks)
        return fail(PKV_ERR_INVALID, "shared_prefix_blocks %d out of 0..max_blocks", a->shared_prefix_blocks);
    if (a->shared_prefix_blocks > 0 && a->cu_q)
        return fail(PKV_ERR_UNSUPPORTED, "a shared prefix is a decode-only option");
    if (a->shared_prefix_blocks > 0 && c->kv_dtype == PKV_F32)
        return fail(PKV_ERR_UNSUPPORTED, "a shared prefix needs a bf16, fp8 or int8 cache");
    if (a->num_seqs == 0) return PKV_OK;
    if (!a->q || !a->out || !a->block_table || !a->kv_lens) return fail(PKV_ERR_INVALID, "null q/out/table/kv_lens");
    if (a->max_blocks <= 0 || a->max_kv_len <= 0)
        return fail(PKV_ERR_INVALID, "max_blocks %d / max_kv_len %d must be positive", a->max_blocks, a->max_kv_len);
    if (static_cast<int64_t>(a->max_kv_len) > static_cast<int64_t>(a->max_blocks) * PKV_BLOCK_SIZE)
        return fail(PKV_ERR_INVALID, "max_kv_len %d exceeds max_blocks * 16", a->max_kv_len);
    // the kernels sum block counts over rows in 32 bits
    if (static_cast<int64_t>(a->num_seqs) * ((a->max_kv_len + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE) > INT32_MAX)
        return fail(PKV_ERR_INVALID, "num_seqs %d x ceil(max_kv_len %d / 16) blocks exceeds 2^31 - 1", a->num_seqs,
                    a->max_kv_len);
    if (a->decode_parts < 0 || a->decode_parts > 4096)
        return fail(PKV_ERR_INVALID, "decode_parts %d must be in [0, 4096]", a->decode_parts);
    if (a->prefill_parts < 0 || a->prefill_parts > 8)
        return fail(PKV_ERR_INVALID, "prefill_parts %d must be in [0, 8]", a->prefill_parts);
    const uintptr_t align = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->out) |
                            reinterpret_cast<uintptr_t>(c->k_pool) | reinterpret_cast<uintptr_t>(c->v_pool) |
                            reinterpret_cast<uintptr_t>(a->workspace);
    if (align & 15u) return fail(PKV_ERR_INVALID, "q, out, pools and workspace must be 16-byte aligned");
    return PKV_OK;
}

}  // namespace pkv
