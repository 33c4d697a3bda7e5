// Writes into the paged cache: new tokens' K/V to their slots (with fp8 or
// int8 quantisation on write), whole-block copies for copy-on-write, and
// swap copies of whole blocks to and from pinned host memory.
//
// A new block is needed every 16 tokens and a token's slot comes from the
// host allocator ([P3] "PagedAttention block management", item (c)); a
// sequence that must write into a shared block first gets its own copy ([P2]
// "Sharing, and what makes a prefix reusable"; [P3] item (g)).  The fp8 cache
// stores one byte per element ([P2] "Quantising the cache"): code = E4M3
// round-to-nearest-even of fp32(x / scale), saturating at +-448.  The int8
// cache ([P3] "M.65 Inference Serving", quantising the KV cache) stores
// code = fp32(x / scale) rounded half to even, clamped to +-127.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

struct WriteParams {
    const void* k_new;     // [n][hkv][128]
    const void* v_new;
    const int32_t* slots;  // [n]
    const int32_t* rows;   // [n] or null
    const int32_t* positions;
    int32_t* table;        // [num_rows][max_blocks] or null
    int32_t* kv_lens;      // [num_rows]
    void* k_pool;          // this layer
    void* v_pool;
    const float* k_scale;  // this layer [hkv]
    const float* v_scale;
    int32_t n, hkv, num_blocks, num_rows, max_blocks;
};

// Four consecutive d of one head of one token: the values as read, and
// their stores into the K tile ([16][128]; bf16: bf16_k_offset) and the V
// tile ([128][16]; bf16: bf16_v_offset; one-byte caches: byte_v_offset).
template <int KV>
struct Quad {
    // one-byte code of a value already divided by its scale
    static __device__ __forceinline__ uint32_t code(float x) {
        if constexpr (KV == PKV_INT8) return int8_code_rne(x);
        else return e4m3_code_rne(x);
    }
    using T = typename std::conditional<KV == PKV_F32, f32x4_t, u32x2_t>::type;  // 4 f32 or 4 bf16
    T k, v;
    __device__ __forceinline__ void load(const WriteParams& p, int64_t e) {  // e: element index, multiple of 4
        if constexpr (KV == PKV_F32) {
            k = ld<f32x4_t>(static_cast<const float*>(p.k_new) + e);
            v = ld<f32x4_t>(static_cast<const float*>(p.v_new) + e);
        } else {
            k = ld<u32x2_t>(static_cast<const uint16_t*>(p.k_new) + e);
            v = ld<u32x2_t>(static_cast<const uint16_t*>(p.v_new) + e);
        }
    }
    __device__ __forceinline__ void store(const WriteParams& p, int64_t tile, int o, int h, int d) const {
        if constexpr (KV == PKV_F32) {
            float* kp = static_cast<float*>(p.k_pool) + tile;
            float* vp = static_cast<float*>(p.v_pool) + tile;
            st<f32x4_t>(kp + o * kD + d, k);
#pragma unroll
            for (int j = 0; j < 4; ++j) vp[(d + j) * kBS + o] = v[j];
        } else if constexpr (KV == PKV_BF16) {
            uint16_t* kp = static_cast<uint16_t*>(p.k_pool) + tile;
            uint16_t* vp = static_cast<uint16_t*>(p.v_pool) + tile;
            st<u32x2_t>(kp + bf16_k_offset(o, d), k);
#pragma unroll
            for (int j = 0; j < 4; ++j) vp[bf16_v_offset(d + j, o)] = static_cast<uint16_t>(v[j >> 1] >> (16 * (j & 1)));
        } else {
            uint8_t* kp = static_cast<uint8_t*>(p.k_pool) + tile;
            uint8_t* vp = static_cast<uint8_t*>(p.v_pool) + tile;
            const float ks = p.k_scale[h];
            const float vs = p.v_scale[h];
            uint32_t kc = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float xk = __uint_as_float((k[j >> 1] >> (16 * (j & 1))) << 16);
                const float xv = __uint_as_float((v[j >> 1] >> (16 * (j & 1))) << 16);
                kc |= code(xk / ks) << (8 * j);
                vp[byte_v_offset(d + j, o)] = static_cast<uint8_t>(code(xv / vs));
            }
            st<uint32_t>(kp + o * kD + d, kc);
        }
    }
};

// One workgroup per token, one thread per four consecutive d of one head.
// Every load that depends on nothing else - slot, row and position (which
// may sit in host memory) and the thread's first four values - is issued
// before any is used, so the kernel waits for one round of loads.
template <int KV>
__global__ __launch_bounds__(256) void kv_write_kernel(const WriteParams p) {
    const int i = blockIdx.x;
    const int t = threadIdx.x;
    const int quads = p.hkv * (kD / 4);
    const int64_t first = static_cast<int64_t>(i) * p.hkv * kD;
    const int slot = p.slots[i];
    const bool upkeep = p.table != nullptr && t == 0;
    const int row = upkeep ? p.rows[i] : 0;
    const int pos = upkeep ? p.positions[i] : 0;
    const int next_row = (upkeep && i + 1 < p.n) ? p.rows[i + 1] : -1;
    Quad<KV> q0;
    if (t < quads) q0.load(p, first + 4 * t);
    const bool slot_ok = slot >= 0 && slot < p.num_blocks * kBS;
    if (!slot_ok) return;
    if (upkeep && row >= 0 && row < p.num_rows && pos >= 0 && pos / kBS < p.max_blocks) {
        p.table[static_cast<int64_t>(row) * p.max_blocks + pos / kBS] = slot / kBS;
        if (next_row != row) p.kv_lens[row] = pos + 1;
    }
    const int blk = slot / kBS;
    const int o = slot % kBS;
    for (int e = t; e < quads; e += blockDim.x) {
        Quad<KV> qv = q0;
        if (e != t) qv.load(p, first + 4 * e);
        const int h = e / (kD / 4);
        const int d = 4 * (e % (kD / 4));
        qv.store(p, (static_cast<int64_t>(blk) * p.hkv + h) * kTile, o, h, d);
    }
}

constexpr int kCopyBatch = 32;
struct CopyParams {
    int32_t src[kCopyBatch];
    int32_t dst[kCopyBatch];
    char* k_pool;
    char* v_pool;
    int64_t block_bytes;  // one (layer, block): hkv * 16 * 128 * elt
    int64_t layer_bytes;  // one layer of one pool
};

// blockIdx: x = copy, y = layer, z = 0 (K) / 1 (V).  Copies one block of one
// layer of one pool with 16-byte accesses (block_bytes is a multiple of 512).
__global__ __launch_bounds__(256) void kv_copy_kernel(const CopyParams p) {
    char* base = (blockIdx.z == 0 ? p.k_pool : p.v_pool) + blockIdx.y * p.layer_bytes;
    const u32x4_t* s = reinterpret_cast<const u32x4_t*>(base + p.src[blockIdx.x] * p.block_bytes);
    u32x4_t* d = reinterpret_cast<u32x4_t*>(base + p.dst[blockIdx.x] * p.block_bytes);
    const int64_t n = p.block_bytes / 16;
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) d[e] = s[e];
}

// Swap copies between the device pools and a pinned host buffer.  A swap
// slot holds one block: [layer][K, V][the block's bytes of that layer and
// pool].  blockIdx: x = block of the batch, y = layer, z = 0 (K) / 1 (V).
constexpr int kSwapBatch = 64;
struct SwapParams {
    int32_t ids[kSwapBatch];
    char* k_pool;
    char* v_pool;
    char* host;           // device address of the host buffer's first slot of this batch
    int64_t block_bytes;  // one (layer, block) of one pool
    int64_t layer_bytes;  // one layer of one pool
    int64_t slot_bytes;   // one block in the host buffer: layers * 2 * block_bytes
};

// Copies block_bytes (a multiple of 4 KiB / 16-byte words) from src to dst,
// each thread taking every 256th word with four loads in flight before their
// stores, so that reads across the host link overlap.
__device__ __forceinline__ void copy_chunk(const u32x4_t* __restrict__ s, u32x4_t* __restrict__ d, int64_t words) {
    for (int64_t e = threadIdx.x; e < words; e += 4 * blockDim.x) {
        u32x4_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = e + k * blockDim.x;
            if (i < words) v[k] = s[i];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = e + k * blockDim.x;
            if (i < words) d[i] = v[k];
        }
    }
}

template <bool OUT>
__global__ __launch_bounds__(256) void kv_swap_kernel(const SwapParams p) {
    char* dev = (blockIdx.z == 0 ? p.k_pool : p.v_pool) + blockIdx.y * p.layer_bytes +
                static_cast<int64_t>(p.ids[blockIdx.x]) * p.block_bytes;
    char* host = p.host + blockIdx.x * p.slot_bytes + (2 * blockIdx.y + blockIdx.z) * p.block_bytes;
    const int64_t words = p.block_bytes / 16;
    if constexpr (OUT)
        copy_chunk(reinterpret_cast<const u32x4_t*>(dev), reinterpret_cast<u32x4_t*>(host), words);
    else
        copy_chunk(reinterpret_cast<const u32x4_t*>(host), reinterpret_cast<u32x4_t*>(dev), words);
}

int64_t swap_block_bytes(const pkv_cache* c) {
    const int64_t elt = c->kv_dtype == PKV_F32 ? 4 : c->kv_dtype == PKV_BF16 ? 2 : 1;
    return static_cast<int64_t>(c->num_layers) * 2 * c->num_kv_heads * kTile * elt;
}

template <bool OUT>
int launch_swap(const pkv_cache* c, const int32_t* ids, int32_t n, const void* host, void* stream) {
    int st = check_cache(c);
    if (st) return st;
    if (n < 0 || (n > 0 && (!ids || !host))) return fail(PKV_ERR_INVALID, "swap: bad arguments");
    if (n == 0) return PKV_OK;
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= c->num_blocks) return fail(PKV_ERR_INVALID, "swap: block id %d out of range", ids[i]);
    if (!OUT) {
        std::vector<int32_t> sorted(ids, ids + n);
        std::sort(sorted.begin(), sorted.end());
        if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
            return fail(PKV_ERR_INVALID, "kv_swap_in: a block id is listed twice");
    }
    void* dev_host = nullptr;
    if (hipHostGetDevicePointer(&dev_host, const_cast<void*>(host), 0) != hipSuccess || !dev_host) {
        (void)hipGetLastError();  // clear the error the lookup left
        return fail(PKV_ERR_INVALID, "swap: the host buffer is not pinned host memory");
    }
    const int64_t elt = c->kv_dtype == PKV_F32 ? 4 : c->kv_dtype == PKV_BF16 ? 2 : 1;
    SwapParams p{};
    p.k_pool = static_cast<char*>(c->k_pool);
    p.v_pool = static_cast<char*>(c->v_pool);
    p.block_bytes = static_cast<int64_t>(c->num_kv_heads) * kTile * elt;
    p.layer_bytes = p.block_bytes * c->num_blocks;
    p.slot_bytes = swap_block_bytes(c);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t base = 0; base < n; base += kSwapBatch) {
        const int32_t k = n - base < kSwapBatch ? n - base : kSwapBatch;
        for (int32_t i = 0; i < k; ++i) p.ids[i] = ids[base + i];
        p.host = static_cast<char*>(dev_host) + base * p.slot_bytes;
        hipLaunchKernelGGL(kv_swap_kernel<OUT>, dim3(k, c->num_layers, 2), dim3(256), 0, s, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "swap launch: %s", hipGetErrorString(e));
    return PKV_OK;
}

}  // namespace
}  // namespace pkv

using pkv::fail;

extern "C" {

int kv_cache_write(const pkv_cache* c, int32_t layer, int32_t n_tokens, int32_t val_dtype, const void* k_new,
                   const void* v_new, const int32_t* slots, const int32_t* rows, const int32_t* positions,
                   int32_t num_rows, int32_t* block_table, int32_t max_blocks, int32_t* kv_lens, void* stream) {
    int st = pkv::check_cache(c);
    if (st) return st;
    if (layer < 0 || layer >= c->num_layers) return fail(PKV_ERR_INVALID, "layer %d out of range", layer);
    if (n_tokens < 0) return fail(PKV_ERR_INVALID, "negative token count");
    const int want = c->kv_dtype == PKV_F32 ? PKV_F32 : PKV_BF16;
    if (val_dtype != want) return fail(PKV_ERR_UNSUPPORTED, "values must be %s for this cache", want == PKV_F32 ? "f32" : "bf16");
    if (n_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !slots) return fail(PKV_ERR_INVALID, "null values or slots");
    if (block_table && (!rows || !positions || !kv_lens || num_rows <= 0 || max_blocks <= 0))
        return fail(PKV_ERR_INVALID, "table upkeep needs rows, positions, kv_lens, num_rows and max_blocks");
    const int64_t elt = c->kv_dtype == PKV_F32 ? 4 : c->kv_dtype == PKV_BF16 ? 2 : 1;
    const int64_t layer_elems = static_cast<int64_t>(c->num_blocks) * c->num_kv_heads * pkv::kTile;
    pkv::WriteParams p{};
    p.k_new = k_new;
    p.v_new = v_new;
    p.slots = slots;
    p.rows = rows;
    p.positions = positions;
    p.table = block_table;
    p.kv_lens = kv_lens;
    p.k_pool = static_cast<char*>(c->k_pool) + layer * layer_elems * elt;
    p.v_pool = static_cast<char*>(c->v_pool) + layer * layer_elems * elt;
    p.k_scale = c->k_scale ? c->k_scale + static_cast<int64_t>(layer) * c->num_kv_heads : nullptr;
    p.v_scale = c->v_scale ? c->v_scale + static_cast<int64_t>(layer) * c->num_kv_heads : nullptr;
    p.n = n_tokens;
    p.hkv = c->num_kv_heads;
    p.num_blocks = c->num_blocks;
    p.num_rows = num_rows;
    p.max_blocks = max_blocks;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (c->kv_dtype) {
        case PKV_F32: hipLaunchKernelGGL(pkv::kv_write_kernel<PKV_F32>, dim3(n_tokens), dim3(256), 0, s, p); break;
        case PKV_BF16: hipLaunchKernelGGL(pkv::kv_write_kernel<PKV_BF16>, dim3(n_tokens), dim3(256), 0, s, p); break;
        case PKV_FP8_E4M3:
            hipLaunchKernelGGL(pkv::kv_write_kernel<PKV_FP8_E4M3>, dim3(n_tokens), dim3(256), 0, s, p);
            break;
        default: hipLaunchKernelGGL(pkv::kv_write_kernel<PKV_INT8>, dim3(n_tokens), dim3(256), 0, s, p); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_cache_write launch: %s", hipGetErrorString(e));
    return PKV_OK;
}

int kv_swap_block_bytes(const pkv_cache* c, size_t* out_bytes) {
    if (!out_bytes) return fail(PKV_ERR_INVALID, "null output");
    int st = pkv::check_cache(c);
    if (st) return st;
    *out_bytes = static_cast<size_t>(pkv::swap_block_bytes(c));
    return PKV_OK;
}

int kv_swap_out(const pkv_cache* c, const int32_t* ids, int32_t n, void* host, void* stream) {
    return pkv::launch_swap<true>(c, ids, n, host, stream);
}

int kv_swap_in(const pkv_cache* c, const void* host, const int32_t* ids, int32_t n, void* stream) {
    return pkv::launch_swap<false>(c, ids, n, host, stream);
}

int kv_copy_blocks(const pkv_cache* c, const pkv_copy* copies, int32_t n, void* stream) {
    int st = pkv::check_cache(c);
    if (st) return st;
    if (n < 0 || (n > 0 && !copies)) return fail(PKV_ERR_INVALID, "bad copy list");
    for (int32_t i = 0; i < n; ++i) {
        const pkv_copy& cp = copies[i];
        if (cp.src < 0 || cp.src >= c->num_blocks || cp.dst < 0 || cp.dst >= c->num_blocks || cp.src == cp.dst)
            return fail(PKV_ERR_INVALID, "copy %d: bad blocks %d -> %d", i, cp.src, cp.dst);
    }
    const int64_t elt = c->kv_dtype == PKV_F32 ? 4 : c->kv_dtype == PKV_BF16 ? 2 : 1;
    pkv::CopyParams p{};
    p.k_pool = static_cast<char*>(c->k_pool);
    p.v_pool = static_cast<char*>(c->v_pool);
    p.block_bytes = static_cast<int64_t>(c->num_kv_heads) * pkv::kTile * elt;
    p.layer_bytes = p.block_bytes * c->num_blocks;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t base = 0; base < n; base += pkv::kCopyBatch) {
        const int32_t k = n - base < pkv::kCopyBatch ? n - base : pkv::kCopyBatch;
        for (int32_t i = 0; i < k; ++i) {
            p.src[i] = copies[base + i].src;
            p.dst[i] = copies[base + i].dst;
        }
        hipLaunchKernelGGL(pkv::kv_copy_kernel, dim3(k, c->num_layers, 2), dim3(256), 0, s, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_copy_blocks launch: %s", hipGetErrorString(e));
    return PKV_OK;
}

}  // extern "C"
