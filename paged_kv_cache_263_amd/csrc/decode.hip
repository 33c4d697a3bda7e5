// Paged GQA decode on gfx950.  The decode work of one kv head - every block of
// every row, in row order - is divided into equal contiguous ranges of blocks,
// one per wavefront; a wavefront streams its range's 16-token blocks through
// the block table, and a merge kernel combines the pieces of rows that were
// divided between wavefronts.
//
// What is computed: softmax(q K^T / sqrt(d)) V for one query per row over the
// row's cached tokens, K/V read from scattered blocks through the table ([P3]
// "PagedAttention block management", item (d)), with a running maximum and
// normaliser carried from block to block so the score row never exists whole
// ([P1] "FlashAttention: why the mechanism this whole layer runs on isn't
// compute-bound").  Query head h reads kv head h / G ([P1] "Kernel
// engineering: the layer underneath everything else here": the GQA repeat).
//
// gfx950 mapping.  The G query heads of one kv head are the N side of two
// small matrix products per block, so both run on the matrix cores:
//   S^T[16 tok x 16 heads]  = K[16 tok x 128] . Q^T       (mfma 16x16x32 bf16, 4 steps over d)
//   O^T[128 x 16 heads]    += V^T[128 x 16 tok] . P^T     (mfma 16x16x16 bf16, 8 tiles over d)
// Lane i holds token / d-row (i % 16) and k-slice (i / 16) of the A operand
// and head (i % 16) of the B operand and of the result, so scores, softmax
// state and output of head i % 16 stay in the lanes that own that head: the
// only cross-lane traffic is the max and sum over the four 16-lane groups
// (two xor shuffles, only when the running maximum moves).  Inside a block K
// is token-major and V d-major, with the 16-byte pieces of bf16 and one-byte
// tiles ordered so that each lane's operands are whole 16-byte loads and each
// load instruction of a wave reads contiguous runs of the tile
// (bf16_k_offset, bf16_v_offset, byte_v_offset); fp32 tiles keep the plain
// [tok][d] and [d][tok] orders.  P is split into a bf16 high part and a bf16 remainder,
// so P.V keeps ~16 mantissa bits.  fp32 caches use the fp32 matrix
// instruction (16x16x4) with the same lanes; one-byte caches (fp8 E4M3 and
// int8) convert their codes to bf16 in registers (exact) and fold the
// per-head scales into the score scale (K) and the final normalisation (V).
//
// Work division.  Rows have very different lengths, so fixed-size chunks per
// row leave some wavefronts long tails of work while others sit idle.  Here
// the row lengths become a prefix sum of blocks per row (the plan: taken by
// every wavefront itself for up to 1024 rows, else by a plan kernel); for kv
// head h, wavefront i of Q takes blocks [floor(i U / Q), floor((i+1) U
// / Q)) of the U blocks of all rows in row order, so every wavefront streams
// the same number of blocks (within one).  A row entirely inside one range is
// finished and written by that wavefront; a row cut by range boundaries is
// left as partial results (running max, normaliser, unnormalised output) -
// at most two per wavefront, one for the row at each end of its range - and
// the merge kernel combines them in wavefront order (over the rows, or, with
// more rows than wavefronts per kv head, over the wavefronts' records of the
// divided rows they began).  The partition depends
// on the lengths only, so every sum is taken in an order fixed by logical
// positions and a permutation of the physical blocks changes no bit of the
// output.
//
// Shared prefix.  When every row's table starts with the same blocks, one
// launch (prefix_decode_kernel) runs the shared-prefix pass over those blocks
// (prefix_tile, prefill_tiles.h) in the same grid as the decode wavefronts
// over the rest, and decode_merge_prefix_kernel combines the two.
#include <cmath>
#include <cstdlib>
#include <type_traits>

#include "device.h"
#include "internal.h"
#include "prefill_tiles.h"

namespace pkv {
namespace {

// Floats of one (row, query head) state over a shared prefix: unnormalised
// output [128], running max (log2 units), normaliser, 2 floats of padding
// (16-byte aligned states).
constexpr int kPrefixState = kD + 4;
// what a finished piece of a row is written as: the output (the wavefront had
// the whole row), the row's suffix state (whole row, shared prefix), or a piece
// for the merge kernel
constexpr int kRowOut = 0, kRowState = 1, kPiece = 2;

struct DecodeParams {
    const void* q;                  // [rows][hq][128]
    void* out;                      // [rows][hq][128]
    const void* k_pool;             // this layer: [num_blocks][hkv][16][128]
    const void* v_pool;             // this layer: [num_blocks][hkv][128][16]
    const float* k_scale;           // this layer: [hkv] (one-byte caches only)
    const float* v_scale;
    const int32_t* __restrict__ table;    // [rows][max_blocks]
    const int32_t* __restrict__ kv_lens;  // [rows]
    int32_t* plan;                  // [rows + 1]: blocks of rows 0..b-1 (0 blocks for an invalid row)
    float* ws_acc;                  // [hkv][Q][2][group][128] partial unnormalised outputs
    float* ws_ml;                   // [hkv][Q][2][group][2] partial (max, normaliser)
    // [hkv][Q] per decode wavefront: {row, its first block, one past its
    // last block, 0} of the row whose first block is in the wavefront's range
    // and that another wavefront continues, else row -1 (no prefix)
    int4* ws_cut;
    int32_t merge_owners;           // the merge kernel's grid runs over wavefronts (ws_cut), not rows
    const float* ws_prefix;         // shared prefix: [parts][rows][hq][kPrefixState] (acc[128], max, normaliser)
    int32_t prefix_blocks;          // S: every row's table starts with the same S blocks (0 = none)
    int32_t prefix_parts;           // key ranges the prefix states were computed over
    int32_t byte_kv;                // one-byte cache: V values carry v_scale
    int32_t rows, num_blocks, hkv, hq, group, max_blocks, max_kv_len, parts;  // parts = Q
    float scale_log2;               // log2(e) / sqrt(d)
    // shared prefix: [rows][hq][kPrefixState] the suffix state of every row
    // that one wavefront finished whole (acc[128] times v_scale, max,
    // normaliser)
    float* ws_rows;
};

// A buffer no wave of the kernel writes, read through the constant address
// space, so that wave-uniform reads of it become scalar loads.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* readonly_scalar(const T* ptr) {
    return (const __attribute__((address_space(4))) T*)(ptr);
}

__device__ __forceinline__ bool row_valid(int L, const DecodeParams& p) {
    return L >= 1 && L <= p.max_kv_len && L <= p.max_blocks * kBS && L >= p.prefix_blocks * kBS;
}

// Blocks of a valid row the decode kernel walks: those past the shared prefix.
__device__ __forceinline__ int suffix_blocks(int L, const DecodeParams& p) {
    return (L + kBS - 1) / kBS - p.prefix_blocks;
}

// First block of wavefront i's range for a head with U blocks over Q parts.
// (U < 2^31, checked on the host, so the result fits 32 bits.)
__device__ __forceinline__ int range_start(int64_t U, int i, int Q) { return static_cast<int>(U * i / Q); }

// Parts actually used: at most one per kMinBlocks blocks, so that no range is
// empty (every wavefront that has a range writes its pieces) and tiny batches
// are not cut into one-block pieces.
constexpr int kMinBlocks = 8;
__device__ __forceinline__ int effective_parts(int64_t U, int parts) {
    const int64_t q = U / kMinBlocks;
    return static_cast<int>(q < 1 ? 1 : (q < parts ? q : parts));
}

template <int QT>
__device__ __forceinline__ void store_out4(void* out, int64_t qrow, int d, f32x4_t v) {
    if constexpr (QT == PKV_F32) {
        st<f32x4_t>(static_cast<float*>(out) + qrow * kD + d, v);
    } else {
        const uint32_t a = bf16_bits_rne(v[0]) | (bf16_bits_rne(v[1]) << 16);
        const uint32_t b = bf16_bits_rne(v[2]) | (bf16_bits_rne(v[3]) << 16);
        st<u32x2_t>(static_cast<uint16_t*>(out) + qrow * kD + d, u32x2_t{a, b});
    }
}

// Buffer descriptor of one tile (a raw buffer of `bytes` bytes from the
// tile's start), built in scalar registers from the wave-uniform tile
// address.  Loads through it take the lane's fixed 32-bit byte offset, so a
// block costs no vector address arithmetic: a 64-bit vector address per block
// could be placed in registers that an in-flight tile load still targets,
// and the wave would then wait for that load before issuing the next tile.
constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, no swizzle
constexpr int kLoadStream = 2;          // cache policy: non-temporal (nt)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* tile, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(tile);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), bytes, kRsrcWord3);
}

// Split p into bf16 high and low parts packed as the B operand (4 tokens).
__device__ __forceinline__ void split_p(const float p[4], i16x4_t& hi, i16x4_t& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = __float_as_uint(p[i]);
        h[i] = u & 0xFFFF0000u;
        l[i] = __float_as_uint(p[i] - __uint_as_float(h[i])) & 0xFFFF0000u;
    }
    hi = __builtin_bit_cast(i16x4_t, u32x2_t{(h[0] >> 16) | h[1], (h[2] >> 16) | h[3]});
    lo = __builtin_bit_cast(i16x4_t, u32x2_t{(l[0] >> 16) | l[1], (l[2] >> 16) | l[3]});
}

// Per-KV-dtype register tiles (one block's K and V for one kv head), the
// query operand, and the two contractions.
template <int KV>
struct Tile;

template <>
struct Tile<PKV_BF16> {
    using Elt = uint16_t;
    using Q = bf16x8_t[4];  // Q[head r][32 ks + 8 g .. +7]
    u32x4_t k[4];           // K[tok r][32 ks + 8 g .. +7]
    u32x2_t v[8];           // V^T[16 n + r][4 g .. 4 g + 3]
    static __device__ __forceinline__ void load_q(Q& q, __amdgpu_buffer_rsrc_t qr, int qoff, int g) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            q[ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 64 * ks + 16 * g, 0, 0));
    }
    // Streaming (non-temporal) loads: a decode step reads each tile once, and
    // with this policy on both K and V the kernel reads the Llama-shaped
    // batch about 10% faster (K alone or V alone gain less).  The one-byte
    // tiles below use it too; it pays only where each load instruction of a
    // wave covers whole 64-byte pieces of the tile.
    // The tile orders of bf16_k_offset and bf16_v_offset make each load
    // instruction read 1 KiB of the tile contiguously.
    // Buffer loads through per-tile descriptors (tile_rsrc).
    __device__ __forceinline__ void load(const Elt* kt, const Elt* vt, int r, int g) {
        const int lane_off = 16 * (16 * g + r);
        const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kt, kTile * 2);
        const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vt, kTile * 2);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            k[ks] = __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off + 1024 * ks, 0, kLoadStream);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // d rows 16 (2m) + r and 16 (2m + 1) + r
            const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(vr, lane_off + 1024 * m, 0, kLoadStream);
            v[2 * m] = u32x2_t{w[0], w[1]};
            v[2 * m + 1] = u32x2_t{w[2], w[3]};
        }
    }
    // Zero this lane's V elements of tokens 4g + i with keep[i] false (the
    // unwritten tail of a block may hold any bits, and 0 * NaN is NaN).
    __device__ __forceinline__ void mask_v(const bool keep[4]) {
        const uint32_t lo = (keep[0] ? 0xFFFFu : 0u) | (keep[1] ? 0xFFFF0000u : 0u);
        const uint32_t hi = (keep[2] ? 0xFFFFu : 0u) | (keep[3] ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int n = 0; n < 8; ++n) v[n] = u32x2_t{v[n][0] & lo, v[n][1] & hi};
    }
    __device__ __forceinline__ f32x4_t scores(const Q& q) const {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k[ks]), q[ks], s, 0, 0, 0);
        return s;
    }
    __device__ __forceinline__ void accumulate(f32x4_t acc[8], const float p[4]) const {
        i16x4_t hi, lo;
        split_p(p, hi, lo);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const i16x4_t a = __builtin_bit_cast(i16x4_t, v[n]);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, hi, acc[n], 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, lo, acc[n], 0, 0, 0);
        }
    }
};

// One-byte (fp8, int8) tiles are read with 16-byte loads (narrower loads cap
// the read rate well below the HBM rate), laid out so that every load
// instruction of a wave reads whole 64-byte pieces of the tile.  K: lane
// (r, g) reads codes 64 s + 16 g .. +15 of token row r for s = 0, 1, and
// matrix step ks takes codes 64 (ks / 2) + 16 g + 8 (ks % 2) .. +7; the query
// operand uses the same order of d (a permutation of the contraction index,
// so the scores are unchanged).  V: the tile layout of byte_v_offset puts the
// lane's 8 words (tokens 4g..4g+3 of d rows 16 n + r) in two 16-byte pieces.
template <int KV>
struct ByteTile {
    using Elt = uint8_t;
    using Q = bf16x8_t[4];
    u32x4_t k[2];  // codes 64 s + 16 g .. +15 of token row r
    u32x4_t v[2];  // word n: tokens 4g..4g+3 of d row 16 n + r
    static __device__ __forceinline__ void load_q(Q& q, __amdgpu_buffer_rsrc_t qr, int qoff, int g) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            q[ks] = __builtin_bit_cast(
                bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 128 * (ks >> 1) + 32 * g + 16 * (ks & 1), 0, 0));
    }
    __device__ __forceinline__ void load(const Elt* kt, const Elt* vt, int r, int g) {
#pragma unroll
        for (int s = 0; s < 2; ++s) k[s] = ld_stream<u32x4_t>(kt + r * kD + 64 * s + 16 * g);
#pragma unroll
        for (int s = 0; s < 2; ++s) v[s] = ld_stream<u32x4_t>(vt + g * 512 + s * 256 + r * 16);
    }
    __device__ __forceinline__ void mask_v(const bool keep[4]) {
        const uint32_t m = (keep[0] ? 0xFFu : 0u) | (keep[1] ? 0xFF00u : 0u) | (keep[2] ? 0xFF0000u : 0u) |
                           (keep[3] ? 0xFF000000u : 0u);
#pragma unroll
        for (int s = 0; s < 2; ++s) v[s] &= u32x4_t{m, m, m, m};
    }
    __device__ __forceinline__ f32x4_t scores(const Q& q) const {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x2_t a = byte4_to_bf16x4<KV>(k[ks >> 1][2 * (ks & 1)]);
            const u32x2_t b = byte4_to_bf16x4<KV>(k[ks >> 1][2 * (ks & 1) + 1]);
            const u32x4_t kb = {a[0], a[1], b[0], b[1]};
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb), q[ks], s, 0, 0, 0);
        }
        return s;
    }
    __device__ __forceinline__ void accumulate(f32x4_t acc[8], const float p[4]) const {
        i16x4_t hi, lo;
        split_p(p, hi, lo);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const i16x4_t a = __builtin_bit_cast(i16x4_t, byte4_to_bf16x4<KV>(v[n >> 2][n & 3]));
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, hi, acc[n], 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, lo, acc[n], 0, 0, 0);
        }
    }
};

template <>
struct Tile<PKV_FP8_E4M3> : ByteTile<PKV_FP8_E4M3> {};
template <>
struct Tile<PKV_INT8> : ByteTile<PKV_INT8> {};

template <>
struct Tile<PKV_F32> {
    using Elt = float;
    using Q = f32x4_t[8];  // Q[head r][32 g + 4 c .. +3]; k-step s = 4 c + i uses d = 32 g + s
    f32x4_t k[8];          // K[tok r][32 g + 4 c .. +3]
    f32x4_t v[8];          // V^T[16 n + r][4 g .. 4 g + 3]; k-step i uses token 4 g + i
    static __device__ __forceinline__ void load_q(Q& q, __amdgpu_buffer_rsrc_t qr, int qoff, int g) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            q[c] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 128 * g + 16 * c, 0, 0));
    }
    __device__ __forceinline__ void load(const Elt* kt, const Elt* vt, int r, int g) {
#pragma unroll
        for (int c = 0; c < 8; ++c) k[c] = ld<f32x4_t>(kt + r * kD + 32 * g + 4 * c);
#pragma unroll
        for (int n = 0; n < 8; ++n) v[n] = ld<f32x4_t>(vt + (16 * n + r) * kBS + 4 * g);
    }
    __device__ __forceinline__ void mask_v(const bool keep[4]) {
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[n][i] = keep[i] ? v[n][i] : 0.f;
    }
    __device__ __forceinline__ f32x4_t scores(const Q& q) const {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) s = __builtin_amdgcn_mfma_f32_16x16x4f32(k[c][i], q[c][i], s, 0, 0, 0);
        return s;
    }
    __device__ __forceinline__ void accumulate(f32x4_t acc[8], const float p[4]) const {
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[n][i], p[i], acc[n], 0, 0, 0);
    }
};

// Online-softmax state of the lanes of one head (i % 16): reference max m
// (log2 units), this lane's partial normaliser l, and the output accumulators.
//
// Rescaling is lazy: p = 2^(s - m) is computed against the current reference
// m, and only when some lane sees a score above m + kLazy does the wave take
// the cross-lane max and rescale l and the accumulators to the new reference.
// So every p is at most 2^kLazy (exact in fp32, and split exactly into bf16
// high and low parts as before), the final result acc / l is unchanged, and
// the rescale - 32 accumulator multiplies plus two lane shuffles - runs only
// in the few blocks where the maximum jumps.
constexpr float kLazy = 8.0f;

struct Online {
    float m = -INFINITY;
    float l = 0.f;
    f32x4_t acc[8];
    __device__ __forceinline__ Online() {
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // One block: tok = first token of this lane's four (4 g + i); tokens at
    // or past t1 are masked (score -inf, V zeroed).  blk_end: one past the
    // block's last token (uniform).
    template <int KV>
    __device__ __forceinline__ void step(Tile<KV>& t, const typename Tile<KV>::Q& q, float scale, int tok, int t1,
                                         int blk_end) {
        if (blk_end > t1) {  // partial (or padding) block: uniform branch, no loads inside
            bool keep[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) keep[i] = tok + i < t1;
            t.mask_v(keep);
        }
        const f32x4_t s = t.scores(q);
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (tok + i < t1) ? s[i] * scale : -INFINITY;
        float mb = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        if (__any(mb > m + kLazy)) {  // rare: a new maximum for some head
            mb = fmaxf(mb, __shfl_xor(mb, 16));
            mb = fmaxf(mb, __shfl_xor(mb, 32));
            const float mn = fmaxf(m, mb);
            const float alpha = __builtin_amdgcn_exp2f(m - mn);
            l *= alpha;
#pragma unroll
            for (int n = 0; n < 8; ++n) acc[n] *= alpha;
            m = mn;
        }
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - m);
        l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        t.accumulate(acc, pr);
    }
};

// Writes NaN over the whole output row b (lanes share the elements).
template <int QT>
__device__ __forceinline__ void nan_row(const DecodeParams& p, int b, int lane, int lanes) {
    for (int e = lane; e < p.hq * kD; e += lanes) {
        if constexpr (QT == PKV_F32)
            static_cast<float*>(p.out)[static_cast<int64_t>(b) * p.hq * kD + e] = __builtin_nanf("");
        else
            static_cast<uint16_t*>(p.out)[static_cast<int64_t>(b) * p.hq * kD + e] = 0x7FC0u;
    }
}

// Plan: prefix sum of blocks per row (invalid rows count 0 blocks and get NaN
// output here).  One workgroup of 1024 threads, rows in chunks of 1024.
template <int QT>
__global__ __launch_bounds__(1024) void decode_plan_kernel(const DecodeParams p) {
    __shared__ int32_t wsum[16];
    __shared__ int32_t carry_sh;
    const int t = threadIdx.x;
    if (t == 0) {
        carry_sh = 0;
        p.plan[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < p.rows; base += 1024) {
        const int b = base + t;
        int nb = 0;
        bool invalid = false;
        if (b < p.rows) {
            const int L = p.kv_lens[b];
            invalid = !row_valid(L, p);
            nb = invalid ? 0 : suffix_blocks(L, p);
        }
        // inclusive scan: within the wave, then across the 16 waves
        int v = nb;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(v, off);
            if ((t & 63) >= off) v += u;
        }
        if ((t & 63) == 63) wsum[t >> 6] = v;
        __syncthreads();
        int add = carry_sh;
        for (int w = 0; w < (t >> 6); ++w) add += wsum[w];
        if (b < p.rows) p.plan[b + 1] = v + add;
        __syncthreads();
        if (t == 1023) carry_sh = v + add;
        __syncthreads();
        if (invalid) nan_row<QT>(p, b, 0, 1);  // the whole row becomes NaN
    }
}

// Index of the row holding block position x: plan[b] <= x < plan[b+1]
// (plan in LDS or in global memory).
__device__ __forceinline__ int find_row(const int32_t* plan, int rows, int64_t x) {
    int lo = 0, hi = rows;  // invariant: plan[lo] <= x < plan[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (plan[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// Batches of at most kLocalPlanRows rows skip the plan kernel: every
// wavefront computes the prefix sum of blocks per row itself, into LDS (one
// coalesced load of 64 row lengths and one wave scan per 64 rows), and
// the first wavefront (writer) also stores it for the merge kernel and writes
// the NaN output of invalid rows.  This takes one short kernel and its
// dependent global loads (a binary search through the global plan) off the
// start of every wavefront.
constexpr int kLocalPlanRows = 1024;

template <int QT>
__device__ __forceinline__ void local_plan(const DecodeParams& p, int32_t* plan_sh, int lane, bool writer) {
    // Every row length is requested before the first is used (one memory
    // round trip, not one per 64 rows) and parked in this lane's own plan
    // slots, which the scan below overwrites in the same order.
    constexpr int kPer = kLocalPlanRows / 64;
    int lens[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int b = 64 * k + lane;
        lens[k] = b < p.rows ? p.kv_lens[b] : 0;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int b = 64 * k + lane;
        if (b < p.rows) plan_sh[b + 1] = lens[k];
    }
    int carry = 0;
#pragma unroll 1
    for (int base = 0; base < p.rows; base += 64) {
        const int b = base + lane;
        int nb = 0;
        bool invalid = false;
        if (b < p.rows) {
            const int L = plan_sh[b + 1];
            invalid = !row_valid(L, p);
            nb = invalid ? 0 : suffix_blocks(L, p);
        }
        int v = nb;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(v, off);
            if (lane >= off) v += u;
        }
        if (b < p.rows) {
            plan_sh[b + 1] = carry + v;
            if (writer) p.plan[b + 1] = carry + v;
        }
        carry += __shfl(v, 63);
        if (writer) {
            uint64_t bad = __ballot(b < p.rows && invalid);
            while (bad) {
                const int k = __builtin_ctzll(bad);
                bad &= bad - 1;
                nan_row<QT>(p, base + k, lane, 64);
            }
        }
    }
    if (lane == 0) {
        plan_sh[0] = 0;
        if (writer) p.plan[0] = 0;
    }
    __syncthreads();
}

// QMEM: the query operand is read from memory at every block (the row's
// query rows stay in the caches) instead of from its LDS slot.  Chosen for
// bf16 caches with at most eight query heads per kv head, where it measured
// faster (Llama-shaped batch, 4 heads: 183 against 189 us; the same lengths
// with 8 heads: 192.0 against 196.8 us per call, and the chunked call's 32
// decode rows 95.8 against 97.4 us).  The shared-prefix launch keeps the
// slots above four heads: there the extra reads meet the prefix pass's in the
// same grid (133 against 145 us).  One-byte tiles are smaller still, so those
// keep the slots.
//
// PREFIX: the rows share their first prefix_blocks blocks, whose states the
// shared-prefix pass computes (concurrently, on another stream, or before);
// this kernel walks the blocks past the prefix only, and a row it finishes
// whole goes to ws_rows as a state, not to the output: the merge kernel
// combines it with the prefix states.
template <int KV>
struct DecodeLds {  // LDS of one decode wavefront: its plan (if it builds one) and its two query slots
    using QReg = typename Tile<KV>::Q;
    static constexpr int kQRegs = static_cast<int>(sizeof(QReg) / sizeof(QReg{}[0]));
    static constexpr int kPlanInts = (kLocalPlanRows + 1 + 3) / 4 * 4;  // 16-byte multiple
    static constexpr int kQSlots = 2 * kQRegs * 64;                     // u32x4_t
    static constexpr int kBytes = kPlanInts * 4 + kQSlots * 16;
};
// One wavefront of the decode grid: vblock is its index in the grid (one
// wavefront per workgroup in decode_kernel; four per workgroup, after the
// shared-prefix pass's workgroups, in prefix_decode_kernel), plan_sh and q_sh
// its LDS; with STASH, stash (stash_bytes of LDS) holds its finished pieces
// until its range is done.
template <int KV, bool LOCAL_PLAN, bool QMEM, bool PREFIX, bool STASH>
__device__ __forceinline__ void decode_wave(const DecodeParams& p, int vblock, int lane, int32_t* plan_sh,
                                            u32x4_t* q_sh, float* stash, int stash_bytes) {
    constexpr int QT = (KV == PKV_F32) ? PKV_F32 : PKV_BF16;
    constexpr int kQBytes = (QT == PKV_F32) ? 4 : 2;
    using Elt = typename Tile<KV>::Elt;
    using QReg = typename Tile<KV>::Q;
    constexpr int kQRegs = DecodeLds<KV>::kQRegs;
    const int r = lane & 15;
    const int g = lane >> 4;
    // kv head fastest: consecutive workgroups are dealt round-robin to the 8
    // XCDs, so with 8 kv heads each XCD streams one head (and keeps that
    // head's shared-prefix blocks in its own L2).
    const int kvh = vblock % p.hkv;
    const int wi = vblock / p.hkv;
    if constexpr (LOCAL_PLAN) local_plan<QT>(p, plan_sh, lane, vblock == 0);
    // The plan, the row lengths and the block table are read wave-uniformly:
    // the plan from LDS (or, when the plan kernel wrote it, through the
    // constant address space) and the other two through the constant address
    // space, so these reads are LDS reads or scalar loads.  A vector load
    // there would be counted with the tile loads, and waiting for it would
    // wait for every tile still in flight.
    const auto* cplan = readonly_scalar(p.plan);
    // Flat block indices (plan entries, range bounds, cursors) are 32-bit:
    // every block count fits (checked on the host), and 32-bit compares stay
    // on the scalar unit, so loop control needs no vector temporaries (a
    // temporary placed in a register that an in-flight tile load still
    // targets would make the wave wait for that load).
    auto plan_at = [&](int i) -> int {
        return __builtin_amdgcn_readfirstlane(LOCAL_PLAN ? plan_sh[i] : cplan[i]);
    };
    const auto* ctable = readonly_scalar(p.table);
    const auto* clens = readonly_scalar(p.kv_lens);
    const int U = plan_at(p.rows);
    const int Q = effective_parts(U, p.parts);
    if (wi >= Q || U <= 0) return;
    const int u0 = range_start(U, wi, Q);
    const int u1 = range_start(U, wi + 1, Q);
    if (u0 >= u1) return;
    const bool head_ok = r < p.group;
    const int skip = PREFIX ? p.prefix_blocks : 0;  // blocks of each row before the first one walked here
    const float nan = __builtin_nanf("");
    const f32x4_t nan4 = {nan, nan, nan, nan};

    float scale = p.scale_log2;
    float vs = 1.f;
    if constexpr (is_byte_dtype(KV)) {
        scale *= p.k_scale[kvh];
        vs = p.v_scale[kvh];
    }
    const Elt* kpool = static_cast<const Elt*>(p.k_pool) + static_cast<int64_t>(kvh) * kTile;
    const Elt* vpool = static_cast<const Elt*>(p.v_pool) + static_cast<int64_t>(kvh) * kTile;
    const int64_t blk_stride = static_cast<int64_t>(p.hkv) * kTile;
    // The G query rows of kv head kvh in a row are contiguous; they are read
    // through a per-row buffer descriptor (scalar base) with the lane's fixed
    // offset, so no 64-bit vector address is computed in the loop (one placed
    // in registers that an in-flight tile load targets would make the wave
    // wait for that load).  Lanes past the G heads read past the descriptor's
    // range, which returns zeros.
    const int q_bytes = p.group * kD * kQBytes;
    const int q_lane = head_ok ? r * kD * kQBytes : q_bytes;
    auto q_rsrc = [&](int row) {
        row = __builtin_amdgcn_readfirstlane(row);  // wave-uniform: scalar address arithmetic
        return tile_rsrc(static_cast<const char*>(p.q) +
                             (static_cast<int64_t>(row) * p.hq + kvh * p.group) * kD * kQBytes,
                         q_bytes);
    };

    // The wavefront's blocks u0 .. u1 - 1 (rows in order, each row's blocks
    // in order) stream through a ring of two register tiles: while block x is
    // computed, block x + 1 is in flight, also across the end of a row, so a
    // new row does not start with a wait for its first tile.  Two cursors
    // walk the rows: the load cursor (row bl, blocks lrb0 .. lrb1 - 1) one
    // block ahead of the compute cursor (row bc).  Entering a row, the load
    // cursor also requests that row's query, which the compute cursor takes
    // over when it gets there.  A block id outside the pool is replaced by
    // block 0 and marks its tile bad (the piece's output becomes NaN).
    const int b_first = __builtin_amdgcn_readfirstlane(find_row(LOCAL_PLAN ? plan_sh : p.plan, p.rows, u0));
    int bl = b_first;
    int lrb0 = plan_at(bl), lrb1 = plan_at(bl + 1);
    int l_len = clens[bl];  // kv_len of row bl
    // The query operand of a row lives in one of two LDS slots ([reg][lane],
    // 16 bytes each): the load cursor fills the next row's slot, the compute
    // cursor reads its row's slot at every block.  Kept out of loop-carried
    // registers, a query load is never waited for at the loop's back edge
    // (a register copy there would also wait for the tile in flight).
    auto q_store = [&](int slot, const QReg& v) {
#pragma unroll
        for (int i = 0; i < kQRegs; ++i) q_sh[(slot * kQRegs + i) * 64 + lane] = __builtin_bit_cast(u32x4_t, v[i]);
    };
    auto q_fetch = [&](int slot, QReg& v) {
#pragma unroll
        for (int i = 0; i < kQRegs; ++i)
            v[i] = __builtin_bit_cast(typename std::remove_reference<decltype(v[0])>::type,
                                      q_sh[(slot * kQRegs + i) * 64 + lane]);
    };
    int lslot = 0;  // slot of the load cursor's row
    auto issue = [&](Tile<KV>& t, bool& tbad, int x) {
        bool entered = false;
        QReg qn;
        if (lrb1 <= x) {
            do {
                ++bl;
                lrb0 = lrb1;
                lrb1 = plan_at(bl + 1);
            } while (lrb1 <= x);
            l_len = clens[bl];
            if constexpr (!QMEM) Tile<KV>::load_q(qn, q_rsrc(bl), q_lane, g);  // requested before the tile, so waited for alone
            entered = true;
        }
        const int32_t id = ctable[static_cast<int64_t>(bl) * p.max_blocks + skip + (x - lrb0)];
        const bool ok = id >= 0 && id < p.num_blocks;
        tbad = !ok;
        const int64_t off = static_cast<int64_t>(ok ? id : 0) * blk_stride;
        t.load(kpool + off, vpool + off, r, g);
        if (entered && !QMEM) {
            lslot ^= 1;
            q_store(lslot, qn);
        }
    };

    Tile<KV> t[2];
    bool tbad[2];
    if constexpr (QMEM) {
        issue(t[0], tbad[0], u0);
    } else {
        QReg q0;
        Tile<KV>::load_q(q0, q_rsrc(b_first), q_lane, g);
        issue(t[0], tbad[0], u0);
        q_store(0, q0);
    }
    int cslot = 0;  // slot of the compute cursor's row

    // compute cursor: row bc with blocks crb0 .. crb1 - 1; the piece (this
    // wavefront's part of the row) ends at flat block piece_end; tokens at or
    // past t1 are masked
    int bc = b_first;
    int crb0 = lrb0, crb1 = lrb1;
    int c_len = l_len;
    int piece_end = u0;  // forces the set-up of the first piece
    int t1 = 0;
    bool pbad = false;
    Online o;
    // Results of finished pieces.  A global store counts in the same in-order
    // counter as the tile loads, so every later wait for a tile would also
    // wait for the store to complete; the results are therefore kept in this
    // wavefront's LDS (the stash: per entry its kind and destination, then the
    // values of the G heads' lanes) and written when the range is done, or
    // earlier when the stash is full.
    const int ent_floats = (4 + 130 * p.group + 3) / 4 * 4;
    const int cap = STASH ? stash_bytes / (ent_floats * 4) : 0;
    const int li = g * p.group + r;  // the lane's place in an entry (lanes with head_ok)
    int nst = 0;
    auto write = [&](int kind, int64_t base, const f32x4_t v[8], float2 ml) {
        if (!head_ok) return;
        const int64_t row = base + r;
        if (kind == kRowOut) {
#pragma unroll
            for (int n = 0; n < 8; ++n) store_out4<QT>(p.out, row, 16 * n + 4 * g, v[n]);
        } else {
            float* a = kind == kRowState ? p.ws_rows + row * kPrefixState : p.ws_acc + row * kD;
            float* m = kind == kRowState ? a + kD : p.ws_ml + 2 * row;
#pragma unroll
            for (int n = 0; n < 8; ++n) st<f32x4_t>(a + 16 * n + 4 * g, v[n]);
            if (g == 0) st<float2>(m, ml);
        }
    };
    auto put = [&](int e, int kind, int64_t base, const f32x4_t v[8], float2 ml) {
        float* ent = stash + e * ent_floats;
        if (lane == 0)
            *reinterpret_cast<int4*>(ent) =
                int4{kind, static_cast<int>(base & 0xFFFFFFFF), static_cast<int>(base >> 32), 0};
        if (head_ok) {
#pragma unroll
            for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4_t*>(ent + 4 + 32 * li + 4 * n) = v[n];
            if (g == 0) *reinterpret_cast<float2*>(ent + 4 + 128 * p.group + 2 * r) = ml;
        }
    };
    auto flush = [&] {
        for (int e = 0; e < nst; ++e) {
            const float* ent = stash + e * ent_floats;
            const int4 meta = *reinterpret_cast<const int4*>(ent);
            const int kind = __builtin_amdgcn_readfirstlane(meta.x);
            const int64_t base = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(meta.z)) << 32) |
                                 static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(meta.y));
            f32x4_t v[8];
            float2 ml = {0.f, 0.f};
            if (head_ok) {
#pragma unroll
                for (int n = 0; n < 8; ++n) v[n] = *reinterpret_cast<const f32x4_t*>(ent + 4 + 32 * li + 4 * n);
                if (g == 0) ml = *reinterpret_cast<const float2*>(ent + 4 + 128 * p.group + 2 * r);
            }
            write(kind, base, v, ml);
        }
    };
    // One block x: computed from `cur` while block x + 1 (the range's last
    // block again at its end: a cache hit, never used) loads into `nxt`.  A
    // new row takes over the load cursor's query slot before that load, which
    // may fill the other slot with the query of the row after.
    auto step = [&](Tile<KV>& cur, bool tb, Tile<KV>& nxt, bool& nb, int x) {
        const bool first = x == piece_end;  // first block of a piece
        if (first && x > u0) {
            // a later row: the load cursor, which loaded block x, is still in
            // it, with its bounds, length and query slot
            bc = bl;
            crb0 = lrb0;
            crb1 = lrb1;
            c_len = l_len;
            cslot = lslot;
        }
        QReg qm;
        if constexpr (QMEM) Tile<KV>::load_q(qm, q_rsrc(bc), q_lane, g);
        issue(nxt, nb, x + 1 < u1 ? x + 1 : u1 - 1);
        if (first) {
            piece_end = crb1 < u1 ? crb1 : u1;
            t1 = min(c_len, (skip + static_cast<int>(piece_end - crb0)) * kBS);
            pbad = false;
            o = Online();
        }
        pbad = pbad || tb;
        const int tok0 = (skip + static_cast<int>(x - crb0)) * kBS;
        QReg q;
        if constexpr (QMEM) {
#pragma unroll
            for (int i = 0; i < kQRegs; ++i) q[i] = qm[i];
        } else {
            q_fetch(cslot, q);
        }
        o.step<KV>(cur, q, scale, tok0 + 4 * g, t1, tok0 + kBS);
        if (x + 1 == piece_end) {  // last block of the piece: its result
            float l = o.l;
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            const bool whole = crb0 >= u0 && crb1 <= u1;  // no other wavefront touches this row
            if constexpr (STASH) {
                const int kind = whole ? (PREFIX ? kRowState : kRowOut) : kPiece;
                const int64_t base = whole ? static_cast<int64_t>(bc) * p.hq + kvh * p.group
                                           : ((static_cast<int64_t>(kvh) * p.parts + wi) * 2 +
                                              (bc == b_first ? 0 : 1)) * p.group;
                f32x4_t v[8];
                const float f = kind == kRowOut ? (pbad ? nan : vs / l) : vs;
#pragma unroll
                for (int n = 0; n < 8; ++n) v[n] = (pbad && kind != kRowOut) ? nan4 : o.acc[n] * f;
                const float2 ml = {o.m, pbad ? nan : l};
                if (cap > 0) {
                    if (nst == cap) {
                        flush();
                        nst = 0;
                    }
                    put(nst++, kind, base, v, ml);
                } else {
                    write(kind, base, v, ml);
                }
            } else if (head_ok) {  // written at once
                const int64_t qrow = static_cast<int64_t>(bc) * p.hq + kvh * p.group + r;
                if (whole && PREFIX) {
                    float* sp = p.ws_rows + qrow * kPrefixState;
#pragma unroll
                    for (int n = 0; n < 8; ++n) st<f32x4_t>(sp + 16 * n + 4 * g, pbad ? nan4 : o.acc[n] * vs);
                    if (g == 0) st<float2>(sp + kD, float2{o.m, pbad ? nan : l});
                } else if (whole) {
                    const float inv = pbad ? nan : vs / l;
#pragma unroll
                    for (int n = 0; n < 8; ++n) store_out4<QT>(p.out, qrow, 16 * n + 4 * g, o.acc[n] * inv);
                } else {
                    const int side = (bc == b_first) ? 0 : 1;
                    const int64_t w = ((static_cast<int64_t>(kvh) * p.parts + wi) * 2 + side) * p.group + r;
#pragma unroll
                    for (int n = 0; n < 8; ++n)
                        st<f32x4_t>(p.ws_acc + w * kD + 16 * n + 4 * g, pbad ? nan4 : o.acc[n] * vs);
                    if (g == 0) st<float2>(p.ws_ml + 2 * w, float2{o.m, pbad ? nan : l});
                }
            }
        }
    };

    // two blocks per trip, so the ring slots are fixed registers
    for (int x = u0; x < u1; x += 2) {
        step(t[0], tbad[0], t[1], tbad[1], x);
        if (x + 1 >= u1) break;
        step(t[1], tbad[1], t[0], tbad[0], x + 1);
    }
    if constexpr (STASH) flush();
    if constexpr (!PREFIX) {
        // the row this wavefront began and another one continues (at most
        // one: the last row of the range), for the merge kernel
        if (lane == 0)
            p.ws_cut[static_cast<int64_t>(kvh) * p.parts + wi] =
                (crb0 >= u0 && crb1 > u1) ? make_int4(bc, crb0, crb1, 0) : make_int4(-1, 0, 0, 0);
    }
}

// Stash bytes of a decode_kernel wavefront: with the plan and query slots,
// the LDS of the four bf16 workgroups a compute unit holds at the default
// partition stays well within its 160 KB.  One-byte caches (eight workgroups
// per CU, long rows with one or two pieces per wavefront) write directly:
// their stash measured slower (fp8 long context 658 against 653 us).
template <int KV, bool QMEM>
constexpr int kStashBytes = KV == PKV_BF16 ? (QMEM ? 24576 : 16384) : 0;

template <int KV, bool LOCAL_PLAN, bool QMEM>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeParams p) {
    __shared__ int32_t plan_sh[LOCAL_PLAN ? kLocalPlanRows + 1 : 1];
    __shared__ u32x4_t q_sh[DecodeLds<KV>::kQSlots];
    __shared__ f32x4_t stash[kStashBytes<KV, QMEM> > 0 ? kStashBytes<KV, QMEM> / 16 : 1];
    decode_wave<KV, LOCAL_PLAN, QMEM, false, (kStashBytes<KV, QMEM> > 0)>(p, blockIdx.x, threadIdx.x, plan_sh, q_sh,
                                             kStashBytes<KV, QMEM> > 0 ? reinterpret_cast<float*>(stash) : nullptr,
                                             kStashBytes<KV, QMEM>);
}

// A decode call with a shared prefix, in one launch: workgroups 0 ..
// n_prefix - 1 run the shared-prefix pass (prefix_tile, 4 waves each), the
// rest run the decode wavefronts over the suffixes, four per workgroup.  The
// pass's workgroups are dispatched first and the two kinds share the compute
// units (two workgroups per CU: one of each while the pass lasts), so the pass
// (matrix cores, on cached prefix tiles) runs under the decode's HBM
// streaming.  Both carve one LDS allocation.
constexpr int kFusedThreads = 256;
static_assert(kFusedThreads == pf::kPrefixThreads, "one workgroup size for both roles");
constexpr int kFusedLds = pf::kPrefixLdsBytes;
template <int KV, bool LOCAL_PLAN, bool QMEM>
__global__ __launch_bounds__(kFusedThreads, 2) void prefix_decode_kernel(const DecodeParams p, const pf::PrefillParams pp,
                                                                         int n_prefix) {
    constexpr int kWaveLds = kFusedLds / 4 / 16 * 16;  // each decode wavefront's share: plan, query slots, stash
    static_assert(DecodeLds<KV>::kBytes < kWaveLds, "four decode wavefronts fit the pass's LDS");
    __shared__ __attribute__((aligned(16))) unsigned char lds[kFusedLds];
    if (static_cast<int>(blockIdx.x) < n_prefix) {
        pf::prefix_tile<KV>(pp, blockIdx.x, lds);
        return;
    }
    // The decode wavefronts issue at the highest wave priority: on a compute
    // unit they share with a pass workgroup, their loads are then issued
    // ahead of the pass's arithmetic (prefix pass + decode on the 256-row
    // batch: 119.8 against 123.2 us event-timed; priority 1: 120.2 us).
    __builtin_amdgcn_s_setprio(3);
    // The wavefront index, taken as wave-uniform: derived from threadIdx.x
    // alone it counts as divergent, and every value computed from it (kv
    // head, range, rows, block-table reads) would move to vector registers,
    // the table reads becoming vector loads that wait for the tile in flight.
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    unsigned char* mine = lds + w * kWaveLds;
    decode_wave<KV, LOCAL_PLAN, QMEM, true, KV == PKV_BF16>(p, (blockIdx.x - n_prefix) * 4 + w, threadIdx.x & 63,
                                            reinterpret_cast<int32_t*>(mine),
                                            reinterpret_cast<u32x4_t*>(mine + DecodeLds<KV>::kPlanInts * 4),
                                            reinterpret_cast<float*>(mine + DecodeLds<KV>::kBytes),
                                            kWaveLds - DecodeLds<KV>::kBytes);
}

// Merge the pieces of one (row, query head) that was divided between
// wavefronts: out = sum_i acc_i 2^(m_i - M) / sum_i l_i 2^(m_i - M),
// M = max_i m_i, in wavefront order.  The pieces are read kMergeBatch at a
// time (indices past the last piece repeat it and are left out of the sums);
// past the first batch the sums are rescaled whenever the maximum moves.
constexpr int kMaxParts = 4096;
constexpr int kMergeBatch = 8;
// One wavefront per (row, kv head, group of kMergeHeads query heads); lane l
// owns d = 2 l, 2 l + 1 of those heads.  The row's plan and wavefront range
// are worked out once; then every load of a batch is issued together, so a
// row cut into at most kMergeBatch pieces costs one round of loads after the
// plan's.  One head per wavefront measured fastest (Llama-shaped batch 4.7
// against 7.2 us with four heads, whose 64 wave-uniform piece addresses per
// batch spilled scalar registers; fp8 long context 7.5 against 16.6 us); the
// shared-prefix merge, with few pieces per row, is fastest at four
// (kPrefixMergeHeads: 10.2 against 15.5 us at one).
// With more rows than wavefronts per kv head, most rows are whole, and a
// wavefront per row and head costs more than the merging itself: the merge
// then runs one wavefront per (decode wavefront, kv head, head group), which
// merges the row that decode wavefront began and another continued, if any
// (recorded by the decode kernel; a row divided between wavefronts has
// exactly one such owner).  Measured per decode call (decode + merge), eight
// query heads per kv head: 1024 rows of 132 tokens 139.6 -> 116.3 us, 512 of
// 264 108.6 -> 96.1, 256 of 528 95.1 -> 90.1.  Wavefronts per workgroup do
// not matter: four or more per workgroup changed nothing, the count of
// wavefronts does.
constexpr int kMergeHeads = 1;
constexpr int kPrefixMergeHeads = 4;

template <int QT>
__device__ __forceinline__ void store_out2(void* out, int64_t qrow, int d, float a, float b) {
    if constexpr (QT == PKV_F32) {
        st<float2>(static_cast<float*>(out) + qrow * kD + d, float2{a, b});
    } else {
        st<uint32_t>(static_cast<uint16_t*>(out) + qrow * kD + d, bf16_bits_rne(a) | (bf16_bits_rne(b) << 16));
    }
}

// Range bounds for the merge kernels: floor(U i / Q), equal to range_start,
// in 32-bit arithmetic (the 64-bit division's inlined code made up most of a
// merge kernel's instructions).  With U = a Q + b (0 <= b < Q), U i / Q =
// a i + b i / Q, where a i <= U < 2^31 and b i < Q^2 <= 2^24 (Q <= 4096, the
// decode's partition limit, checked on the host).
struct RangeBounds {
    int a, b, Q;
    __device__ RangeBounds(int64_t U, int Q_) : a(static_cast<int>(U) / Q_), b(static_cast<int>(U) % Q_), Q(Q_) {}
    __device__ int start(int i) const { return a * i + (b * i) / Q; }
};

// The wavefronts whose ranges meet a row's blocks [rb0, rb1) of U: the row's
// pieces come from wavefronts i0 .. i0 + n - 1.  Only the first can have
// started its range in an earlier row (then this row is its second piece,
// side0 = 1); every later one starts inside this row, so the row is its first
// piece.  The first guesses (in floating point) are moved to the exact
// wavefronts by the loops.
__device__ __forceinline__ void row_pieces(const DecodeParams& p, int64_t U, int64_t rb0, int64_t rb1, int& i0, int& n,
                                           int& side0) {
    const int Q = effective_parts(U, p.parts);
    const RangeBounds rs(U, Q);
    const float qu = static_cast<float>(Q) / static_cast<float>(U);
    const int r0 = static_cast<int>(rb0), r1 = static_cast<int>(rb1) - 1;
    i0 = min(max(static_cast<int>(static_cast<float>(r0) * qu), 0), Q - 1);
    while (i0 + 1 < Q && rs.start(i0 + 1) <= r0) ++i0;
    while (i0 > 0 && rs.start(i0) > r0) --i0;
    int i1 = min(max(static_cast<int>(static_cast<float>(r1) * qu), 0), Q - 1);
    while (i1 + 1 < Q && rs.start(i1 + 1) <= r1) ++i1;
    while (i1 > 0 && rs.start(i1) > r1) --i1;
    n = i1 - i0 + 1;
    side0 = rs.start(i0) < r0 ? 1 : 0;
}

template <int QT>
__global__ __launch_bounds__(64) void decode_merge_kernel(const DecodeParams p) {
    // kv head fastest, as in the decode kernel, so a head's partial results
    // are read on the XCD that wrote them
    const int hgroups = (p.group + kMergeHeads - 1) / kMergeHeads;
    const int kvh = static_cast<int>(blockIdx.x % p.hkv);
    const int rest = static_cast<int>(blockIdx.x / p.hkv);
    const int h0 = (rest % hgroups) * kMergeHeads;
    const int d = 2 * threadIdx.x;
    const int grp = p.group;
    const int nh = min(kMergeHeads, grp - h0);  // heads of this wavefront
    int b;
    int64_t U, rb0, rb1;
    if (p.merge_owners) {
        // rest / hgroups is a decode wavefront: the row it began that another
        // continues, if any (the records of wavefronts past the effective
        // count are left from earlier calls)
        const int i = rest / hgroups;
        const int4 cut = p.ws_cut[static_cast<int64_t>(kvh) * p.parts + i];
        U = p.plan[p.rows];
        if (U <= 0 || i >= effective_parts(U, p.parts) || cut.x < 0) return;
        b = cut.x;
        rb0 = cut.y;
        rb1 = cut.z;
    } else {
        b = rest / hgroups;
        U = p.plan[p.rows];
        rb0 = p.plan[b];
        rb1 = p.plan[b + 1];
        if (rb1 <= rb0 || U <= 0) return;  // an invalid row (NaN from the plan)
    }
    const int64_t row_q = static_cast<int64_t>(b) * p.hq + kvh * grp;  // query row of head 0 of the group
    int i0, n, side0;
    row_pieces(p, U, rb0, rb1, i0, n, side0);
    if (n == 1) return;  // written directly by the one wavefront
    const float* __restrict__ ws_ml = p.ws_ml;
    const float* __restrict__ ws_acc = p.ws_acc;
    const int64_t base0 = (static_cast<int64_t>(kvh) * p.parts + i0) * 2 * grp;
    // slot of (head hh, piece k), the piece clamped to the last one
#define PKV_MERGE_SLOT(hh, k) (base0 + (hh) + (2 * min((k), n - 1) + ((k) == 0 ? side0 : 0)) * grp)
    float mx[kMergeHeads];
    float2 num[kMergeHeads];
    float den[kMergeHeads];
#pragma unroll
    for (int a = 0; a < kMergeHeads; ++a) {
        mx[a] = -INFINITY;
        num[a] = float2{0.f, 0.f};
        den[a] = 0.f;
    }
    float2 ml[kMergeHeads][kMergeBatch];
    float2 acc[kMergeHeads][kMergeBatch];
    for (int k0 = 0; k0 < n; k0 += kMergeBatch) {
#pragma unroll
        for (int a = 0; a < kMergeHeads; ++a) {
            const int hh = h0 + min(a, nh - 1);
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
                const int64_t sl = PKV_MERGE_SLOT(hh, k0 + j);
                ml[a][j] = ld<float2>(ws_ml + 2 * sl);
                acc[a][j] = ld<float2>(ws_acc + sl * kD + d);
            }
        }
        // every load of the batch is in flight before the first is used
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < kMergeHeads; ++a) {
            float bm = mx[a];
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) bm = fmaxf(bm, ml[a][j].x);  // repeats are real pieces
            if (bm > mx[a]) {  // the maximum moved: rescale what is summed (nothing in the first batch)
                const float r = mx[a] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx[a] - bm);
                num[a].x *= r;
                num[a].y *= r;
                den[a] *= r;
                mx[a] = bm;
            }
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
                if (k0 + j < n) {
                    const float w = __builtin_amdgcn_exp2f(ml[a][j].x - mx[a]);
                    num[a].x += acc[a][j].x * w;
                    num[a].y += acc[a][j].y * w;
                    den[a] += ml[a][j].y * w;
                }
            }
        }
    }
#pragma unroll
    for (int a = 0; a < kMergeHeads; ++a)
        if (a < nh) store_out2<QT>(p.out, row_q + h0 + a, d, num[a].x / den[a], num[a].y / den[a]);
#undef PKV_MERGE_SLOT
}

// Shared prefix: the output of (row, query head) combines the states of the
// prefix's key ranges (from the shared-prefix pass) with the row's suffix
// pieces - its state in ws_rows when one wavefront finished the row, else the
// divided pieces in the slots - by the max/normaliser algebra of the online
// softmax, in that order.  The prefix states carry no v_scale, the suffix
// states do.  A row with no block past the prefix is its prefix states alone.
// One wavefront per (row, kv head, group of kPrefixMergeHeads query heads),
// kv head fastest, lanes as in decode_merge_kernel.
template <int QT>
__global__ __launch_bounds__(64) void decode_merge_prefix_kernel(const DecodeParams p) {
    const int hgroups = (p.group + kPrefixMergeHeads - 1) / kPrefixMergeHeads;
    const int kvh = static_cast<int>(blockIdx.x % p.hkv);
    const int rest = static_cast<int>(blockIdx.x / p.hkv);
    const int h0 = (rest % hgroups) * kPrefixMergeHeads;
    const int b = rest / hgroups;
    const int d = 2 * threadIdx.x;
    const int grp = p.group;
    const int nh = min(kPrefixMergeHeads, grp - h0);
    if (!row_valid(p.kv_lens[b], p)) return;  // NaN from the plan
    const int64_t row_q = static_cast<int64_t>(b) * p.hq + kvh * grp;
    const int64_t U = p.plan[p.rows];
    const int64_t rb0 = p.plan[b];
    const int64_t rb1 = p.plan[b + 1];
    int i0 = 0, n = 0, side0 = 0;
    if (rb1 > rb0) row_pieces(p, U, rb0, rb1, i0, n, side0);
    const int64_t base0 = (static_cast<int64_t>(kvh) * p.parts + i0) * 2 * grp;
    const int64_t pstride = static_cast<int64_t>(p.rows) * p.hq * kPrefixState;
    const float vs = p.byte_kv ? p.v_scale[kvh] : 1.f;
    const int parts = p.prefix_parts;
    // slot of suffix piece k (n > 1) of head hh: wavefront i0 + k, side side0 for the first
    auto slot = [&](int hh, int k) { return base0 + hh + (2 * k + (k == 0 ? side0 : 0)) * grp; };
    if (parts <= 2 && n <= 2) {
        // the usual case: every state of the wavefront's heads requested at
        // once (indices past the last repeat it and are left out)
        float2 ml[kPrefixMergeHeads][4], ac[kPrefixMergeHeads][4];  // prefix ranges 0, 1, suffix pieces 0, 1
#pragma unroll
        for (int a = 0; a < kPrefixMergeHeads; ++a) {
            const int hh = h0 + min(a, nh - 1);
            const float* ps = p.ws_prefix + (row_q + hh) * kPrefixState;
            const float* rs = p.ws_rows + (row_q + hh) * kPrefixState;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float* sk = ps + min(k, parts - 1) * pstride;
                ml[a][k] = ld<float2>(sk + kD);
                ac[a][k] = ld<float2>(sk + d);
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (n <= 1) {  // the whole-row state (read and left out when n == 0)
                    ml[a][2 + k] = ld<float2>(rs + kD);
                    ac[a][2 + k] = ld<float2>(rs + d);
                } else {
                    const int64_t sl = slot(hh, k);
                    ml[a][2 + k] = ld<float2>(p.ws_ml + 2 * sl);
                    ac[a][2 + k] = ld<float2>(p.ws_acc + sl * kD + d);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < kPrefixMergeHeads; ++a) {
            if (a < nh) {
                auto used = [&](int k) { return k < 2 ? k < parts : k - 2 < n; };
                float mx = -INFINITY;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (used(k)) mx = fmaxf(mx, ml[a][k].x);
                float2 num = {0.f, 0.f};
                float den = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if (used(k)) {
                        const float w = __builtin_amdgcn_exp2f(ml[a][k].x - mx);
                        const float wa = k < 2 ? w * vs : w;
                        num.x += ac[a][k].x * wa;
                        num.y += ac[a][k].y * wa;
                        den += ml[a][k].y * w;
                    }
                }
                store_out2<QT>(p.out, row_q + h0 + a, d, num.x / den, num.y / den);
            }
        }
        return;
    }
    for (int hh = h0; hh < h0 + nh; ++hh) {
        const float* ps = p.ws_prefix + (row_q + hh) * kPrefixState;
        const float* rs = p.ws_rows + (row_q + hh) * kPrefixState;
        auto slot = [&](int k) { return base0 + hh + (2 * k + (k == 0 ? side0 : 0)) * grp; };
        auto piece_ml = [&](int k) { return n == 1 ? ld<float2>(rs + kD) : ld<float2>(p.ws_ml + 2 * slot(k)); };
        auto piece_acc = [&](int k) { return n == 1 ? ld<float2>(rs + d) : ld<float2>(p.ws_acc + slot(k) * kD + d); };
        float mx = -INFINITY;
        for (int k = 0; k < parts; ++k) mx = fmaxf(mx, ps[k * pstride + kD]);
        for (int k = 0; k < n; ++k) mx = fmaxf(mx, piece_ml(k).x);
        float2 num = {0.f, 0.f};
        float den = 0.f;
        for (int k = 0; k < parts; ++k) {
            const float w = __builtin_amdgcn_exp2f(ps[k * pstride + kD] - mx);
            const float2 a = ld<float2>(ps + k * pstride + d);
            num.x += a.x * (w * vs);
            num.y += a.y * (w * vs);
            den += ps[k * pstride + kD + 1] * w;
        }
        for (int k = 0; k < n; ++k) {
            const float2 ml = piece_ml(k);
            const float w = __builtin_amdgcn_exp2f(ml.x - mx);
            const float2 a = piece_acc(k);
            num.x += a.x * w;
            num.y += a.y * w;
            den += ml.y * w;
        }
        store_out2<QT>(p.out, row_q + hh, d, num.x / den, num.y / den);
    }
}

// Wavefronts per kv head, as a count per CU over all CUs: four (one per
// SIMD) for bf16 caches, eight for the others.  These are the measured best
// under streaming tile loads: bf16 decode of the Llama-shaped batch takes
// 190 us at four per CU, 194-196 at eight and 198-199 at five (an uneven
// share of the SIMDs); one-byte caches need eight wavefronts in flight (669 us
// against 779 at four on the long-context fp8 batch).  The registers allow
// two wavefronts per SIMD for every cache type but fp32, which fits one.
// PKV_DECODE_WAVES_PER_CU overrides the default for tuning runs.
int decode_parts_auto(int hkv, int kv_dtype) {
    static const int env = [] {
        const char* e = std::getenv("PKV_DECODE_WAVES_PER_CU");
        const int v = e ? std::atoi(e) : 0;
        return v < 0 ? 0 : (v > 32 ? 32 : v);
    }();
    const int per_cu = env > 0 ? env : (kv_dtype == PKV_BF16 ? 4 : 8);
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    const int parts = (cus * per_cu + hkv - 1) / hkv;
    return parts < 1 ? 1 : (parts > kMaxParts ? kMaxParts : parts);
}

template <bool LOCAL>
void launch_decode_kernel(int kv_dtype, dim3 grid, hipStream_t stream, const DecodeParams& p) {
    switch (kv_dtype) {
        case PKV_F32:
            hipLaunchKernelGGL((decode_kernel<PKV_F32, LOCAL, false>), grid, dim3(64), 0, stream, p);
            break;
        case PKV_BF16:
            if (p.group <= 8)
                hipLaunchKernelGGL((decode_kernel<PKV_BF16, LOCAL, true>), grid, dim3(64), 0, stream, p);
            else
                hipLaunchKernelGGL((decode_kernel<PKV_BF16, LOCAL, false>), grid, dim3(64), 0, stream, p);
            break;
        case PKV_FP8_E4M3:
            hipLaunchKernelGGL((decode_kernel<PKV_FP8_E4M3, LOCAL, false>), grid, dim3(64), 0, stream, p);
            break;
        default:
            hipLaunchKernelGGL((decode_kernel<PKV_INT8, LOCAL, false>), grid, dim3(64), 0, stream, p);
            break;
    }
}

// (no shared prefix with an fp32 cache: refused by the argument checks)
template <bool LOCAL>
void launch_prefix_decode_kernel(int kv_dtype, dim3 grid, hipStream_t stream, const DecodeParams& p,
                                 const pf::PrefillParams& pp, int n_prefix) {
    const dim3 block(kFusedThreads);
    switch (kv_dtype) {
        case PKV_BF16:
            if (p.group <= 4)
                hipLaunchKernelGGL((prefix_decode_kernel<PKV_BF16, LOCAL, true>), grid, block, 0, stream, p, pp,
                                   n_prefix);
            else
                hipLaunchKernelGGL((prefix_decode_kernel<PKV_BF16, LOCAL, false>), grid, block, 0, stream, p, pp,
                                   n_prefix);
            break;
        case PKV_FP8_E4M3:
            hipLaunchKernelGGL((prefix_decode_kernel<PKV_FP8_E4M3, LOCAL, false>), grid, block, 0, stream, p, pp,
                               n_prefix);
            break;
        default:
            hipLaunchKernelGGL((prefix_decode_kernel<PKV_INT8, LOCAL, false>), grid, block, 0, stream, p, pp,
                               n_prefix);
            break;
    }
}

}  // namespace

int32_t decode_parts(const pkv_cache* c, const pkv_attn_args* a) {
    if (a->decode_parts > 0) return a->decode_parts < kMaxParts ? a->decode_parts : kMaxParts;
    return decode_parts_auto(c->num_kv_heads, c->kv_dtype);
}

size_t decode_workspace_bytes(const pkv_cache* c, const pkv_attn_args* a, int32_t rows) {
    if (rows <= 0) return 0;
    const int64_t Q = decode_parts(c, a);
    const int64_t group = a->num_q_heads / c->num_kv_heads;
    const int64_t plan = (static_cast<int64_t>(rows) + 1 + 3) / 4 * 4;  // int32, 16-byte multiple
    const int64_t slots = static_cast<int64_t>(c->num_kv_heads) * Q * 2 * group;
    const int64_t cuts = static_cast<int64_t>(c->num_kv_heads) * Q;  // int4 each
    // shared prefix: the states of its key ranges, then the rows' suffix states
    const int64_t prefix = a->shared_prefix_blocks > 0 ? (static_cast<int64_t>(prefix_parts(c, a, rows)) + 1) * rows *
                                                             a->num_q_heads * kPrefixState
                                                       : 0;
    return static_cast<size_t>(plan * 4 + slots * (kD + 2) * 4 + cuts * 16 + prefix * 4);
}

// Launch decode over `rows` rows whose q/out/table/kv_lens start at the given
// pointers (used by paged_attn_decode and by the decode rows of a prefill call).
int launch_decode(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, int32_t max_kv_len, const void* q,
                  void* out, const int32_t* table, const int32_t* kv_lens, void* workspace, size_t ws_bytes,
                  hipStream_t stream) {
    auto mark = [&](int i) {
        if (a->events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(a->events[i]), stream);
    };
    if (rows <= 0) {
        for (int i = 0; i < 3; ++i) mark(i);
        return PKV_OK;
    }
    const size_t need = decode_workspace_bytes(c, a, rows);
    if (!workspace || ws_bytes < need)
        return fail(PKV_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need, workspace ? ws_bytes : 0);
    const int32_t Q = decode_parts(c, a);
    const int64_t grid = static_cast<int64_t>(Q) * c->num_kv_heads;

    const int64_t elt = c->kv_dtype == PKV_F32 ? 4 : c->kv_dtype == PKV_BF16 ? 2 : 1;
    const int64_t layer_elems = static_cast<int64_t>(c->num_blocks) * c->num_kv_heads * kTile;
    DecodeParams p{};
    p.q = q;
    p.out = out;
    p.k_pool = static_cast<const char*>(c->k_pool) + a->layer * layer_elems * elt;
    p.v_pool = static_cast<const char*>(c->v_pool) + a->layer * layer_elems * elt;
    p.k_scale = c->k_scale ? c->k_scale + static_cast<int64_t>(a->layer) * c->num_kv_heads : nullptr;
    p.v_scale = c->v_scale ? c->v_scale + static_cast<int64_t>(a->layer) * c->num_kv_heads : nullptr;
    p.table = table;
    p.kv_lens = kv_lens;
    const int64_t plan_ints = (static_cast<int64_t>(rows) + 1 + 3) / 4 * 4;
    const int64_t slots = static_cast<int64_t>(c->num_kv_heads) * Q * 2 * (a->num_q_heads / c->num_kv_heads);
    p.plan = static_cast<int32_t*>(workspace);
    p.ws_acc = reinterpret_cast<float*>(static_cast<int32_t*>(workspace) + plan_ints);
    p.ws_ml = p.ws_acc + slots * kD;
    p.ws_cut = reinterpret_cast<int4*>(p.ws_ml + slots * 2);  // 16-byte aligned: slots is even
    p.prefix_blocks = a->shared_prefix_blocks;
    p.prefix_parts = a->shared_prefix_blocks > 0 ? prefix_parts(c, a, rows) : 0;
    p.ws_prefix = a->shared_prefix_blocks > 0
                      ? reinterpret_cast<float*>(p.ws_cut + static_cast<int64_t>(c->num_kv_heads) * Q)
                      : nullptr;
    p.ws_rows = a->shared_prefix_blocks > 0
                    ? const_cast<float*>(p.ws_prefix) + static_cast<int64_t>(p.prefix_parts) * rows * a->num_q_heads *
                                                            kPrefixState
                    : nullptr;
    p.byte_kv = is_byte_dtype(c->kv_dtype) ? 1 : 0;
    p.rows = rows;
    p.num_blocks = c->num_blocks;
    p.hkv = c->num_kv_heads;
    p.hq = a->num_q_heads;
    p.group = a->num_q_heads / c->num_kv_heads;
    p.max_blocks = a->max_blocks;
    p.max_kv_len = max_kv_len;
    p.parts = Q;
    p.scale_log2 = kLog2e / sqrtf(static_cast<float>(kD));

    const bool f32 = a->q_dtype == PKV_F32;
    const bool local = rows <= kLocalPlanRows;
    if (!local) {
        if (f32)
            hipLaunchKernelGGL(decode_plan_kernel<PKV_F32>, dim3(1), dim3(1024), 0, stream, p);
        else
            hipLaunchKernelGGL(decode_plan_kernel<PKV_BF16>, dim3(1), dim3(1024), 0, stream, p);
    }
    mark(0);
    const bool prefix = p.prefix_blocks > 0;
    if (prefix) {
        pf::PrefillParams pp;
        const int n_prefix = prefix_pass_params(c, a, rows, q, table, const_cast<float*>(p.ws_prefix), &pp);
        const dim3 g(static_cast<unsigned>(n_prefix + (grid + 3) / 4));
        if (local)
            launch_prefix_decode_kernel<true>(c->kv_dtype, g, stream, p, pp, n_prefix);
        else
            launch_prefix_decode_kernel<false>(c->kv_dtype, g, stream, p, pp, n_prefix);
    } else {
        const dim3 g1(static_cast<unsigned>(grid));
        if (local)
            launch_decode_kernel<true>(c->kv_dtype, g1, stream, p);
        else
            launch_decode_kernel<false>(c->kv_dtype, g1, stream, p);
    }
    mark(1);
    const int heads = prefix ? kPrefixMergeHeads : kMergeHeads;
    const int64_t hgroups = (a->num_q_heads / c->num_kv_heads + heads - 1) / heads;
    // Without a prefix only rows divided between wavefronts need merging, and
    // each has one owner (the wavefront holding its first block); with more
    // rows than wavefronts per kv head the grid runs over the wavefronts'
    // owner records instead of the rows.
    p.merge_owners = !prefix && rows > Q ? 1 : 0;
    const int64_t units = p.merge_owners ? Q : rows;
    const dim3 mgrid(static_cast<unsigned>(units * c->num_kv_heads * hgroups));
    if (prefix)  // (bf16 queries: a shared prefix needs a bf16 or one-byte cache)
        hipLaunchKernelGGL(decode_merge_prefix_kernel<PKV_BF16>, mgrid, dim3(64), 0, stream, p);
    else if (f32)
        hipLaunchKernelGGL(decode_merge_kernel<PKV_F32>, mgrid, dim3(64), 0, stream, p);
    else
        hipLaunchKernelGGL(decode_merge_kernel<PKV_BF16>, mgrid, dim3(64), 0, stream, p);
    mark(2);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return PKV_OK;
}

}  // namespace pkv

extern "C" {

int paged_attn_workspace_size(const pkv_cache* c, const pkv_attn_args* a, size_t* bytes) {
    if (!bytes) return pkv::fail(PKV_ERR_INVALID, "null output");
    *bytes = 0;
    int st = pkv::check_attn(c, a);
    if (st) return st;
    if (a->num_seqs == 0) return PKV_OK;
    // A prefill call uses the decode path for its decode rows; its chunk rows
    // need the states of their key ranges when the tiles are split (after the
    // decode part, 256-byte aligned).
    const int32_t rows = a->cu_q ? a->num_decode : a->num_seqs;
    *bytes = pkv::decode_workspace_bytes(c, a, rows);
    if (a->cu_q) {
        const size_t pre = pkv::prefill_workspace_bytes(c, a);
        if (pre > 0) *bytes = (*bytes + 255) / 256 * 256 + pre;
    }
    return PKV_OK;
}

int paged_attn_decode(const pkv_cache* c, const pkv_attn_args* a, void* stream) {
    int st = pkv::check_attn(c, a);
    if (st) return st;
    return pkv::launch_decode(c, a, a->num_seqs, a->max_kv_len, a->q, a->out, a->block_table, a->kv_lens,
                              a->workspace, a->workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
