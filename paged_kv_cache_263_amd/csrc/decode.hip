// Paged GQA decode on gfx950: one wavefront per (row, kv head, key chunk)
// streams the chunk's 16-token blocks through the block table, and a second
// kernel merges the chunks of rows that were split.
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
// (two xor shuffles).  With K stored [tok][d] and V stored [d][tok] inside a
// block, every lane's operand is one contiguous 16 / 8 / 4-byte load and a
// wave reads each 4 KiB (bf16) tile in whole cache lines.  P is split into a
// bf16 high part and a bf16 remainder, so P.V keeps ~16 mantissa bits.
// fp32 caches use the fp32 matrix instruction (16x16x4) with the same lanes;
// fp8 caches convert E4M3 bytes to bf16 in registers (exact) and fold the
// per-head scales into the score scale (K) and the final normalisation (V).
//
// The order of every sum depends on logical token positions only (fixed
// chunk boundaries, fixed merge order), so a permutation of the physical
// blocks changes no bit of the output.
#include <cmath>
#include <cstdlib>

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

struct DecodeParams {
    const void* q;            // [rows][hq][128]
    void* out;                // [rows][hq][128]
    const void* k_pool;       // this layer: [num_blocks][hkv][16][128]
    const void* v_pool;       // this layer: [num_blocks][hkv][128][16]
    const float* k_scale;     // this layer: [hkv] (fp8 only)
    const float* v_scale;
    const int32_t* table;     // [rows][max_blocks]
    const int32_t* kv_lens;   // [rows]
    float* ws_acc;            // [rows][hq][max_splits][128]
    float* ws_ml;             // [rows][hq][max_splits][2]
    int32_t num_blocks, hkv, hq, group, max_blocks, max_kv_len, split_tokens, max_splits;
    float scale_log2;         // log2(e) / sqrt(d)
};

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
    static __device__ __forceinline__ void load_q(Q& q, const void* qp, bool ok, int g) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4_t x = ok ? ld<u32x4_t>(static_cast<const uint16_t*>(qp) + 32 * ks + 8 * g) : u32x4_t{0, 0, 0, 0};
            q[ks] = __builtin_bit_cast(bf16x8_t, x);
        }
    }
    __device__ __forceinline__ void load(const Elt* kt, const Elt* vt, int r, int g) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) k[ks] = ld<u32x4_t>(kt + r * kD + 32 * ks + 8 * g);
#pragma unroll
        for (int n = 0; n < 8; ++n) v[n] = ld<u32x2_t>(vt + (16 * n + r) * kBS + 4 * g);
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

template <>
struct Tile<PKV_FP8_E4M3> {
    using Elt = uint8_t;
    using Q = bf16x8_t[4];
    u32x2_t k[4];   // 8 codes: K[tok r][32 ks + 8 g .. +7]
    uint32_t v[8];  // 4 codes: V^T[16 n + r][4 g .. 4 g + 3]
    static __device__ __forceinline__ void load_q(Q& q, const void* qp, bool ok, int g) {
        Tile<PKV_BF16>::load_q(q, qp, ok, g);
    }
    __device__ __forceinline__ void load(const Elt* kt, const Elt* vt, int r, int g) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) k[ks] = ld<u32x2_t>(kt + r * kD + 32 * ks + 8 * g);
#pragma unroll
        for (int n = 0; n < 8; ++n) v[n] = ld<uint32_t>(vt + (16 * n + r) * kBS + 4 * g);
    }
    __device__ __forceinline__ void mask_v(const bool keep[4]) {
        const uint32_t m = (keep[0] ? 0xFFu : 0u) | (keep[1] ? 0xFF00u : 0u) | (keep[2] ? 0xFF0000u : 0u) |
                           (keep[3] ? 0xFF000000u : 0u);
#pragma unroll
        for (int n = 0; n < 8; ++n) v[n] &= m;
    }
    __device__ __forceinline__ f32x4_t scores(const Q& q) const {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x2_t a = fp8x4_to_bf16x4(k[ks][0]);
            const u32x2_t b = fp8x4_to_bf16x4(k[ks][1]);
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
            const i16x4_t a = __builtin_bit_cast(i16x4_t, fp8x4_to_bf16x4(v[n]));
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, hi, acc[n], 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, lo, acc[n], 0, 0, 0);
        }
    }
};

template <>
struct Tile<PKV_F32> {
    using Elt = float;
    using Q = f32x4_t[8];  // Q[head r][32 g + 4 c .. +3]; k-step s = 4 c + i uses d = 32 g + s
    f32x4_t k[8];          // K[tok r][32 g + 4 c .. +3]
    f32x4_t v[8];          // V^T[16 n + r][4 g .. 4 g + 3]; k-step i uses token 4 g + i
    static __device__ __forceinline__ void load_q(Q& q, const void* qp, bool ok, int g) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            q[c] = ok ? ld<f32x4_t>(static_cast<const float*>(qp) + 32 * g + 4 * c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
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

template <int KV, int NBUF>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeParams p) {
    constexpr int QT = (KV == PKV_F32) ? PKV_F32 : PKV_BF16;
    constexpr int kQBytes = (QT == PKV_F32) ? 4 : 2;
    using Elt = typename Tile<KV>::Elt;
    const int lane = threadIdx.x;
    const int r = lane & 15;
    const int g = lane >> 4;
    // blockIdx -> (row, split, kv head); kv head fastest so that consecutive
    // workgroups (dealt round-robin to the 8 XCDs) keep one kv head per XCD.
    const int per_row = p.max_splits * p.hkv;
    const int row = blockIdx.x / per_row;
    const int rem = blockIdx.x - row * per_row;
    const int split = rem / p.hkv;
    const int kvh = rem - split * p.hkv;

    const int L = p.kv_lens[row];
    const bool row_ok = L >= 1 && L <= p.max_kv_len && L <= p.max_blocks * kBS;
    const int nsplit = row_ok ? (L + p.split_tokens - 1) / p.split_tokens : 1;
    if (split >= nsplit) return;
    const bool head_ok = r < p.group;
    const int64_t qrow = static_cast<int64_t>(row) * p.hq + kvh * p.group + (head_ok ? r : 0);
    const float nan = __builtin_nanf("");
    const f32x4_t nan4 = {nan, nan, nan, nan};

    const int t0 = split * p.split_tokens;
    const int t1 = min(L, t0 + p.split_tokens);
    const int nblk = row_ok ? (t1 - t0 + kBS - 1) / kBS : 0;
    const int32_t* trow = p.table + static_cast<int64_t>(row) * p.max_blocks + t0 / kBS;
    const int tb = lane < nblk ? trow[lane] : 0;
    const bool bad = !row_ok || __any(lane < nblk && (tb < 0 || tb >= p.num_blocks));
    if (bad) {  // invalid row or block id: the row's output becomes NaN
        if (!head_ok) return;
        if (nsplit == 1) {
#pragma unroll
            for (int n = 0; n < 8; ++n) store_out4<QT>(p.out, qrow, 16 * n + 4 * g, nan4);
        } else {
            const int64_t w = qrow * p.max_splits + split;
#pragma unroll
            for (int n = 0; n < 8; ++n) st<f32x4_t>(p.ws_acc + w * kD + 16 * n + 4 * g, nan4);
            if (g == 0) st<float2>(p.ws_ml + 2 * w, float2{0.f, nan});
        }
        return;
    }

    float scale = p.scale_log2;
    if constexpr (KV == PKV_FP8_E4M3) scale *= p.k_scale[kvh];

    const Elt* kpool = static_cast<const Elt*>(p.k_pool) + static_cast<int64_t>(kvh) * kTile;
    const Elt* vpool = static_cast<const Elt*>(p.v_pool) + static_cast<int64_t>(kvh) * kTile;
    const int64_t blk_stride = static_cast<int64_t>(p.hkv) * kTile;

    typename Tile<KV>::Q q;
    Tile<KV>::load_q(q, static_cast<const char*>(p.q) + qrow * kD * kQBytes, head_ok, g);

    Online o;
    // Ring of NBUF register tiles: while block j is computed, blocks
    // j+1 .. j+NBUF-1 are in flight.  The trip count is padded to a multiple
    // of NBUF and every load is unconditional (block index clamped to the
    // last block, a cache hit), so no branch sits between a load and its use
    // and the compiler's wait counts let the prefetched loads stay in flight.
    // Padding steps are fully masked and change nothing.
    const int niter = (nblk + NBUF - 1) / NBUF * NBUF;
    auto tile_off = [&](int j) -> int64_t {
        return static_cast<int64_t>(__builtin_amdgcn_readlane(tb, min(j, nblk - 1))) * blk_stride;
    };
    Tile<KV> t[NBUF];
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) {
        const int64_t b = tile_off(u);
        t[u].load(kpool + b, vpool + b, r, g);
    }
    for (int j0 = 0; j0 < niter; j0 += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
            const int j = j0 + u;
            const int64_t b = tile_off(j + NBUF - 1);
            t[(u + NBUF - 1) % NBUF].load(kpool + b, vpool + b, r, g);
            o.step<KV>(t[u], q, scale, t0 + j * kBS + 4 * g, t1, t0 + (j + 1) * kBS);
        }
    }

    float l = o.l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    float vs = 1.f;
    if constexpr (KV == PKV_FP8_E4M3) vs = p.v_scale[kvh];
    if (!head_ok) return;
    if (nsplit == 1) {
        const float inv = vs / l;
#pragma unroll
        for (int n = 0; n < 8; ++n) store_out4<QT>(p.out, qrow, 16 * n + 4 * g, o.acc[n] * inv);
    } else {
        const int64_t w = qrow * p.max_splits + split;
#pragma unroll
        for (int n = 0; n < 8; ++n) st<f32x4_t>(p.ws_acc + w * kD + 16 * n + 4 * g, o.acc[n] * vs);
        if (g == 0) st<float2>(p.ws_ml + 2 * w, float2{o.m, l});
    }
}

// Merge the chunks of one (row, query head): out = sum_i acc_i 2^(m_i - M) /
// sum_i l_i 2^(m_i - M), M = max_i m_i.  The weights are computed once into
// LDS; each lane (one per d) then sums the chunks in chunk order.
constexpr int kMaxSplits = 4096;
template <int QT>
__global__ __launch_bounds__(128) void decode_merge_kernel(const DecodeParams p) {
    __shared__ float wsh[kMaxSplits];
    __shared__ float red[2];
    const int64_t qrow = blockIdx.x;
    const int row = static_cast<int>(qrow / p.hq);
    const int d = threadIdx.x;
    const int L = p.kv_lens[row];
    const bool row_ok = L >= 1 && L <= p.max_kv_len && L <= p.max_blocks * kBS;
    const int nsplit = row_ok ? (L + p.split_tokens - 1) / p.split_tokens : 1;
    if (nsplit <= 1) return;
    const float* ml = p.ws_ml + 2 * qrow * p.max_splits;
    float mx = -INFINITY;
    for (int i = d; i < nsplit; i += 128) mx = fmaxf(mx, ml[2 * i]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((d & 63) == 0) red[d >> 6] = mx;
    __syncthreads();
    mx = fmaxf(red[0], red[1]);
    for (int i = d; i < nsplit; i += 128) wsh[i] = __builtin_amdgcn_exp2f(ml[2 * i] - mx);
    __syncthreads();
    // denominator in chunk order (every lane computes the same sum)
    float den = 0.f;
    for (int i = 0; i < nsplit; ++i) den += ml[2 * i + 1] * wsh[i];
    const float* acc = p.ws_acc + qrow * p.max_splits * kD + d;
    float num = 0.f;
    int i = 0;
    for (; i + 4 <= nsplit; i += 4) {
        const float a0 = acc[static_cast<int64_t>(i) * kD], a1 = acc[static_cast<int64_t>(i + 1) * kD];
        const float a2 = acc[static_cast<int64_t>(i + 2) * kD], a3 = acc[static_cast<int64_t>(i + 3) * kD];
        num += a0 * wsh[i];
        num += a1 * wsh[i + 1];
        num += a2 * wsh[i + 2];
        num += a3 * wsh[i + 3];
    }
    for (; i < nsplit; ++i) num += acc[static_cast<int64_t>(i) * kD] * wsh[i];
    const float o = num / den;
    if constexpr (QT == PKV_F32) {
        static_cast<float*>(p.out)[qrow * kD + d] = o;
    } else {
        static_cast<uint16_t*>(p.out)[qrow * kD + d] = static_cast<uint16_t>(bf16_bits_rne(o));
    }
}

// Blocks in flight per wavefront (2..4).  PKV_DECODE_DEPTH overrides the
// default for tuning runs.
int decode_pipeline_depth() {
    static const int depth = [] {
        const char* e = std::getenv("PKV_DECODE_DEPTH");
        const int v = e ? std::atoi(e) : 3;
        return v < 2 ? 2 : (v > 4 ? 4 : v);
    }();
    return depth;
}

}  // namespace

// Launch decode over `rows` rows whose q/out/table/kv_lens start at the given
// pointers (used by paged_attn_decode and by the decode rows of a prefill call).
int launch_decode(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, int32_t max_kv_len, const void* q,
                  void* out, const int32_t* table, const int32_t* kv_lens, void* workspace, size_t ws_bytes,
                  hipStream_t stream) {
    if (rows <= 0) {
        for (int i = 0; i < 3; ++i)
            if (a->events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(a->events[i]), stream);
        return PKV_OK;
    }
    const int32_t st_tokens = decode_split_tokens(c, a, rows, max_kv_len);
    const int32_t splits = (max_kv_len + st_tokens - 1) / st_tokens;
    const size_t need = decode_workspace_bytes(c, a, rows, max_kv_len);
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(PKV_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need, workspace ? ws_bytes : 0);
    if (splits > kMaxSplits) return fail(PKV_ERR_INVALID, "more than %d key chunks per row", kMaxSplits);
    const int64_t grid = static_cast<int64_t>(rows) * splits * c->num_kv_heads;
    if (grid > INT32_MAX) return fail(PKV_ERR_INVALID, "decode launch too large");

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
    const int64_t accs = static_cast<int64_t>(rows) * a->num_q_heads * splits * kD;
    p.ws_acc = need ? static_cast<float*>(workspace) : nullptr;
    p.ws_ml = need ? static_cast<float*>(workspace) + accs : nullptr;
    p.num_blocks = c->num_blocks;
    p.hkv = c->num_kv_heads;
    p.hq = a->num_q_heads;
    p.group = a->num_q_heads / c->num_kv_heads;
    p.max_blocks = a->max_blocks;
    p.max_kv_len = max_kv_len;
    p.split_tokens = st_tokens;
    p.max_splits = splits;
    p.scale_log2 = kLog2e / sqrtf(static_cast<float>(kD));

    auto mark = [&](int i) {
        if (a->events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(a->events[i]), stream);
    };
    mark(0);
    const dim3 g1(static_cast<unsigned>(grid));
    const int depth = decode_pipeline_depth();
    switch (c->kv_dtype) {
        case PKV_F32:
            hipLaunchKernelGGL((decode_split_kernel<PKV_F32, 2>), g1, dim3(64), 0, stream, p);
            break;
        case PKV_BF16:
            if (depth <= 2) hipLaunchKernelGGL((decode_split_kernel<PKV_BF16, 2>), g1, dim3(64), 0, stream, p);
            else if (depth == 3) hipLaunchKernelGGL((decode_split_kernel<PKV_BF16, 3>), g1, dim3(64), 0, stream, p);
            else hipLaunchKernelGGL((decode_split_kernel<PKV_BF16, 4>), g1, dim3(64), 0, stream, p);
            break;
        default:
            if (depth <= 2) hipLaunchKernelGGL((decode_split_kernel<PKV_FP8_E4M3, 2>), g1, dim3(64), 0, stream, p);
            else if (depth == 3) hipLaunchKernelGGL((decode_split_kernel<PKV_FP8_E4M3, 3>), g1, dim3(64), 0, stream, p);
            else hipLaunchKernelGGL((decode_split_kernel<PKV_FP8_E4M3, 4>), g1, dim3(64), 0, stream, p);
            break;
    }
    mark(1);
    if (splits > 1) {
        const int64_t mgrid = static_cast<int64_t>(rows) * a->num_q_heads;
        if (a->q_dtype == PKV_F32)
            hipLaunchKernelGGL(decode_merge_kernel<PKV_F32>, dim3(static_cast<unsigned>(mgrid)), dim3(128), 0, stream, p);
        else
            hipLaunchKernelGGL(decode_merge_kernel<PKV_BF16>, dim3(static_cast<unsigned>(mgrid)), dim3(128), 0, stream, p);
    }
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
    // need no workspace.
    const int32_t rows = a->cu_q ? a->num_decode : a->num_seqs;
    const int32_t len = (a->cu_q && a->max_decode_kv_len > 0) ? a->max_decode_kv_len : a->max_kv_len;
    *bytes = pkv::decode_workspace_bytes(c, a, rows, len);
    return PKV_OK;
}

int paged_attn_decode(const pkv_cache* c, const pkv_attn_args* a, void* stream) {
    int st = pkv::check_attn(c, a);
    if (st) return st;
    return pkv::launch_decode(c, a, a->num_seqs, a->max_kv_len, a->q, a->out, a->block_table, a->kv_lens,
                              a->workspace, a->workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
