// Device code of the prefill kernels that the decode path also runs: the
// staging of K/V tiles into LDS (layouts, registers), the helpers of the
// 32x32x16 score and P.V products, and the shared-prefix pass over one tile of
// decode rows (prefix_tile), which a decode launch runs in the same grid as
// its wavefronts.  The chunk kernel, the merge of key ranges and the host
// side are in prefill.hip.
#pragma once

#include <cmath>

#include "device.h"
#include "internal.h"

namespace pkv {
namespace pf {

constexpr int kKeys = 64;              // keys per iteration (4 blocks)
constexpr int kKStride = kD + 8;       // padded K row (elements)
constexpr int kKStage = kKeys * kKStride;  // elements of one K stage
constexpr int kVStage = 4 * kTile;         // elements of one V stage (4 tiles [128][16])
constexpr float kLazy = 8.0f;              // rescale threshold (log2 units)
constexpr int kPrefixThreads = 256;        // shared-prefix pass: 4 waves
constexpr int kPrefixRows = 128;           // query rows per shared-prefix workgroup

typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct PrefillParams {
    const void* q;          // [total_q][hq][128] bf16
    void* out;
    const void* k_pool;     // this layer
    const void* v_pool;
    const float* k_scale;   // this layer [hkv]
    const float* v_scale;
    const int32_t* table;   // [num_seqs][max_blocks]
    const int32_t* kv_lens; // [num_seqs]
    const int32_t* cu_q;    // [num_seqs + 1]
    int32_t row0, num_blocks, hkv, hq, group, max_blocks, max_kv_len, max_q_len, q_tiles, total_q, tile_tokens;
    float scale_log2;
    // key ranges per tile; with parts > 1 (and always in the shared-prefix
    // pass) the state of (range, query, head) goes to
    // states[part][query][hq][kState] instead of the output, query = the
    // global query index (the decode row in the shared-prefix pass)
    float* states;
    int32_t parts;
    // shared-prefix pass (prefix_tile): the decode rows' queries over the
    // first prefix_tokens keys of table row 0
    int32_t prefix_tokens;
};

// Floats of one (query, head) state: unnormalised output [128], running max
// (log2 units), normaliser, padding (the decode kernel reads the same layout
// for the shared-prefix states).
constexpr int kState = kD + 4;

// LDS element offset of tokens 8 h .. 8 h + 7 of d row d inside a staged V
// tile: rows of 16 tokens, the two halves swapped in rows with bit 3 of d
// set, so that the 16 lanes of one operand read (d rows r .. r + 15, same h)
// cover all 64 banks.
__device__ __forceinline__ int v_lds_offset(int d, int h) { return d * kBS + 8 * (h ^ ((d >> 3) & 1)); }

// bf16 V piece staged by thread u of the V group: a permutation of the pieces
// inside each wave's contiguous 1 KiB of the tile (so the global load stays
// one contiguous run per wave), chosen so that every 16 lanes of the two
// 8-byte LDS stores below write distinct banks.  Lane 16 a + b takes d row
// r = 4 a + b % 4 (and r + 16) of the wave's 32 rows, token group
// g = 2 h + (b / 4) % 2 with h = (b / 8) ^ (a / 2).
struct VPiece {
    int r, g;
};
__device__ __forceinline__ VPiece v_piece(int u) {
    const int a = (u >> 4) & 3, b = u & 15;
    const int r = 4 * a + (b & 3);
    const int h = ((b >> 3) & 1) ^ (a >> 1);
    return VPiece{r, 2 * h + ((b >> 2) & 1)};
}

// Staging registers of one iteration's tiles: 16 bytes of each of the 4
// tiles per thread.  The K group (threads u = 0..255 of group 0) holds K
// tiles, the V group V tiles, in the same registers.
//
// K (k_load, k_store): bf16 tiles (bf16_k_offset): piece u, token u % 16, d
// 8 (u / 16) .. +7, so the group reads each 4 KiB tile contiguously.
// One-byte tiles: row u / 16, codes (u % 16) * 8 .. +7, held as codes in the
// registers and converted to bf16 by the LDS store (so the conversion does not
// wait for the load in the phase that issues it).  Tile addresses are uniform
// (one per block) and the thread's offset inside a tile is fixed.
template <int KV>
struct Stage {
    u32x4_t k[4];
    __device__ __forceinline__ void k_load(const char* const kb[4], uint32_t koff) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (KV == PKV_BF16) {
                k[b] = ld<u32x4_t>(kb[b] + koff);
            } else {
                const u32x2_t kk = ld<u32x2_t>(kb[b] + koff);
                k[b] = u32x4_t{kk[0], kk[1], 0u, 0u};
            }
        }
    }
    // 8 codes (two words) as 8 bf16 values
    static __device__ __forceinline__ u32x4_t widen(uint32_t w0, uint32_t w1) {
        const u32x2_t a = byte4_to_bf16x4<KV>(w0), b = byte4_to_bf16x4<KV>(w1);
        return u32x4_t{a[0], a[1], b[0], b[1]};
    }
    __device__ __forceinline__ void k_store(uint16_t* ks, int u) const {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (KV == PKV_BF16)
                st<u32x4_t>(ks + (b * kBS + (u & 15)) * kKStride + 8 * (u >> 4), k[b]);
            else
                st<u32x4_t>(ks + (b * kBS + (u >> 4)) * kKStride + (u & 15) * 8, widen(k[b][0], k[b][1]));
        }
    }

    // V (v_load, v_store): bf16 (bf16_v_offset): piece 64 (u / 64) + 16 g + r
    // (v_piece), tokens 4g..4g+3 of d rows 32 (u / 64) + r and that + 16.
    // One-byte tiles: d row u / 2, tokens (u % 2) * 8 .. +7, as two 4-byte
    // words at voff and voff1 (byte_v_offset).
    __device__ __forceinline__ void v_load(const char* const vb[4], uint32_t voff, uint32_t voff1) {
        u32x4_t* v = k;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (KV == PKV_BF16)
                v[b] = ld<u32x4_t>(vb[b] + voff);
            else
                v[b] = u32x4_t{ld<uint32_t>(vb[b] + voff), ld<uint32_t>(vb[b] + voff1), 0u, 0u};
        }
    }
    // Zero V of tokens at or past valid[b] (the row's partial last block and
    // blocks past its end, which hold whatever the clamped load read; 0 * NaN
    // is NaN).  Only the iteration that reaches the row's end calls this.
    __device__ __forceinline__ void mask_tail(const int valid[4], int u) {
        u32x4_t* v = k;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t w[4] = {v[b][0], v[b][1], v[b][2], v[b][3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (KV == PKV_BF16) {  // bf16 element e: token 4 g + e % 4
                    if (4 * v_piece(u).g + (e & 3) >= valid[b]) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                } else {  // code byte e: token (u % 2) * 8 + e (a zero code is 0.0)
                    if ((u & 1) * 8 + e >= valid[b]) w[e >> 2] &= ~(0xFFu << (8 * (e & 3)));
                }
            }
            v[b] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
    }
    __device__ __forceinline__ void v_store(uint16_t* vs, int u) const {
        const u32x4_t* v = k;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (KV == PKV_BF16) {
                const VPiece vp = v_piece(u);
                const int g = vp.g;
                const int d0 = 32 * (u >> 6) + vp.r;
                uint16_t* vt = vs + b * kTile + 4 * (g & 1);
                st<u32x2_t>(vt + v_lds_offset(d0, g >> 1), u32x2_t{v[b][0], v[b][1]});
                st<u32x2_t>(vt + v_lds_offset(d0 + 16, g >> 1), u32x2_t{v[b][2], v[b][3]});
            } else {
                st<u32x4_t>(vs + b * kTile + v_lds_offset(u >> 1, u & 1), widen(v[b][0], v[b][1]));
            }
        }
    }
};

// Score product operand row for lane row m (0..31) of a 32-key tile: bits 2
// and 3 of the key index swapped.  Result register i of lane group g (lanes
// 32 g .. 32 g + 31) then holds key 16 (i / 8) + 8 g + i % 8 of the tile.
__device__ __forceinline__ int key_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Two probabilities as a bf16 pair, rounded to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}


// The shared-prefix pass of a decode call: every decode row's query (one per
// row, total_q rows) over the first prefix_tokens keys of table row 0, no
// causal mask, the keys split into p.parts ranges of whole iterations; the
// state of (range, row, head) goes to states[part][row][hq][kState].
//
// A pass over a 2000-token prefix gives each tile only tens of iterations, so
// it uses smaller workgroups than the chunk rows: 4 waves (128 query rows,
// 128 / G rows of the batch with all G heads), two per compute unit, one
// barrier per iteration, every thread staging 16 bytes of each K and V tile
// (one register stage, two LDS buffers) - the pipeline fill of the 8-wave
// ping-pong costs more than it gains over so few iterations.  The products
// and the softmax are the ones of the chunk kernel.
//
// One workgroup of the pass (kPrefixThreads threads; block = its index in the
// pass), on kPrefixLdsBytes of LDS at lds: the kernel that runs it also runs
// the decode wavefronts of the same call (prefix_decode_kernel).
constexpr int kPrefixLdsBytes = (2 * kKStage + 2 * kVStage) * 2 + kPrefixRows * 4;
template <int KV>
__device__ __forceinline__ void prefix_tile(const PrefillParams& p, int block, unsigned char* lds) {
    auto ks = reinterpret_cast<uint16_t(*)[kKStage]>(lds);
    auto vs = reinterpret_cast<uint16_t(*)[kVStage]>(lds + 2 * kKStage * 2);
    int* broken = reinterpret_cast<int*>(lds + (2 * kKStage + 2 * kVStage) * 2);
    constexpr int kElt = (KV == PKV_BF16) ? 2 : 1;

    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int lane = t & 63;
    const int c32 = lane & 31;
    const int g = lane >> 5;
    // block -> (q tile, key range, kv head), kv head fastest
    const int kvh = block % p.hkv;
    const int part = (block / p.hkv) % p.parts;
    const int qt = block / (p.hkv * p.parts);
    const int C = p.total_q;
    const int j0 = qt * p.tile_tokens;
    if (j0 >= C) return;
    const int L = p.prefix_tokens;
    const bool row_ok = L >= kBS;

    // The caller promises that every row's table starts with row 0's first
    // prefix_tokens / 16 block ids.  Each workgroup checks the promise for its
    // own rows; a row that breaks it gets a NaN state, so its output is NaN
    // like that of any other invalid row.
    for (int i = t; i < p.tile_tokens; i += kPrefixThreads) broken[i] = 0;
    __syncthreads();
    {
        const int S = L / kBS;
        const int ntok = min(p.tile_tokens, C - j0);
        for (int e = t; e < ntok * S; e += kPrefixThreads) {
            const int r = e / S, b = e - r * S;
            if (p.table[static_cast<int64_t>(j0 + r) * p.max_blocks + b] != p.table[b]) broken[r] = 1;
        }
        // (read after the barrier that follows the first stage store)
    }
    const int n_iter = row_ok ? (L + kKeys - 1) / kKeys : 0;
    const int nblk_seq = (L + kBS - 1) / kBS;
    const int64_t blk_bytes = static_cast<int64_t>(p.hkv) * kTile * kElt;
    const int32_t* trow = p.table;  // the prefix is row 0's

    const int n = 32 * wave + c32;
    const int tok = n / p.group;
    const int hh = n - tok * p.group;
    const bool qrow_ok = tok < p.tile_tokens && j0 + tok < C;
    const int j = min(j0 + tok, C - 1);
    const int last_key = L - 1;  // every row sees the whole prefix

    float scale = p.scale_log2;
    if constexpr (is_byte_dtype(KV)) scale *= p.k_scale[kvh];

    bf16x8_t qop[8];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                             (static_cast<int64_t>(j) * p.hq + kvh * p.group + hh) * kD;
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
            const u32x4_t x = qrow_ok ? ld<u32x4_t>(qp + 16 * sd + 8 * g) : u32x4_t{0, 0, 0, 0};
            qop[sd] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    float m = -INFINITY;
    float l = 0.f;
    f32x16_t acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
    const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

    const char* const kpool = static_cast<const char*>(p.k_pool) + static_cast<int64_t>(kvh) * kTile * kElt;
    const char* const vpool = static_cast<const char*>(p.v_pool) + static_cast<int64_t>(kvh) * kTile * kElt;
    const uint32_t koff = static_cast<uint32_t>(KV == PKV_BF16 ? 16 * t : ((t >> 4) * kD + (t & 15) * 8) * kElt);
    const uint32_t voff = static_cast<uint32_t>(
        KV == PKV_BF16 ? 16 * (64 * (t >> 6) + 16 * v_piece(t).g + v_piece(t).r) : byte_v_offset(t >> 1, (t & 1) * 8));
    const uint32_t voff1 = static_cast<uint32_t>(KV == PKV_BF16 ? 0 : byte_v_offset(t >> 1, (t & 1) * 8 + 4));
    const int krow0 = key_row(c32) * kKStride + 8 * g;
    const int vrow0 = v_lds_offset(c32, g);

    bool bad = false;
    Stage<KV> sk, sv;  // every thread stages a piece of K and of V
    // block ids read one staging step ahead of their tiles (as in the chunk
    // kernel); ids holds those of the next stage_load
    int32_t ids[4];
    auto load_ids = [&](int it) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int lb = min(it * 4 + b, nblk_seq - 1);
            ids[b] = lb >= 0 ? trow[lb] : 0;
        }
    };
    auto stage_load = [&](int it, int next) {
        const char* kb[4];
        const char* vb[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            int32_t id = __builtin_amdgcn_readfirstlane(ids[b]);
            if (id < 0 || id >= p.num_blocks) {
                bad = bad || nblk_seq > 0;  // (a row with no blocks reads block 0 unchecked)
                id = 0;
            }
            kb[b] = kpool + id * blk_bytes;
            vb[b] = vpool + id * blk_bytes;
        }
        sk.k_load(kb, koff);
        sv.v_load(vb, voff, voff1);
        load_ids(next);
    };
    auto stage_store = [&](int it, int buf) {
        if ((it + 1) * kKeys > L) {
            int valid[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) valid[b] = min(kBS, max(0, L - (it * 4 + b) * kBS));
            sv.mask_tail(valid, t);
        }
        sk.k_store(ks[buf], t);
        sv.v_store(vs[buf], t);
    };

    auto compute = [&](int it, int buf) {
        const uint16_t* kc = ks[buf] + krow0;
        const uint16_t* vc = vs[buf] + vrow0;
        const int kbase = it * kKeys;
        f32x16_t sc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[kt][i] = 0.f;
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ld<u32x4_t>(kc + 32 * kt * kKStride + 16 * sd));
                sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[sd], sc[kt], 0, 0, 0);
            }
        }
        if (kbase + kKeys - 1 > last_key) {  // the range's end inside this iteration
            const int lastc = last_key - kbase - 8 * g;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kt + 16 * (i >> 3) + (i & 7) > lastc) sc[kt][i] = -INFINITY;
        }
        float mb = sc[0][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mb = fmaxf(mb, sc[0][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mb = fmaxf(mb, sc[1][i]);
        mb *= scale;
        if (__any(mb > m + kLazy)) {
            mb = fmaxf(mb, __shfl_xor(mb, 32));
            const float mn = fmaxf(m, mb);
            const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
            m = mn;
        }
        const float neg_m = m == -INFINITY ? 0.f : -m;
        u32x4_t pw[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kt][8 * h + 2 * e], scale, neg_m));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kt][8 * h + 2 * e + 1], scale, neg_m));
                    const uint32_t w = pack_bf16(p0, p1);
                    pw[kt][h][e] = w;
                    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, l, false);
                }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x8_t b = __builtin_bit_cast(bf16x8_t, pw[kt][h]);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x8_t a =
                        __builtin_bit_cast(bf16x8_t, ld<u32x4_t>(vc + (2 * kt + h) * kTile + 32 * dt * kBS));
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[dt], 0, 0, 0);
                }
            }
    };

    // one register stage and two LDS buffers: the loads for iteration it + 1
    // are issued before iteration it is computed and stored after it
    const int it_begin = static_cast<int>(static_cast<int64_t>(n_iter) * part / p.parts);
    const int it_end = static_cast<int>(static_cast<int64_t>(n_iter) * (part + 1) / p.parts);
    const int last = max(it_end - 1, it_begin);
    load_ids(it_begin);
    stage_load(it_begin, min(it_begin + 1, last));
    if (it_end > it_begin) stage_store(it_begin, 0);
    __syncthreads();
    for (int it = it_begin; it < it_end; ++it) {
        const int cur = (it - it_begin) & 1;
        stage_load(min(it + 1, last), min(it + 2, last));
        compute(it, cur);
        if (it + 1 < it_end) stage_store(it + 1, cur ^ 1);
        __syncthreads();
    }

    bad = bad || !row_ok || (qrow_ok && broken[tok] != 0);
    l += __shfl_xor(l, 32);
    if (!qrow_ok) return;
    const float nan = __builtin_nanf("");
    float* sp = p.states + ((static_cast<int64_t>(part) * p.total_q + j) * p.hq + kvh * p.group + hh) * kState;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t v = {acc[dt][4 * q4], acc[dt][4 * q4 + 1], acc[dt][4 * q4 + 2], acc[dt][4 * q4 + 3]};
            st<f32x4_t>(sp + 32 * dt + 8 * q4 + 4 * g, bad ? f32x4_t{nan, nan, nan, nan} : v);
        }
    if (g == 0) st<float2>(sp + kD, float2{m, bad ? nan : l});
}

}  // namespace pf

// Parameters of the shared-prefix pass of a decode call over `rows` rows
// (every row's state over each of prefix_parts() ranges of the first
// a->shared_prefix_blocks blocks of table row 0, into states
// [parts][rows][hq][kState]); returns the workgroups of the pass.
int prefix_pass_params(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, const void* q,
                       const int32_t* table, float* states, pf::PrefillParams* p);

}  // namespace pkv
