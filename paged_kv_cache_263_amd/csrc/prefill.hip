// Chunked prefill batched with decode rows, on gfx950.
//
// A long prompt is processed in chunks interleaved with decode steps of other
// requests ([P1] "Serving systems: the layer that survives real traffic"; [P3]
// "prefill vs decode phase separation", item (e)).  A chunk row holds C
// queries that are the last C of its L cached tokens (their K/V are already in
// the cache): query j attends keys 0..L-C+j.  Prefill attention is a dense,
// compute-bound contraction ([P3] same section, item (a)), so both products
// run on the matrix cores with shapes the hardware takes whole ([P1] "Kernel
// engineering: the layer underneath everything else here" on tile shapes).
//
// Work decomposition: one workgroup (4 waves) per (chunk row, kv head, tile
// of query rows).  A query row is one (token, query head) pair; the G heads of
// one kv head share its K/V, so a tile holds 128 / G consecutive tokens with
// all G heads each (128 rows), and wave w owns rows 32 w .. 32 w + 31 (row n
// is token n / G, head n % G).  Per iteration the workgroup gathers 64 keys
// (4 blocks, through the block table) into LDS - K as [key][d] with rows
// padded to 136 elements, V as [d][16 tokens] tiles with the two 8-token
// halves of a row swapped on alternate groups of 8 rows (both layouts keep the
// operand reads free of bank conflicts) - double buffered, one barrier per
// iteration.  Each
// wave then computes, on the 32x32x16 bf16 matrix instruction:
//   S^T[64 keys x 32 rows] = K . Q^T        (2 key tiles x 8 steps over d)
//   O^T[128 x 32 rows]    += V^T . P^T      (4 d tiles x 4 steps of 16 keys)
// The lane holding a score column keeps that row's softmax state: running
// max (rescaled lazily, only when a score passes it by 2^8) and normaliser.
// The rows of K fed to the score product are permuted (bits 2 and 3 of the
// key index swapped), so that the score registers come out holding, for each
// 16-key step, exactly the 8 consecutive keys the P.V operand of that lane
// needs: P goes from the score registers to the second product with no lane
// exchange, and V is read in the cache's token order.  P is rounded to bf16 once;
// the normaliser sums the same rounded values (bf16 dot products with 1.0),
// so the rounding largely cancels between numerator and denominator.
// fp8 and int8 caches are converted to bf16 while staging (exact) with the
// per-head scales folded into the score scale and the output.
#include <cmath>

#include <cstdlib>

#include "device.h"
#include "internal.h"

namespace pkv {

int launch_decode(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, int32_t max_kv_len, const void* q,
                  void* out, const int32_t* table, const int32_t* kv_lens, void* workspace, size_t ws_bytes,
                  hipStream_t stream);

namespace {

constexpr int kRows = 128;             // query rows per workgroup (4 waves x 32)
constexpr int kKeys = 64;              // keys per iteration (4 blocks)
constexpr int kKStride = kD + 8;       // padded K row (elements)
constexpr int kKStage = kKeys * kKStride;  // elements of one K stage
constexpr int kVStage = 4 * kTile;         // elements of one V stage (4 tiles [128][16])
constexpr float kLazy = 8.0f;              // rescale threshold (log2 units)

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
    // shared-prefix pass (PREFIX kernels): the decode rows' queries (one per
    // row, total_q rows) over the first prefix_tokens keys of table row 0, no
    // causal mask, the keys split into prefix_parts ranges of whole
    // iterations; the state of (part, row, head) goes to
    // states[part][row][hq][kPrefixState]
    float* states;
    int32_t prefix_tokens, prefix_parts;
};

// Floats of one (row, query head) shared-prefix state: unnormalised output
// [128], running max (log2 units), normaliser, padding (the decode kernel
// reads the same layout).
constexpr int kPrefixState = kD + 4;

// LDS element offset of tokens 8 h .. 8 h + 7 of d row d inside a staged V
// tile: rows of 16 tokens, the two halves swapped in rows with bit 3 of d
// set, so that the 16 lanes of one operand read (d rows r .. r + 15, same h)
// cover all 64 banks.
__device__ __forceinline__ int v_lds_offset(int d, int h) { return d * kBS + 8 * (h ^ ((d >> 3) & 1)); }

// bf16 V piece staged by thread t: a permutation of the pieces inside each
// wave's contiguous 1 KiB of the tile (so the global load stays one
// contiguous run per wave), chosen so that every 16 lanes of the two 8-byte
// LDS stores below write distinct banks.  Lane 16 a + b takes d row
// r = 4 a + b % 4 (and r + 16) of the wave's 32 rows, token group
// g = 2 h + (b / 4) % 2 with h = (b / 8) ^ (a / 2).
struct VPiece {
    int r, g;
};
__device__ __forceinline__ VPiece v_piece(int t) {
    const int a = (t >> 4) & 3, b = t & 15;
    const int r = 4 * a + (b & 3);
    const int h = ((b >> 3) & 1) ^ (a >> 1);
    return VPiece{r, 2 * h + ((b >> 2) & 1)};
}

// Staging registers for one iteration: thread t owns 16 bytes of each of the
// iteration's 4 K tiles and 4 V tiles.  bf16 tiles (bf16_k_offset,
// bf16_v_offset): K piece t, token t%16, d 8(t/16)..+7; V piece
// 64 (t/64) + 16 g + r (v_piece), tokens 4g..4g+3 of d rows 32(t/64) + r and
// that + 16; 256 threads read each 4 KiB tile contiguously.
// One-byte tiles: K row t/16, elements (t%16)*8..+7, and V d row t/2, tokens
// (t%2)*8..+7, their codes converted to bf16 on load.
// The tile addresses are uniform (one per block) and the thread's offset
// inside a tile is fixed, so a load costs no vector arithmetic.
template <int KV>
struct Stage {
    u32x4_t k[4], v[4];
    // voff: this thread's V piece (bf16); one-byte tiles keep it as two 4-byte
    // words at voff and voff1 (byte_v_offset)
    __device__ __forceinline__ void load(const char* const kb[4], const char* const vb[4], uint32_t koff,
                                         uint32_t voff, uint32_t voff1) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (KV == PKV_BF16) {
                k[b] = ld<u32x4_t>(kb[b] + koff);
                v[b] = ld<u32x4_t>(vb[b] + voff);
            } else {
                const u32x2_t kk = ld<u32x2_t>(kb[b] + koff);
                const u32x2_t vv = {ld<uint32_t>(vb[b] + voff), ld<uint32_t>(vb[b] + voff1)};
                const u32x2_t k0 = byte4_to_bf16x4<KV>(kk[0]), k1 = byte4_to_bf16x4<KV>(kk[1]);
                const u32x2_t v0 = byte4_to_bf16x4<KV>(vv[0]), v1 = byte4_to_bf16x4<KV>(vv[1]);
                k[b] = u32x4_t{k0[0], k0[1], k1[0], k1[1]};
                v[b] = u32x4_t{v0[0], v0[1], v1[0], v1[1]};
            }
        }
    }
    // Zero V of tokens at or past valid[b] (the row's partial last block and
    // blocks past its end, which hold whatever the clamped load read; 0 * NaN
    // is NaN).  Only the iteration that reaches the row's end calls this.
    __device__ __forceinline__ void mask_tail(const int valid[4], int t) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t w[4] = {v[b][0], v[b][1], v[b][2], v[b][3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // token of element e
                const int tok = KV == PKV_BF16 ? 4 * v_piece(t).g + (e & 3) : (t & 1) * 8 + e;
                if (tok >= valid[b]) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            }
            v[b] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
    }
    __device__ __forceinline__ void store(uint16_t* ks, uint16_t* vs, int t) const {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (KV == PKV_BF16) {
                st<u32x4_t>(ks + (b * kBS + (t & 15)) * kKStride + 8 * (t >> 4), k[b]);
                const VPiece vp = v_piece(t);
                const int g = vp.g;
                const int d0 = 32 * (t >> 6) + vp.r;
                uint16_t* vt = vs + b * kTile + 4 * (g & 1);
                st<u32x2_t>(vt + v_lds_offset(d0, g >> 1), u32x2_t{v[b][0], v[b][1]});
                st<u32x2_t>(vt + v_lds_offset(d0 + 16, g >> 1), u32x2_t{v[b][2], v[b][3]});
            } else {
                st<u32x4_t>(ks + (b * kBS + (t >> 4)) * kKStride + (t & 15) * 8, k[b]);
                st<u32x4_t>(vs + b * kTile + v_lds_offset(t >> 1, t & 1), v[b]);
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

// PREFIX: the shared-prefix pass of a decode call (see PrefillParams); else a
// chunked-prefill row.
template <int KV, bool PREFIX>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][kKStage];
    __shared__ __attribute__((aligned(16))) uint16_t vs[2][kVStage];
    constexpr int kElt = (KV == PKV_BF16) ? 2 : 1;

    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int lane = t & 63;
    const int c32 = lane & 31;  // score column = query row within the wave
    const int g = lane >> 5;    // lane group
    // blockIdx -> (row, q tile, kv head), kv head fastest (one kv head per XCD).
    const int per_row = p.q_tiles * p.hkv;
    const int row = PREFIX ? 0 : p.row0 + blockIdx.x / per_row;
    const int kvh = blockIdx.x % p.hkv;
    const int qt = PREFIX ? blockIdx.x / (p.hkv * p.prefix_parts) : (blockIdx.x % per_row) / p.hkv;
    const int part = PREFIX ? (blockIdx.x / p.hkv) % p.prefix_parts : 0;

    const int qbeg = PREFIX ? 0 : p.cu_q[row];
    const int C = PREFIX ? p.total_q : p.cu_q[row + 1] - qbeg;
    const int j0 = qt * p.tile_tokens;
    if (j0 >= C || qbeg < 0 || qbeg + C > p.total_q) return;  // (a malformed cu_q writes nothing)
    // P: keys before the chunk (prefix pass: the prefix; every query sees all of it)
    const int L = PREFIX ? p.prefix_tokens : p.kv_lens[row];
    // a chunk row with more queries than max_q_len is invalid: every query of
    // it gets NaN, the last tile filling the queries that no tile owns
    const int covered = p.q_tiles * p.tile_tokens;
    const bool over = !PREFIX && C > p.max_q_len;
    const bool row_ok = PREFIX ? L >= kBS
                               : C >= 1 && L >= C && L <= p.max_kv_len && L <= p.max_blocks * kBS && !over;
    if (!PREFIX && C > covered && qt == p.q_tiles - 1) {
        const u32x4_t nan8 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};  // bf16 NaN x 8
        const int pieces = (C - covered) * p.group * (kD / 8);
        for (int e = t; e < pieces; e += 256) {
            const int tok_e = covered + e / (p.group * (kD / 8));
            const int rest = e % (p.group * (kD / 8));
            uint16_t* o = static_cast<uint16_t*>(p.out) +
                          (static_cast<int64_t>(qbeg + tok_e) * p.hq + kvh * p.group + rest / (kD / 8)) * kD +
                          8 * (rest % (kD / 8));
            st<u32x4_t>(o, nan8);
        }
    }
    // Prefix pass: the caller promises that every row's table starts with
    // row 0's first prefix_tokens / 16 block ids.  Each workgroup checks the
    // promise for its own rows; a row that breaks it gets a NaN state, so its
    // output is NaN like that of any other invalid row.
    __shared__ int broken[kRows];
    if constexpr (PREFIX) {
        for (int i = t; i < p.tile_tokens; i += 256) broken[i] = 0;
        __syncthreads();
        const int S = p.prefix_tokens / kBS;
        const int ntok = min(p.tile_tokens, C - j0);
        for (int e = t; e < ntok * S; e += 256) {
            const int r = e / S, b = e - r * S;
            if (p.table[static_cast<int64_t>(j0 + r) * p.max_blocks + b] != p.table[b]) broken[r] = 1;
        }
        // (read after the barrier that follows the first stage store)
    }
    const int P = PREFIX ? L : L - C;
    const int jmax = min(j0 + p.tile_tokens, C);  // exclusive
    const int kend = row_ok ? (PREFIX ? P : P + jmax) : 0;  // keys this tile needs
    const int n_iter = (kend + kKeys - 1) / kKeys;
    const int nblk_seq = (L + kBS - 1) / kBS;
    const int64_t blk_bytes = static_cast<int64_t>(p.hkv) * kTile * kElt;
    const int32_t* trow = p.table + static_cast<int64_t>(row) * p.max_blocks;

    // this lane's query row: token j0 + n / G, head n % G (tokens past the
    // chunk's end are clamped and not stored)
    const int n = 32 * wave + c32;
    const int tok = n / p.group;
    const int hh = n - tok * p.group;
    const bool qrow_ok = tok < p.tile_tokens && j0 + tok < C;
    const int j = min(j0 + tok, C - 1);
    const int qpos = PREFIX ? P - 1 : P + j;    // keys 0..qpos are visible
    const int first_pos = PREFIX ? P - 1 : P + j0;  // the smallest qpos in the tile

    float scale = p.scale_log2;
    float vscale = 1.f;
    if constexpr (is_byte_dtype(KV)) {
        scale *= p.k_scale[kvh];
        vscale = p.v_scale[kvh];
    }

    // Q^T operand: Q[row][16 s + 8 g .. +7] for the 8 steps over d
    bf16x8_t qop[8];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                             (static_cast<int64_t>(qbeg + j) * p.hq + kvh * p.group + hh) * kD;
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
            const u32x4_t x = qrow_ok ? ld<u32x4_t>(qp + 16 * sd + 8 * g) : u32x4_t{0, 0, 0, 0};
            qop[sd] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    float m = -INFINITY;  // reference max (log2 units), same in both lane groups
    float l = 0.f;        // this lane's part of the normaliser
    f32x16_t acc[4];      // O^T d tiles: d = 32 dt + 8 (i / 4) + 4 g + i % 4
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
    // LDS element offsets of this lane's operands
    const int krow0 = key_row(c32) * kKStride + 8 * g;  // + (32 kt) * kKStride + 16 sd
    const int vrow0 = v_lds_offset(c32, g);             // + b * kTile + (32 dt) * kBS

    // Tile addresses of iteration it's 4 blocks (uniform).  Blocks past the
    // row's end read its last block (their V is zeroed by mask_tail, their
    // keys are masked); a block id outside the pool reads block 0 and makes
    // the output NaN.
    bool bad = false;
    auto stage_load = [&](Stage<KV>& sr, int it) {
        const char* kb[4];
        const char* vb[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int lb = min(it * 4 + b, nblk_seq - 1);
            int32_t id = lb >= 0 ? trow[lb] : 0;
            if (id < 0 || id >= p.num_blocks) {
                bad = bad || lb >= 0;
                id = 0;
            }
            kb[b] = kpool + id * blk_bytes;
            vb[b] = vpool + id * blk_bytes;
        }
        sr.load(kb, vb, koff, voff, voff1);
    };
    auto stage_store = [&](Stage<KV>& sr, int it, int buf) {
        if ((it + 1) * kKeys > L) {  // the iteration that reaches the row's end
            int valid[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) valid[b] = min(kBS, max(0, L - (it * 4 + b) * kBS));
            sr.mask_tail(valid, t);
        }
        sr.store(ks[buf], vs[buf], t);
    };

    // one iteration over the 64 keys staged in LDS buffer buf
    auto compute = [&](int it, int buf) {
        const uint16_t* kc = ks[buf] + krow0;
        const uint16_t* vc = vs[buf] + vrow0;
        const int kbase = it * kKeys;
        f32x16_t s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ld<u32x4_t>(kc + 32 * kt * kKStride + 16 * sd));
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[sd], s[kt], 0, 0, 0);
            }
        }
        // online softmax.  Scores stay unscaled until the exponent (scale >
        // 0, so the maximum commutes with it); keys can pass a query's
        // position only in the iterations that reach the diagonal, so only
        // those take the masked path (a uniform branch).
        float x[32];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) x[16 * kt + i] = s[kt][i];
        if (kbase + kKeys - 1 > first_pos) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kbase + 32 * kt + 16 * (i >> 3) + 8 * g + (i & 7) > qpos) x[16 * kt + i] = -INFINITY;
        }
        float mb = x[0];
#pragma unroll
        for (int i = 1; i < 31; i += 2) mb = fmaxf(fmaxf(mb, x[i]), x[i + 1]);
        mb = fmaxf(mb, x[31]) * scale;
        if (__any(mb > m + kLazy)) {  // rare: a new maximum for some row
            mb = fmaxf(mb, __shfl_xor(mb, 32));
            const float mn = fmaxf(m, mb);
            const float alpha = __builtin_amdgcn_exp2f(m - mn);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
            m = mn;
        }
        const float neg_m = -m;
        // P^T operand of step (kt, h): keys 32 kt + 16 h + 8 g .. +7
        u32x4_t pk[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float pr[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pr[e] = __builtin_amdgcn_exp2f(fmaf(x[16 * kt + 8 * h + e], scale, neg_m));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = pack_bf16(pr[2 * e], pr[2 * e + 1]);
                    pk[kt][h][e] = w;
                    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, l, false);
                }
            }
        // O^T += V^T . P^T: step (kt, h) covers block 2 kt + h
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x8_t b = __builtin_bit_cast(bf16x8_t, pk[kt][h]);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x8_t a =
                        __builtin_bit_cast(bf16x8_t, ld<u32x4_t>(vc + (2 * kt + h) * kTile + 32 * dt * kBS));
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[dt], 0, 0, 0);
                }
            }
    };

    // One register stage and two LDS buffers: the loads for iteration it + 1
    // are issued before iteration it is computed and stored to the other LDS
    // buffer after it.  The loads are unconditional (clamped iteration), so no
    // branch sits between a load and its use.
    // (a prefix-pass workgroup walks its part's range of iterations)
    const int it_begin = PREFIX ? static_cast<int>(static_cast<int64_t>(n_iter) * part / p.prefix_parts) : 0;
    const int it_end = PREFIX ? static_cast<int>(static_cast<int64_t>(n_iter) * (part + 1) / p.prefix_parts) : n_iter;
    Stage<KV> sreg;
    const int last = max(it_end - 1, it_begin);
    stage_load(sreg, it_begin);
    if (it_end > it_begin) stage_store(sreg, it_begin, 0);
    __syncthreads();
    for (int it = it_begin; it < it_end; ++it) {
        const int cur = (it - it_begin) & 1;
        stage_load(sreg, min(it + 1, last));
        compute(it, cur);
        if (it + 1 < it_end) stage_store(sreg, it + 1, cur ^ 1);
        __syncthreads();
    }

    bad = bad || !row_ok;
    if constexpr (PREFIX) bad = bad || (qrow_ok && broken[tok] != 0);
    l += __shfl_xor(l, 32);
    if (!qrow_ok) return;
    if constexpr (PREFIX) {  // the state, unnormalised (the decode kernel continues from it)
        const float nan = __builtin_nanf("");
        float* sp = p.states + ((static_cast<int64_t>(part) * p.total_q + j) * p.hq + kvh * p.group + hh) * kPrefixState;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4_t v = {acc[dt][4 * q4], acc[dt][4 * q4 + 1], acc[dt][4 * q4 + 2], acc[dt][4 * q4 + 3]};
                st<f32x4_t>(sp + 32 * dt + 8 * q4 + 4 * g, bad ? f32x4_t{nan, nan, nan, nan} : v);
            }
        if (g == 0) st<float2>(sp + kD, float2{m, bad ? nan : l});
        return;
    }
    const float inv = bad ? __builtin_nanf("") : vscale / l;
    uint16_t* op = static_cast<uint16_t*>(p.out) +
                   (static_cast<int64_t>(qbeg + j) * p.hq + kvh * p.group + hh) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const uint32_t a = bf16_bits_rne(acc[dt][4 * q4] * inv) | (bf16_bits_rne(acc[dt][4 * q4 + 1] * inv) << 16);
            const uint32_t b2 =
                bf16_bits_rne(acc[dt][4 * q4 + 2] * inv) | (bf16_bits_rne(acc[dt][4 * q4 + 3] * inv) << 16);
            st<u32x2_t>(op + 32 * dt + 8 * q4 + 4 * g, u32x2_t{a, b2});
        }
}

}  // namespace

// Key ranges the shared-prefix pass splits into: enough workgroups for one
// per compute unit (measured on 256 rows: two ranges beat four by 5 us, as
// each range's states are written and combined), each range at least one
// 64-key iteration, at most 8.
int prefix_parts(const pkv_cache* c, const pkv_attn_args* a, int32_t rows) {
    const int32_t group = a->num_q_heads / c->num_kv_heads;
    const int64_t tiles = static_cast<int64_t>((rows + kRows / group - 1) / (kRows / group)) * c->num_kv_heads;
    const int64_t iters = (static_cast<int64_t>(a->shared_prefix_blocks) * kBS + kKeys - 1) / kKeys;
    static const int env = [] {  // PKV_PREFIX_PARTS overrides the count for tuning runs
        const char* e = std::getenv("PKV_PREFIX_PARTS");
        return e ? std::atoi(e) : 0;
    }();
    int64_t parts = env > 0 ? env : (256 + tiles - 1) / tiles;
    parts = parts < 1 ? 1 : (parts > 8 ? 8 : parts);
    return static_cast<int>(parts < iters ? parts : (iters < 1 ? 1 : iters));
}

// The shared-prefix pass of a decode call: every row's (query head) state over
// the first 16 * S tokens of table row 0, into states [rows][hq][kPrefixState].
int launch_prefix_states(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, const void* q,
                         const int32_t* table, float* states, void* stream_ptr) {
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    if (c->kv_dtype == PKV_F32) return fail(PKV_ERR_UNSUPPORTED, "a shared prefix needs a bf16, fp8 or int8 cache");
    const int32_t group = a->num_q_heads / c->num_kv_heads;
    const int32_t tile_tokens = kRows / group;
    const int32_t q_tiles = (rows + tile_tokens - 1) / tile_tokens;
    const int64_t elt = c->kv_dtype == PKV_BF16 ? 2 : 1;
    const int64_t layer_elems = static_cast<int64_t>(c->num_blocks) * c->num_kv_heads * kTile;
    PrefillParams p{};
    p.q = q;
    p.k_pool = static_cast<const char*>(c->k_pool) + a->layer * layer_elems * elt;
    p.v_pool = static_cast<const char*>(c->v_pool) + a->layer * layer_elems * elt;
    p.k_scale = c->k_scale ? c->k_scale + static_cast<int64_t>(a->layer) * c->num_kv_heads : nullptr;
    p.v_scale = c->v_scale ? c->v_scale + static_cast<int64_t>(a->layer) * c->num_kv_heads : nullptr;
    p.table = table;
    p.row0 = 0;
    p.num_blocks = c->num_blocks;
    p.hkv = c->num_kv_heads;
    p.hq = a->num_q_heads;
    p.group = group;
    p.max_blocks = a->max_blocks;
    p.max_kv_len = a->max_kv_len;
    p.q_tiles = q_tiles;
    p.total_q = rows;
    p.tile_tokens = tile_tokens;
    p.scale_log2 = kLog2e / sqrtf(static_cast<float>(kD));
    p.states = states;
    p.prefix_tokens = a->shared_prefix_blocks * kBS;
    p.prefix_parts = prefix_parts(c, a, rows);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(q_tiles) * c->num_kv_heads * p.prefix_parts));
    if (c->kv_dtype == PKV_BF16)
        hipLaunchKernelGGL((prefill_kernel<PKV_BF16, true>), grid, dim3(256), 0, stream, p);
    else if (c->kv_dtype == PKV_FP8_E4M3)
        hipLaunchKernelGGL((prefill_kernel<PKV_FP8_E4M3, true>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<PKV_INT8, true>), grid, dim3(256), 0, stream, p);
    return PKV_OK;
}

}  // namespace pkv

using pkv::fail;

extern "C" int paged_attn_prefill_chunk(const pkv_cache* c, const pkv_attn_args* a, void* stream) {
    int st = pkv::check_attn(c, a);
    if (st) return st;
    if (a->num_seqs == 0) return PKV_OK;
    if (c->kv_dtype == PKV_F32) return fail(PKV_ERR_UNSUPPORTED, "chunked prefill supports bf16, fp8 and int8 caches");
    if (!a->cu_q) return fail(PKV_ERR_INVALID, "prefill needs cu_q");
    if (a->num_decode < 0 || a->num_decode > a->num_seqs) return fail(PKV_ERR_INVALID, "bad num_decode %d", a->num_decode);
    const int32_t n_pre = a->num_seqs - a->num_decode;
    if (n_pre > 0 && (a->max_q_len <= 0 || a->total_q < a->num_decode + n_pre))
        return fail(PKV_ERR_INVALID, "max_q_len must be positive and total_q must cover every row");
    hipStream_t s = static_cast<hipStream_t>(stream);

    // decode rows: queries 0..num_decode-1, one per row
    const int32_t dec_len = a->max_decode_kv_len > 0 ? a->max_decode_kv_len : a->max_kv_len;
    if (dec_len > a->max_kv_len) return fail(PKV_ERR_INVALID, "max_decode_kv_len exceeds max_kv_len");
    st = pkv::launch_decode(c, a, a->num_decode, dec_len, a->q, a->out, a->block_table, a->kv_lens,
                            a->workspace, a->workspace_bytes, s);
    if (st) return st;
    if (n_pre == 0) {
        if (a->events[3]) (void)hipEventRecord(static_cast<hipEvent_t>(a->events[3]), s);
        return PKV_OK;
    }

    const int32_t group = a->num_q_heads / c->num_kv_heads;
    const int32_t tile_tokens = pkv::kRows / group;
    const int32_t q_tiles = (a->max_q_len + tile_tokens - 1) / tile_tokens;
    const int64_t grid = static_cast<int64_t>(n_pre) * q_tiles * c->num_kv_heads;
    if (grid > INT32_MAX) return fail(PKV_ERR_INVALID, "prefill launch too large");
    const int64_t elt = c->kv_dtype == PKV_BF16 ? 2 : 1;
    const int64_t layer_elems = static_cast<int64_t>(c->num_blocks) * c->num_kv_heads * pkv::kTile;
    pkv::PrefillParams p{};
    p.q = a->q;
    p.out = a->out;
    p.k_pool = static_cast<const char*>(c->k_pool) + a->layer * layer_elems * elt;
    p.v_pool = static_cast<const char*>(c->v_pool) + a->layer * layer_elems * elt;
    p.k_scale = c->k_scale ? c->k_scale + static_cast<int64_t>(a->layer) * c->num_kv_heads : nullptr;
    p.v_scale = c->v_scale ? c->v_scale + static_cast<int64_t>(a->layer) * c->num_kv_heads : nullptr;
    p.table = a->block_table;
    p.kv_lens = a->kv_lens;
    p.cu_q = a->cu_q;
    p.row0 = a->num_decode;
    p.num_blocks = c->num_blocks;
    p.hkv = c->num_kv_heads;
    p.hq = a->num_q_heads;
    p.group = group;
    p.max_blocks = a->max_blocks;
    p.max_kv_len = a->max_kv_len;
    p.max_q_len = a->max_q_len;
    p.q_tiles = q_tiles;
    p.total_q = a->total_q;
    p.tile_tokens = tile_tokens;
    p.scale_log2 = pkv::kLog2e / sqrtf(static_cast<float>(pkv::kD));
    if (c->kv_dtype == PKV_BF16)
        hipLaunchKernelGGL((pkv::prefill_kernel<PKV_BF16, false>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, p);
    else if (c->kv_dtype == PKV_FP8_E4M3)
        hipLaunchKernelGGL((pkv::prefill_kernel<PKV_FP8_E4M3, false>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((pkv::prefill_kernel<PKV_INT8, false>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, p);
    if (a->events[3]) (void)hipEventRecord(static_cast<hipEvent_t>(a->events[3]), s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    return PKV_OK;
}
