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
// Work decomposition: one workgroup (8 waves) per (chunk row, tile of query
// rows, key range, kv head).  A query row is one (token, query head) pair; the
// G heads of one kv head share its K/V, so a tile holds 256 / G consecutive
// tokens with all G heads each (256 rows), and wave w owns rows 32 w .. 32 w +
// 31 (row n is token n / G, head n % G).  Per iteration the workgroup walks 64
// keys (4 blocks, gathered through the block table) staged in LDS - K as
// [key][d] with rows padded to 136 elements, V as [d][16 tokens] tiles with
// the two 8-token halves of a row swapped on alternate groups of 8 rows (both
// layouts keep the operand reads free of bank conflicts).  Each wave computes,
// on the 32x32x16 bf16 matrix instruction:
//   S^T[64 keys x 32 rows] = K . Q^T        (2 key tiles x 8 steps over d)
//   O^T[128 x 32 rows]    += V^T . P^T      (4 d tiles x 4 steps of 16 keys)
// and between the two the online softmax of its 64 x 32 scores (exponentials,
// maxima, the bf16 rounding of P and the normaliser), which costs the vector
// unit about as long as the products cost the matrix unit.
//
// Ping-pong.  The 8 waves form two groups of 4, one wave of each group per
// SIMD.  Workgroup barriers cut the iterations into phases, and the groups
// swap roles at every barrier.  In its matrix phase a wave computes the
// exponentials of iteration i between the P.V products that consume them,
// then K.Q^T of iteration i + 1; in its other phase it masks and takes the
// maxima of those new scores (and, rarely, rescales) and stages the next K or
// V tile.  The vector work of the exponentials runs in the shadow of the
// wave's own products (measured faster than leaving the whole softmax to the
// other phase), and the other group's short phase keeps the SIMD's second
// wave off the matrix unit.  Group 0 stages the K tiles and group 1 the V
// tiles, from registers loaded two phases earlier; two LDS buffers for K and
// two for V are enough for this order (a buffer is rewritten only after both
// groups have read it).  One staged tile serves 256 query rows.
//
// The lane holding a score column keeps that row's softmax state: running max
// (rescaled lazily, only when a score passes it by 2^8) and normaliser.  The
// rows of K fed to the score product are permuted (bits 2 and 3 of the key
// index swapped), so that the score registers come out holding, for each
// 16-key step, exactly the 8 consecutive keys the P.V operand of that lane
// needs: P goes from the score registers to the second product with no lane
// exchange, and V is read in the cache's token order.  P is rounded to bf16
// once; the normaliser sums the same rounded values (bf16 dot products with
// 1.0), so the rounding largely cancels between numerator and denominator.
// fp8 and int8 caches are converted to bf16 while staging (exact) with the
// per-head scales folded into the score scale and the output.
//
// Key ranges.  When the tiles alone would leave compute units idle, each tile's
// keys are split into ranges (whole iterations); a range's state (unnormalised
// output, running max, normaliser) goes to the workspace and a merge kernel
// combines the ranges of every query with the max/normaliser algebra of the
// online softmax.  The same products and softmax, without the causal mask,
// compute the decode rows' states over a prefix all rows share (the
// shared-prefix pass: prefix_tile in prefill_tiles.h, which the decode launch
// runs).
#include <cmath>

#include <cstdlib>
#include <type_traits>

#include "device.h"
#include "internal.h"
#include "prefill_tiles.h"

using namespace pkv::pf;

namespace pkv {

int launch_decode(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, int32_t max_kv_len, const void* q,
                  void* out, const int32_t* table, const int32_t* kv_lens, void* workspace, size_t ws_bytes,
                  hipStream_t stream);

namespace {

constexpr int kThreads = 512;          // 8 waves: two groups of 4, one wave of each per SIMD
constexpr int kRows = 256;             // query rows per workgroup (8 waves x 32)
constexpr int kMaxParts = 8;               // key ranges per tile

// Workgroup barrier that orders LDS only: the stores before it are complete
// (lgkmcnt) and no LDS access moves across it, while global loads issued
// before it stay in flight (the staging loads run two phases ahead).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Chunk rows of a prefill call.
template <int KV>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][kKStage];
    __shared__ __attribute__((aligned(16))) uint16_t vs[2][kVStage];
    constexpr int kElt = (KV == PKV_BF16) ? 2 : 1;

    const int t = threadIdx.x;
    const int wave = t >> 6;
    // 0: stages K, starts with the matrix phase; 1: stages V.  Read through
    // readfirstlane so the compiler sees a wave-uniform value and branches on
    // it with scalar branches, each group's phases compiled as straight code.
    const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
    const int u = t & 255;      // thread index within its group
    const int lane = t & 63;
    const int c32 = lane & 31;  // score column = query row within the wave
    const int g = lane >> 5;    // lane group
    // blockIdx -> (row, q tile, key range, kv head), kv head fastest (one kv
    // head per XCD: the workgroups of one head share its K/V in that L2).
    const int per_row = p.q_tiles * p.parts * p.hkv;
    const int row = p.row0 + blockIdx.x / per_row;
    const int kvh = blockIdx.x % p.hkv;
    const int part = (blockIdx.x / p.hkv) % p.parts;
    const int qt = (blockIdx.x % per_row) / (p.hkv * p.parts);
    const bool split = p.parts > 1;  // states to the workspace, not outputs

    const int qbeg = p.cu_q[row];
    const int C = p.cu_q[row + 1] - qbeg;
    const int j0 = qt * p.tile_tokens;
    if (j0 >= C || qbeg < 0 || qbeg + C > p.total_q) return;  // (a malformed cu_q writes nothing)
    const int L = p.kv_lens[row];
    // a chunk row with more queries than max_q_len is invalid: every query of
    // it gets NaN, the last tile filling the queries that no tile owns
    const int covered = p.q_tiles * p.tile_tokens;
    const bool over = C > p.max_q_len;
    const bool row_ok = C >= 1 && L >= C && L <= p.max_kv_len && L <= p.max_blocks * kBS && !over;
    if (C > covered && qt == p.q_tiles - 1 && part == 0) {
        // bf16 NaN x 8 into the output, or NaN states (normaliser NaN) when
        // the ranges are merged later
        const u32x4_t nan8 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
        const int per_tok = p.group * (split ? 1 : kD / 8);
        const int pieces = (C - covered) * per_tok;
        for (int e = t; e < pieces; e += kThreads) {
            const int tok_e = covered + e / per_tok;
            const int rest = e % per_tok;
            const int64_t q_h = static_cast<int64_t>(qbeg + tok_e) * p.hq + kvh * p.group;
            if (split) {
                st<float2>(p.states + (q_h + rest) * kState + kD, float2{0.f, __builtin_nanf("")});
            } else {
                uint16_t* o = static_cast<uint16_t*>(p.out) + (q_h + rest / (kD / 8)) * kD + 8 * (rest % (kD / 8));
                st<u32x4_t>(o, nan8);
            }
        }
    }
    const int P = L - C;  // keys before the chunk
    const int jmax = min(j0 + p.tile_tokens, C);  // exclusive
    const int kend = row_ok ? P + jmax : 0;  // keys this tile needs
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
    const int qpos = P + j;        // keys 0..qpos are visible
    const int first_pos = P + j0;  // the smallest qpos in the tile

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
    f32x16_t acc[4];      // O^T d tiles: d = 32 dt + 8 (i / 4) + 4 g + i % 4
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
    const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

    const char* const kpool = static_cast<const char*>(p.k_pool) + static_cast<int64_t>(kvh) * kTile * kElt;
    const char* const vpool = static_cast<const char*>(p.v_pool) + static_cast<int64_t>(kvh) * kTile * kElt;
    const uint32_t koff = static_cast<uint32_t>(KV == PKV_BF16 ? 16 * u : ((u >> 4) * kD + (u & 15) * 8) * kElt);
    const uint32_t voff = static_cast<uint32_t>(
        KV == PKV_BF16 ? 16 * (64 * (u >> 6) + 16 * v_piece(u).g + v_piece(u).r) : byte_v_offset(u >> 1, (u & 1) * 8));
    const uint32_t voff1 = static_cast<uint32_t>(KV == PKV_BF16 ? 0 : byte_v_offset(u >> 1, (u & 1) * 8 + 4));
    // LDS element offsets of this lane's operands
    const int krow0 = key_row(c32) * kKStride + 8 * g;  // + (32 kt) * kKStride + 16 sd
    const int vrow0 = v_lds_offset(c32, g);             // + b * kTile + (32 dt) * kBS

    // Tile addresses of iteration it's 4 blocks (uniform).  Blocks past the
    // row's end read its last block (their V is zeroed by mask_tail, their
    // keys are masked); a block id outside the pool reads block 0 and makes
    // the output NaN.
    bool bad = false;
    // The block ids of an iteration are read from the table one staging step
    // before its tiles are loaded (ids holds the next iteration's), so no
    // phase waits out a table read before it can issue its tile loads.
    int32_t ids[4];
    auto load_ids = [&](int it) {
#pragma unroll
        for (int b = 0; b < 4; ++b) ids[b] = trow[min(it * 4 + b, nblk_seq - 1)];
    };
    auto tiles = [&](const char* const pool, const char* tb[4]) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            int32_t id = __builtin_amdgcn_readfirstlane(ids[b]);  // the same in every lane
            if (id < 0 || id >= p.num_blocks) {
                bad = true;
                id = 0;
            }
            tb[b] = pool + id * blk_bytes;
        }
    };
    Stage<KV> sr;
    // load the tiles of iteration it (ids holds its block ids), then read the
    // ids of iteration it + 1 (clamped to the row's blocks: in the table)
    auto k_load = [&](int it) {
        const char* kb[4];
        tiles(kpool, kb);
        sr.k_load(kb, koff);
        load_ids(it + 1);
    };
    auto v_load = [&](int it) {
        const char* vb[4];
        tiles(vpool, vb);
        sr.v_load(vb, voff, voff1);
        load_ids(it + 1);
    };
    auto k_store = [&](int it) { sr.k_store(ks[it & 1], u); };
    auto v_store = [&](int it) {
        if ((it + 1) * kKeys > L) {  // the iteration that reaches the row's end
            int valid[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) valid[b] = min(kBS, max(0, L - (it * 4 + b) * kBS));
            sr.mask_tail(valid, u);
        }
        sr.v_store(vs[it & 1], u);
    };

    // Scores of the iteration this wave works on, and its P operand: step
    // (kt, h) covers keys 32 kt + 16 h + 8 g .. +7 (block 2 kt + h).
    f32x16_t s[2];
    u32x4_t pk[2][2];
    // The scheduling barriers at the end of qk and pv keep each operand read
    // four products ahead of its use: in its matrix phase this wave is the
    // only one issuing products on its SIMD, so nothing else hides the LDS
    // latency.
    auto prefetch4 = [](auto products) {
        constexpr int kAhead = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // four LDS reads
#pragma unroll
        for (int n = 0; n < decltype(products)::value - kAhead; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a product
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the read four ahead
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    };
    // S^T = K . Q^T over the 64 keys of iteration it (K in buffer it & 1)
    auto qk = [&](int it) {
        const uint16_t* kc = ks[it & 1] + krow0;
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
    };
    // O^T += V^T . P^T over iteration it's 64 keys (V in buffer it & 1)
    auto pv = [&](int it) {
        const uint16_t* vc = vs[it & 1] + vrow0;
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
    // Online softmax of iteration it's scores (in place in s), in two parts
    // that run in different phases.  smax: the causal mask, the maximum and
    // the lazy rescale; sexp: the exponentials, their bf16 rounding into pk
    // and the normaliser.  sexp runs in the wave's own matrix phase, between
    // the P.V products that consume its results, so the vector unit works in
    // the shadow of this wave's products while the other group's wave runs
    // its (shorter) smax and staging.
    // Scores stay unscaled until the exponent (scale > 0, so the maximum
    // commutes with it); keys can pass a query's position only in the
    // iterations that reach the diagonal, so only those take the masked path
    // (a uniform branch).  The maximum and the normaliser are accumulated in
    // four independent chains (one per 16-key step), so that one wave's
    // dependent instructions do not wait on each other.
    float lp[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's normaliser, per step
    auto smax = [&](int it) {
        const int kbase = it * kKeys;
        if (kbase + kKeys - 1 > first_pos) {
            // score (kt, i) is key kbase + 8 g + c with c = 32 kt + 16 (i / 8) + i % 8
            const int last = qpos - kbase - 8 * g;  // the largest visible c
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kt + 16 * (i >> 3) + (i & 7) > last) s[kt][i] = -INFINITY;
        }
        float mc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int kt = c >> 1, o = 8 * (c & 1);
            float x = fmaxf(s[kt][o], s[kt][o + 1]);
#pragma unroll
            for (int e = 2; e < 8; e += 2) x = fmaxf(fmaxf(x, s[kt][o + e]), s[kt][o + e + 1]);
            mc[c] = x;
        }
        float mb = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3])) * scale;
        // A row can still have seen no key at all (m = -inf): in a key range
        // past its diagonal every score is masked.  Its state stays (-inf, 0,
        // 0) and contributes nothing when the ranges are merged.
        if (__any(mb > m + kLazy)) {  // rare: a new maximum for some row
            mb = fmaxf(mb, __shfl_xor(mb, 32));
            const float mn = fmaxf(m, mb);
            const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
            for (int c = 0; c < 4; ++c) lp[c] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
            m = mn;
        }
    };
    auto sexp = [&] {
        // The scores enter this phase here: a barrier does not order plain
        // arithmetic, and the compiler would otherwise hoist part of the
        // exponentials into the previous phase.
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) asm volatile("" : "+v"(s[kt]));
        const float neg_m = m == -INFINITY ? 0.f : -m;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * h + 2 * e], scale, neg_m));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * h + 2 * e + 1], scale, neg_m));
                    const uint32_t w = pack_bf16(p0, p1);
                    pk[kt][h][e] = w;
                    lp[2 * kt + h] =
                        __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, lp[2 * kt + h], false);
                }
            }
    };
    // Every product of a matrix phase is issued before its barrier (the
    // empty statements take the results as operands).
    auto pin_s = [&] {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) asm volatile("" : "+v"(s[kt]));
    };
    auto pin_acc = [&] {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) asm volatile("" : "+v"(acc[dt]));
    };
    // A wave's matrix phase: P.V of iteration it, then K.Q^T of iteration
    // it + 1 (next: there is one), with the operand reads four products ahead
    // across both.
    auto mma_phase = [&](int it, auto next) {
        sexp();
        pv(it);
        if constexpr (decltype(next)::value) {
            qk(it + 1);
            prefetch4(std::integral_constant<int, 32>{});
            pin_s();
        } else {
            prefetch4(std::integral_constant<int, 16>{});
        }
        pin_acc();
    };
    const std::true_type with_qk{};
    const std::false_type last_pv{};

    // The workgroup's iterations: its key range of the tile's n_iter.
    const int ib = static_cast<int>(static_cast<int64_t>(n_iter) * part / p.parts);
    const int ie = static_cast<int>(static_cast<int64_t>(n_iter) * (part + 1) / p.parts);
    // Schedule (phases end at a barrier; group 0 = A, group 1 = B):
    //   prologue: A stages K(ib), K(ib+1) and loads K(ib+2); B stages V(ib) and loads V(ib+1)
    //   P0: A: qk(ib)
    //   P1: A: smax(ib)                                      B: qk(ib)
    //   for it = ib .. ie-1:
    //     a: A: sexp(it), pv(it), qk(it+1)                   B: smax(it), store V(it+1), load V(it+2)
    //     b: A: smax(it+1), store K(it+2), load K(it+3)      B: sexp(it), pv(it), qk(it+1)
    // (no qk(it+1) in the last iteration).  K(x) lands in ks[x & 1] in phase
    // b of iteration x - 2, after both groups read K(x - 2) (B in phase b of
    // iteration x - 3); V(x) lands in vs[x & 1] in phase a of iteration x - 1,
    // after both read V(x - 2) (B in phase b of iteration x - 2).  Each group
    // runs its own loop (straight code per phase for the compiler; the last
    // iteration is peeled so the matrix phase has no branch); both pass the
    // same barriers.
    if (ie > ib) {
        load_ids(ib);
        if (grp == 0) {
            k_load(ib);
            k_store(ib);
            if (ib + 1 < ie) {
                k_load(ib + 1);
                k_store(ib + 1);
            }
            if (ib + 2 < ie) k_load(ib + 2);
            lds_barrier();
            qk(ib);
            lds_barrier();
            smax(ib);
            lds_barrier();
            for (int it = ib; it + 1 < ie; ++it) {
                mma_phase(it, with_qk);
                lds_barrier();
                smax(it + 1);
                if (it + 2 < ie) {
                    k_store(it + 2);
                    if (it + 3 < ie) k_load(it + 3);
                }
                lds_barrier();
            }
            mma_phase(ie - 1, last_pv);
            lds_barrier();
            lds_barrier();
        } else {
            v_load(ib);
            v_store(ib);
            if (ib + 1 < ie) v_load(ib + 1);
            lds_barrier();
            lds_barrier();
            qk(ib);
            lds_barrier();
            for (int it = ib; it + 1 < ie; ++it) {
                smax(it);
                v_store(it + 1);
                if (it + 2 < ie) v_load(it + 2);
                lds_barrier();
                mma_phase(it, with_qk);
                lds_barrier();
            }
            smax(ie - 1);
            lds_barrier();
            mma_phase(ie - 1, last_pv);
            lds_barrier();
        }
    }

    bad = bad || !row_ok;
    float l = (lp[0] + lp[1]) + (lp[2] + lp[3]);
    l += __shfl_xor(l, 32);
    if (!qrow_ok) return;
    if (split) {  // the range's state, unnormalised (merged later)
        const float nan = __builtin_nanf("");
        const int64_t qi = qbeg + j;
        float* sp = p.states + ((static_cast<int64_t>(part) * p.total_q + qi) * p.hq + kvh * p.group + hh) * kState;
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

// Combines the key ranges of chunk queries q0 .. total_q - 1: for query q and
// head h, with range k's state (acc_k, m_k, l_k) and M = max_k m_k, the output
// is sum_k acc_k 2^(m_k - M) / sum_k l_k 2^(m_k - M), times v_scale of h's kv
// head.  32 threads per (query, head), 4 d each; ranges in order.
__global__ __launch_bounds__(256) void prefill_merge_kernel(const PrefillParams p, int q0) {
    const int64_t qh = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);  // (q - q0) * hq + h
    const int d = 4 * (threadIdx.x & 31);
    if (qh >= static_cast<int64_t>(p.total_q - q0) * p.hq) return;
    const int64_t q = q0 + qh / p.hq;
    const int h = static_cast<int>(qh % p.hq);
    const int64_t stride = static_cast<int64_t>(p.total_q) * p.hq * kState;
    const float* s0 = p.states + (q * p.hq + h) * kState;
    float mk[kMaxParts];
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) mk[k] = k < p.parts ? s0[k * stride + kD] : -INFINITY;
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) mx = fmaxf(mx, mk[k]);
    float lsum = 0.f;
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) {
        if (k < p.parts) {
            const float w = __builtin_amdgcn_exp2f(mk[k] - mx);
            lsum += s0[k * stride + kD + 1] * w;
            o += ld<f32x4_t>(s0 + k * stride + d) * w;
        }
    }
    const float vscale = p.v_scale ? p.v_scale[h / p.group] : 1.f;
    const float inv = vscale / lsum;
    const uint32_t a = bf16_bits_rne(o[0] * inv) | (bf16_bits_rne(o[1] * inv) << 16);
    const uint32_t b = bf16_bits_rne(o[2] * inv) | (bf16_bits_rne(o[3] * inv) << 16);
    st<u32x2_t>(static_cast<uint16_t*>(p.out) + (q * p.hq + h) * kD + d, u32x2_t{a, b});
}

int device_cus() {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    return cus;
}

// PKV_PREFIX_PARTS overrides the shared-prefix pass's key-range count for tuning runs.
int env_int(const char* name) {
    const char* e = std::getenv(name);
    return e ? std::atoi(e) : 0;
}

}  // namespace

// Key ranges the shared-prefix pass splits into: enough workgroups for one
// per compute unit (measured on 256 rows of a 2000-token prefix: two ranges
// beat four, as each range's states are written and combined), each range at
// least one 64-key iteration, at most 8.
int prefix_parts(const pkv_cache* c, const pkv_attn_args* a, int32_t rows) {
    const int32_t group = a->num_q_heads / c->num_kv_heads;
    const int64_t tiles =
        static_cast<int64_t>((rows + kPrefixRows / group - 1) / (kPrefixRows / group)) * c->num_kv_heads;
    const int64_t iters = (static_cast<int64_t>(a->shared_prefix_blocks) * kBS + kKeys - 1) / kKeys;
    static const int env = env_int("PKV_PREFIX_PARTS");
    int64_t parts = env > 0 ? env : (device_cus() + tiles - 1) / tiles;
    parts = parts < 1 ? 1 : (parts > kMaxParts ? kMaxParts : parts);
    return static_cast<int>(parts < iters ? parts : (iters < 1 ? 1 : iters));
}

// Key ranges per tile of a chunked-prefill launch: when the (row, q tile, kv
// head) tiles are fewer than the compute units, enough ranges for one
// workgroup per compute unit, each at least 8 iterations of the longest row,
// at most 8.
int prefill_parts(const pkv_cache* c, const pkv_attn_args* a) {
    const int32_t n_pre = a->num_seqs - a->num_decode;
    if (!a->cu_q || n_pre <= 0 || a->max_q_len <= 0) return 1;
    if (a->prefill_parts > 0) return a->prefill_parts < kMaxParts ? a->prefill_parts : kMaxParts;
    const int32_t group = a->num_q_heads / c->num_kv_heads;
    const int32_t tile_tokens = kRows / group;
    const int64_t tiles = static_cast<int64_t>(n_pre) * ((a->max_q_len + tile_tokens - 1) / tile_tokens) *
                          c->num_kv_heads;
    int64_t parts = (device_cus() + tiles - 1) / tiles;
    const int64_t by_len = (static_cast<int64_t>(a->max_kv_len) + 8 * kKeys - 1) / (8 * kKeys);
    if (parts > by_len) parts = by_len;
    return static_cast<int>(parts < 1 ? 1 : (parts > kMaxParts ? kMaxParts : parts));
}

// Workspace of the chunk rows: range states when split (bytes).
size_t prefill_workspace_bytes(const pkv_cache* c, const pkv_attn_args* a) {
    const int parts = prefill_parts(c, a);
    if (parts <= 1) return 0;
    return static_cast<size_t>(parts) * static_cast<size_t>(a->total_q) * a->num_q_heads * kState * sizeof(float);
}

int prefix_pass_params(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, const void* q,
                       const int32_t* table, float* states, pf::PrefillParams* out) {
    const int32_t group = a->num_q_heads / c->num_kv_heads;
    const int32_t tile_tokens = kPrefixRows / group;
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
    p.parts = prefix_parts(c, a, rows);
    *out = p;
    return q_tiles * c->num_kv_heads * p.parts;
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

    // workspace: the decode rows' part, then the chunk rows' range states
    const size_t dec_bytes = pkv::decode_workspace_bytes(c, a, a->num_decode);
    const size_t pre_off = (dec_bytes + 255) / 256 * 256;
    const size_t pre_bytes = pkv::prefill_workspace_bytes(c, a);
    if (pre_bytes > 0 && (!a->workspace || a->workspace_bytes < pre_off + pre_bytes))
        return fail(PKV_ERR_WORKSPACE, "prefill needs %zu workspace bytes, got %zu", pre_off + pre_bytes,
                    a->workspace ? a->workspace_bytes : 0);

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
    const int32_t parts = pkv::prefill_parts(c, a);
    const int64_t grid = static_cast<int64_t>(n_pre) * q_tiles * parts * c->num_kv_heads;
    if (grid > INT32_MAX) return fail(PKV_ERR_INVALID, "prefill launch too large");
    const int64_t elt = c->kv_dtype == PKV_BF16 ? 2 : 1;
    const int64_t layer_elems = static_cast<int64_t>(c->num_blocks) * c->num_kv_heads * pkv::kTile;
    pkv::pf::PrefillParams p{};
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
    p.parts = parts;
    p.states = parts > 1 ? reinterpret_cast<float*>(static_cast<char*>(a->workspace) + pre_off) : nullptr;
    const dim3 g1(static_cast<unsigned>(grid));
    if (c->kv_dtype == PKV_BF16)
        hipLaunchKernelGGL((pkv::prefill_kernel<PKV_BF16>), g1, dim3(pkv::kThreads), 0, s, p);
    else if (c->kv_dtype == PKV_FP8_E4M3)
        hipLaunchKernelGGL((pkv::prefill_kernel<PKV_FP8_E4M3>), g1, dim3(pkv::kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((pkv::prefill_kernel<PKV_INT8>), g1, dim3(pkv::kThreads), 0, s, p);
    if (parts > 1) {
        // the chunk rows' queries are num_decode .. total_q - 1 (decode row i holds query i)
        const int64_t pairs = static_cast<int64_t>(a->total_q - a->num_decode) * a->num_q_heads;
        const dim3 mg(static_cast<unsigned>((pairs + 7) / 8));
        hipLaunchKernelGGL(pkv::prefill_merge_kernel, mg, dim3(256), 0, s, p, a->num_decode);
    }
    if (a->events[3]) (void)hipEventRecord(static_cast<hipEvent_t>(a->events[3]), s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    return PKV_OK;
}
