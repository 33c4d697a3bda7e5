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
// Work decomposition: one workgroup (4 waves) per (chunk row, kv head, tile of
// 16 query tokens); the G query heads of the kv head are split over the waves
// (NT heads per wave), so each staged K/V tile serves 16 * G query rows.
// Per iteration the workgroup gathers 64 keys (4 blocks, through the block
// table) into LDS - K as [key][d] with rows padded to 136 elements, V as
// [block][d][16 tokens] with rows padded to 20 elements, both to keep the
// operand reads free of bank conflicts - double buffered, one barrier per
// iteration.  Each wave then computes, per head tile (16 tokens of one head):
//   S^T[64 keys x 16 tokens] = K . Q^T           (16 x mfma 16x16x32 bf16)
//   O^T[128 x 16 tokens]    += V^T . P^T         (8 d-tiles x 2 key halves, P rounded to bf16)
// with the running max / normaliser of the decode kernel (rescaled lazily,
// only when a score passes the reference max by 2^8) and the causal mask
// applied only where a key can pass a query's position.  For P.V the 32 keys
// of one instruction are taken in the order the score tiles leave them in the
// lanes (keys 4g..4g+3 of two consecutive blocks), and V is read in the same
// order, so no lane exchange is needed between the two products.
// fp8 caches are converted to bf16 while staging (exact) with the per-head
// scales folded into the score scale and the output.
#include <cmath>

#include "device.h"
#include "internal.h"

namespace pkv {

int launch_decode(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, int32_t max_kv_len, const void* q,
                  void* out, const int32_t* table, const int32_t* kv_lens, void* workspace, size_t ws_bytes,
                  hipStream_t stream);

namespace {

constexpr int kQTile = 16;             // query tokens per workgroup
constexpr int kKeys = 64;              // keys per iteration (4 blocks)
constexpr int kKStride = kD + 8;       // padded K row (elements)
constexpr int kVStride = kBS + 4;      // padded V^T row (elements)
constexpr int kKStage = 4 * kBS * kKStride;   // elements of one K stage
constexpr int kVStage = 4 * kD * kVStride;    // elements of one V stage
constexpr float kLazy = 8.0f;                 // rescale threshold (log2 units)

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
    int32_t row0, num_blocks, hkv, hq, group, max_blocks, max_kv_len, q_tiles, total_q;
    float scale_log2;
};

// 8 probabilities as one bf16 MFMA operand, rounded to nearest even (a pair
// per v_cvt_pk_bf16_f32).  Each p is in (0, 2^8], so its relative rounding
// error is at most 2^-9 and the output moves by at most 2^-9 of the spread of
// the values it averages.
__device__ __forceinline__ bf16x8_t to_bf16x8(const float p[8]) {
    bf16x8_t r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(p[i]);
    return r;
}

// Staging registers for one iteration: thread t owns 16 bytes of each of the
// iteration's 4 K tiles (row t/16, elements (t%16)*8..+7) and 4 V^T tiles
// (d row t/2, tokens (t%2)*8..+7); fp8 codes are converted to bf16 on load.
// The tile addresses are uniform (one per block) and the thread's offset
// inside a tile is fixed, so a load costs no vector arithmetic.
template <int KV>
struct Stage {
    u32x4_t k[4], v[4];
    // voff: this thread's V^T piece (bf16); fp8 tiles keep it as two 4-byte
    // words at voff and voff1 (fp8_v_offset)
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
                const u32x2_t k0 = fp8x4_to_bf16x4(kk[0]), k1 = fp8x4_to_bf16x4(kk[1]);
                const u32x2_t v0 = fp8x4_to_bf16x4(vv[0]), v1 = fp8x4_to_bf16x4(vv[1]);
                k[b] = u32x4_t{k0[0], k0[1], k1[0], k1[1]};
                v[b] = u32x4_t{v0[0], v0[1], v1[0], v1[1]};
            }
        }
    }
    // Zero V^T of tokens at or past valid[b] (the row's partial last block and
    // blocks past its end, which hold whatever the clamped load read; 0 * NaN
    // is NaN).  Only the iteration that reaches the row's end calls this.
    __device__ __forceinline__ void mask_tail(const int valid[4], int t) {
        const int tok0 = (t & 1) * 8;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t w[4] = {v[b][0], v[b][1], v[b][2], v[b][3]};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (tok0 + e >= valid[b]) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            v[b] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
    }
    __device__ __forceinline__ void store(uint16_t* ks, uint16_t* vs, int t) const {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            st<u32x4_t>(ks + (b * kBS + (t >> 4)) * kKStride + (t & 15) * 8, k[b]);
            uint16_t* vrow = vs + (b * kD + (t >> 1)) * kVStride + (t & 1) * 8;
            st<u32x2_t>(vrow, u32x2_t{v[b][0], v[b][1]});
            st<u32x2_t>(vrow + 4, u32x2_t{v[b][2], v[b][3]});
        }
    }
};

// bf16 1.0 in both halves: the A operand of the "ones" tile whose product
// with P^T is the row sum of P.
constexpr uint32_t kOnes2 = 0x3F803F80u;

template <int KV, int NT>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][kKStage];
    __shared__ __attribute__((aligned(16))) uint16_t vs[2][kVStage];
    constexpr int kElt = (KV == PKV_BF16) ? 2 : 1;

    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int lane = t & 63;
    const int r = lane & 15;
    const int g = lane >> 4;
    // blockIdx -> (row, q tile, kv head), kv head fastest (one kv head per XCD).
    const int per_row = p.q_tiles * p.hkv;
    const int row = p.row0 + blockIdx.x / per_row;
    const int rem = blockIdx.x % per_row;
    const int qt = rem / p.hkv;
    const int kvh = rem % p.hkv;

    const int qbeg = p.cu_q[row];
    const int C = p.cu_q[row + 1] - qbeg;
    const int j0 = qt * kQTile;
    if (j0 >= C || qbeg < 0 || qbeg + C > p.total_q) return;  // (a malformed cu_q writes nothing)
    const int L = p.kv_lens[row];
    const bool row_ok = C >= 1 && L >= C && L <= p.max_kv_len && L <= p.max_blocks * kBS;
    const int P = L - C;
    const int jmax = min(j0 + kQTile, C);         // exclusive
    const int kend = row_ok ? P + jmax : 0;       // keys this tile needs
    const int n_iter = (kend + kKeys - 1) / kKeys;
    const int nblk_seq = (L + kBS - 1) / kBS;
    const int64_t blk_bytes = static_cast<int64_t>(p.hkv) * kTile * kElt;
    const int32_t* trow = p.table + static_cast<int64_t>(row) * p.max_blocks;

    // this lane's query token (clamped for tile rows past the chunk's end)
    const int j = min(j0 + r, C - 1);
    const int qpos = P + j;  // keys 0..qpos are visible

    float scale = p.scale_log2;
    float vscale = 1.f;
    if constexpr (KV == PKV_FP8_E4M3) {
        scale *= p.k_scale[kvh];
        vscale = p.v_scale[kvh];
    }

    // Q^T operands of this wave's heads: Q[token j][head][32 ks + 8 g .. +7]
    bf16x8_t qop[NT][4];
    bool head_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int hh = wave * NT + nt;
        head_ok[nt] = hh < p.group;
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                             (static_cast<int64_t>(qbeg + j) * p.hq + kvh * p.group + (head_ok[nt] ? hh : 0)) * kD;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const u32x4_t x = head_ok[nt] ? ld<u32x4_t>(qp + 32 * k4 + 8 * g) : u32x4_t{0, 0, 0, 0};
            qop[nt][k4] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    // acc[nt][0..7]: O^T d-tiles; acc[nt][8]: the row sum of P (ones tile)
    float m[NT];
    f32x4_t acc[NT][9];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m[nt] = -INFINITY;
#pragma unroll
        for (int i = 0; i < 9; ++i) acc[nt][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{kOnes2, kOnes2, kOnes2, kOnes2});

    const char* const kpool = static_cast<const char*>(p.k_pool) + static_cast<int64_t>(kvh) * kTile * kElt;
    const char* const vpool = static_cast<const char*>(p.v_pool) + static_cast<int64_t>(kvh) * kTile * kElt;
    const uint32_t koff = static_cast<uint32_t>(((t >> 4) * kD + (t & 15) * 8) * kElt);
    const uint32_t voff = static_cast<uint32_t>(
        KV == PKV_BF16 ? ((t >> 1) * kBS + (t & 1) * 8) * kElt : fp8_v_offset(t >> 1, (t & 1) * 8));
    const uint32_t voff1 = static_cast<uint32_t>(KV == PKV_BF16 ? 0 : fp8_v_offset(t >> 1, (t & 1) * 8 + 4));

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
        const uint16_t* kc = ks[buf];
        const uint16_t* vc = vs[buf];
        const int kbase = it * kKeys;
        // S^T tiles: s[nt][b] holds keys kbase + 16 b + 4 g + i for token row r
        f32x4_t s[NT][4];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int b = 0; b < 4; ++b) s[nt][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ld<u32x4_t>(kc + (b * kBS + r) * kKStride + 32 * k4 + 8 * g));
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    s[nt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[nt][k4], s[nt][b], 0, 0, 0);
            }
        }
        // online softmax per head tile.  Scores stay unscaled until the
        // exponent (scale > 0, so the maximum commutes with it); keys can pass
        // a query's position only in the iterations that reach the diagonal,
        // so only those take the masked path (a uniform branch).
        const bool need_mask = kbase + kKeys - 1 > P + j0;
        bf16x8_t pb[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float x[16];
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[4 * b + i] = s[nt][b][i];
            if (need_mask) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (kbase + 16 * b + 4 * g + i > qpos) x[4 * b + i] = -INFINITY;
            }
            float mb = fmaxf(fmaxf(x[0], x[1]), x[2]);
#pragma unroll
            for (int i = 3; i < 16; i += 2) mb = fmaxf(fmaxf(mb, x[i]), x[i + 1 < 16 ? i + 1 : i]);
            mb *= scale;
            // lazy rescale (as in the decode kernel): only when some score
            // passes the reference max by more than kLazy
            if (__any(mb > m[nt] + kLazy)) {
                mb = fmaxf(mb, __shfl_xor(mb, 16));
                mb = fmaxf(mb, __shfl_xor(mb, 32));
                const float mn = fmaxf(m[nt], mb);
                const float alpha = __builtin_amdgcn_exp2f(m[nt] - mn);
#pragma unroll
                for (int i = 0; i < 9; ++i) acc[nt][i] *= alpha;
                m[nt] = mn;
            }
            const float neg_m = -m[nt];
            float pr[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(x[i], scale, neg_m));
            // k-step h covers blocks 2h, 2h+1: this lane's 8 keys are
            // (block 2h: 4g..4g+3, block 2h+1: 4g..4g+3)
#pragma unroll
            for (int h = 0; h < 2; ++h) pb[nt][h] = to_bf16x8(pr + 8 * h);
        }
        // O^T += V^T . P^T, and the row sum of P through the ones tile
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint16_t* v0 = vc + ((2 * h) * kD + 16 * mt + r) * kVStride + 4 * g;
                const uint16_t* v1 = vc + ((2 * h + 1) * kD + 16 * mt + r) * kVStride + 4 * g;
                const u32x2_t a0 = ld<u32x2_t>(v0);
                const u32x2_t a1 = ld<u32x2_t>(v1);
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, u32x4_t{a0[0], a0[1], a1[0], a1[1]});
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[nt][h], acc[nt][mt], 0, 0, 0);
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt][8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[nt][h], acc[nt][8], 0, 0, 0);
    };

    // One register stage and two LDS buffers: the loads for iteration it + 1
    // are issued before iteration it is computed and stored to the other LDS
    // buffer after it.  The loads are unconditional (clamped iteration), so no
    // branch sits between a load and its use.
    Stage<KV> sreg;
    const int last = max(n_iter - 1, 0);
    stage_load(sreg, 0);
    if (n_iter > 0) stage_store(sreg, 0, 0);
    __syncthreads();
    for (int it = 0; it < n_iter; ++it) {
        const int cur = it & 1;
        stage_load(sreg, min(it + 1, last));
        compute(it, cur);
        if (it + 1 < n_iter) stage_store(sreg, it + 1, cur ^ 1);
        __syncthreads();
    }

    bad = bad || !row_ok;
    const bool tok_ok = j0 + r < C;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (!head_ok[nt] || !tok_ok) continue;
        const float inv = bad ? __builtin_nanf("") : vscale / acc[nt][8][0];
        const int hh = wave * NT + nt;
        uint16_t* op = static_cast<uint16_t*>(p.out) +
                       (static_cast<int64_t>(qbeg + j0 + r) * p.hq + kvh * p.group + hh) * kD;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const f32x4_t v = acc[nt][mt] * inv;
            const uint32_t a = bf16_bits_rne(v[0]) | (bf16_bits_rne(v[1]) << 16);
            const uint32_t b2 = bf16_bits_rne(v[2]) | (bf16_bits_rne(v[3]) << 16);
            st<u32x2_t>(op + 16 * mt + 4 * g, u32x2_t{a, b2});
        }
    }
}

template <int KV>
void launch_prefill_kv(int nt, dim3 grid, hipStream_t s, const PrefillParams& p) {
    switch (nt) {
        case 1: hipLaunchKernelGGL((prefill_kernel<KV, 1>), grid, dim3(256), 0, s, p); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<KV, 2>), grid, dim3(256), 0, s, p); break;
        case 3: hipLaunchKernelGGL((prefill_kernel<KV, 3>), grid, dim3(256), 0, s, p); break;
        default: hipLaunchKernelGGL((prefill_kernel<KV, 4>), grid, dim3(256), 0, s, p); break;
    }
}

}  // namespace
}  // namespace pkv

using pkv::fail;

extern "C" int paged_attn_prefill_chunk(const pkv_cache* c, const pkv_attn_args* a, void* stream) {
    int st = pkv::check_attn(c, a);
    if (st) return st;
    if (a->num_seqs == 0) return PKV_OK;
    if (c->kv_dtype == PKV_F32) return fail(PKV_ERR_UNSUPPORTED, "chunked prefill supports bf16 and fp8 caches");
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
    const int32_t nt = (group + 3) / 4;
    const int32_t q_tiles = (a->max_q_len + pkv::kQTile - 1) / pkv::kQTile;
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
    p.q_tiles = q_tiles;
    p.total_q = a->total_q;
    p.scale_log2 = pkv::kLog2e / sqrtf(static_cast<float>(pkv::kD));
    if (c->kv_dtype == PKV_BF16)
        pkv::launch_prefill_kv<PKV_BF16>(nt, dim3(static_cast<unsigned>(grid)), s, p);
    else
        pkv::launch_prefill_kv<PKV_FP8_E4M3>(nt, dim3(static_cast<unsigned>(grid)), s, p);
    if (a->events[3]) (void)hipEventRecord(static_cast<hipEvent_t>(a->events[3]), s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    return PKV_OK;
}
