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
//   O^T[128 x 16 tokens]    += V^T . P^T         (8 d-tiles x 2 key halves, P as bf16 hi + lo)
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

// Split 8 probabilities into bf16 high parts (truncated) and bf16 remainders,
// packed as two MFMA operands; v_perm_b32 picks the upper halves of two fp32
// values into one register (bytes 2,3 of the second source, then of the first).
__device__ __forceinline__ uint32_t pack_hi16(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
__device__ __forceinline__ void split_p8(const float p[8], bf16x8_t& hi, bf16x8_t& lo) {
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = p[i] - __uint_as_float(__float_as_uint(p[i]) & 0xFFFF0000u);
    hi = __builtin_bit_cast(bf16x8_t, u32x4_t{pack_hi16(p[0], p[1]), pack_hi16(p[2], p[3]), pack_hi16(p[4], p[5]),
                                              pack_hi16(p[6], p[7])});
    lo = __builtin_bit_cast(bf16x8_t, u32x4_t{pack_hi16(r[0], r[1]), pack_hi16(r[2], r[3]), pack_hi16(r[4], r[5]),
                                              pack_hi16(r[6], r[7])});
}

// Staging registers for one iteration: thread t owns chunk t of each of the 4
// blocks, for K (row t/16, 8 elements at (t%16)*8) and for V^T (d row t/2,
// tokens (t%2)*8..+7).
template <int KV>
struct Stage {
    u32x4_t k[4], v[4];  // bf16 values (fp8 converted on load)
    // valid[b]: tokens of block b at or past it are unwritten (only the row's
    // last block is partial); their V is zeroed, since 0 * NaN is NaN.
    __device__ __forceinline__ void load(const void* kp, const void* vp, const int64_t blk[4], const int valid[4],
                                         int t) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (blk[b] < 0) {
                k[b] = u32x4_t{0, 0, 0, 0};
                v[b] = u32x4_t{0, 0, 0, 0};
                continue;
            }
            if constexpr (KV == PKV_BF16) {
                const uint16_t* kt = static_cast<const uint16_t*>(kp) + blk[b];
                const uint16_t* vt = static_cast<const uint16_t*>(vp) + blk[b];
                k[b] = ld<u32x4_t>(kt + (t >> 4) * kD + (t & 15) * 8);
                v[b] = ld<u32x4_t>(vt + (t >> 1) * kBS + (t & 1) * 8);
            } else {
                const uint8_t* kt = static_cast<const uint8_t*>(kp) + blk[b];
                const uint8_t* vt = static_cast<const uint8_t*>(vp) + blk[b];
                const u32x2_t kk = ld<u32x2_t>(kt + (t >> 4) * kD + (t & 15) * 8);
                const u32x2_t vv = ld<u32x2_t>(vt + (t >> 1) * kBS + (t & 1) * 8);
                const u32x2_t k0 = fp8x4_to_bf16x4(kk[0]), k1 = fp8x4_to_bf16x4(kk[1]);
                const u32x2_t v0 = fp8x4_to_bf16x4(vv[0]), v1 = fp8x4_to_bf16x4(vv[1]);
                k[b] = u32x4_t{k0[0], k0[1], k1[0], k1[1]};
                v[b] = u32x4_t{v0[0], v0[1], v1[0], v1[1]};
            }
            if (valid[b] < kBS) {  // V^T chunk: tokens (t & 1) * 8 .. +7 of d row t / 2
                const int tok0 = (t & 1) * 8;
                uint32_t w[4] = {v[b][0], v[b][1], v[b][2], v[b][3]};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (tok0 + e >= valid[b]) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                v[b] = u32x4_t{w[0], w[1], w[2], w[3]};
            }
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

template <int KV, int NT>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][kKStage];
    __shared__ __attribute__((aligned(16))) uint16_t vs[2][kVStage];

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
    const int64_t blk_stride = static_cast<int64_t>(p.hkv) * kTile;
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

    float m[NT], l[NT];
    f32x4_t acc[NT][8];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m[nt] = -INFINITY;
        l[nt] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[nt][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const int koff = kvh * kTile;
    const void* kp = static_cast<const char*>(p.k_pool) + static_cast<int64_t>(koff) * (KV == PKV_BF16 ? 2 : 1);
    const void* vp = static_cast<const char*>(p.v_pool) + static_cast<int64_t>(koff) * (KV == PKV_BF16 ? 2 : 1);

    bool bad = false;
    auto block_offsets = [&](int it, int64_t blk[4], int valid[4]) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int lb = it * 4 + b;
            int32_t id = -1;
            if (lb < nblk_seq) id = trow[lb];
            if (lb < nblk_seq && (id < 0 || id >= p.num_blocks)) {
                bad = true;
                id = -1;
            }
            blk[b] = id < 0 ? -1 : static_cast<int64_t>(id) * blk_stride;
            valid[b] = min(kBS, max(0, L - lb * kBS));
        }
    };

    Stage<KV> sreg;
    if (n_iter > 0) {
        int64_t blk[4];
        int valid[4];
        block_offsets(0, blk, valid);
        sreg.load(kp, vp, blk, valid, t);
        sreg.store(ks[0], vs[0], t);
    }
    __syncthreads();

    for (int it = 0; it < n_iter; ++it) {
        const int cur = it & 1;
        if (it + 1 < n_iter) {
            int64_t blk[4];
            int valid[4];
            block_offsets(it + 1, blk, valid);
            sreg.load(kp, vp, blk, valid, t);
        }
        const uint16_t* kc = ks[cur];
        const uint16_t* vc = vs[cur];
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
        bf16x8_t phi[NT][2], plo[NT][2];
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
                l[nt] *= alpha;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[nt][i] *= alpha;
                m[nt] = mn;
            }
            const float neg_m = -m[nt];
            float pr[16];
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                pr[i] = __builtin_amdgcn_exp2f(fmaf(x[i], scale, neg_m));
                sum += pr[i];
            }
            l[nt] += sum;
            // k-step h covers blocks 2h, 2h+1: this lane's 8 keys are
            // (block 2h: 4g..4g+3, block 2h+1: 4g..4g+3)
#pragma unroll
            for (int h = 0; h < 2; ++h) split_p8(pr + 8 * h, phi[nt][h], plo[nt][h]);
        }
        // O^T += V^T . P^T
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
                for (int nt = 0; nt < NT; ++nt) {
                    acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi[nt][h], acc[nt][mt], 0, 0, 0);
                    acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo[nt][h], acc[nt][mt], 0, 0, 0);
                }
            }
        }
        if (it + 1 < n_iter) sreg.store(ks[cur ^ 1], vs[cur ^ 1], t);
        __syncthreads();
    }

    bad = bad || !row_ok;
    const bool tok_ok = j0 + r < C;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float lt = l[nt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        if (!head_ok[nt] || !tok_ok) continue;
        const float inv = bad ? __builtin_nanf("") : vscale / lt;
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
