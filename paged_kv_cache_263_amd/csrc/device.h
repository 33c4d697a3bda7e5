// Device-side helpers shared by the library's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedkv.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kD = PKV_HEAD_DIM;       // head dimension
constexpr int kBS = PKV_BLOCK_SIZE;    // tokens per block
constexpr int kTile = kBS * kD;        // elements of one (block, kv head) tile
constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
__device__ __forceinline__ T ld(const void* p) {
    return *static_cast<const T*>(p);
}
// A load marked non-temporal (the `nt` cache policy): data read once per
// call, such as the K/V tiles a decode step streams, so the caches treat it
// as streaming rather than keeping it at the expense of other lines.
template <typename T>
__device__ __forceinline__ T ld_stream(const void* p) {
    return __builtin_nontemporal_load(static_cast<const T*>(p));
}
template <typename T>
__device__ __forceinline__ void st(void* p, T v) {
    *static_cast<T*>(p) = v;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Four fp8 E4M3 bytes -> four bf16 (exact).  An E4M3 value has at most four
// significant bits and an exponent inside bf16's range, so it is a bf16 value.
// gfx950 converts two codes straight to a bf16 pair (v_cvt_scalef32_pk_bf16_fp8
// with scale 1.0): one instruction per pair.  Checked bit for bit over all
// 65536 code pairs against converting to fp32 (exact) and keeping the high
// halves, which took two instructions per pair.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16x4(uint32_t w) {
    return u32x2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

// Four int8 codes -> four bf16 (exact: every integer in -127..127 has at
// most 7 significant bits).  Each byte converts sign-extended to fp32 (exact,
// low 16 bits zero) and the two high halves of each pair are packed with one
// v_perm_b32 (bytes 2, 3 of the first value, then of the second).
__device__ __forceinline__ u32x2_t int8x4_to_bf16x4(uint32_t w) {
    const float f0 = static_cast<float>(static_cast<int8_t>(w & 0xFFu));
    const float f1 = static_cast<float>(static_cast<int8_t>((w >> 8) & 0xFFu));
    const float f2 = static_cast<float>(static_cast<int8_t>((w >> 16) & 0xFFu));
    const float f3 = static_cast<float>(static_cast<int8_t>(w >> 24));
    return u32x2_t{__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u),
                   __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u)};
}

// fp32 -> int8 code (as the low byte): nearest integer, ties to even,
// clamped to -127..127.
__device__ __forceinline__ uint32_t int8_code_rne(float x) {
    const float r = fminf(fmaxf(__builtin_rintf(x), -127.0f), 127.0f);
    return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu;
}

// One-byte cache dtypes (codes times a per-(layer, kv head) fp32 scale).
constexpr bool is_byte_dtype(int kv) { return kv == PKV_FP8_E4M3 || kv == PKV_INT8; }

// Four one-byte codes of the cache's dtype -> four bf16.
template <int KV>
__device__ __forceinline__ u32x2_t byte4_to_bf16x4(uint32_t w) {
    if constexpr (KV == PKV_INT8) return int8x4_to_bf16x4(w);
    else return fp8x4_to_bf16x4(w);
}

// Element offset of (token, d) inside a bf16 K tile (16 tokens x 128 d,
// 4 KiB): 16-byte pieces of 8 consecutive d, ordered by d / 8, then token.
// Lane 16 g + r of the decode kernel feeds matrix step ks with token r, d
// 32 ks + 8 g .. +7 - piece 64 ks + 16 g + r - so each of its four load
// instructions reads 1 KiB of the tile contiguously; the prefill kernel's
// thread t stages piece t.
__device__ __forceinline__ int bf16_k_offset(int tok, int d) { return (d >> 3) * 128 + tok * 8 + (d & 7); }

// Element offset of (d row, token) inside a bf16 V tile (128 d x 16 tokens):
// with d = 16 n + r, n = 2 m + h and token = 4 g + i, at m * 512 +
// (16 g + r) * 8 + h * 4 + i.  Decode lane 16 g + r feeds the matrix cores
// tokens 4g..4g+3 of d rows 16 n + r, n = 0..7; piece m of that lane holds
// n = 2 m and 2 m + 1, so its four loads read 1 KiB contiguously each.
__device__ __forceinline__ int bf16_v_offset(int d, int tok) {
    return (d >> 5) * 512 + ((tok >> 2) * 16 + (d & 15)) * 8 + ((d >> 4) & 1) * 4 + (tok & 3);
}

// Byte offset of (d row, token) inside a one-byte (fp8 or int8) V tile
// (2 KiB): tokens in groups of 4, then d / 64, then d % 16, then (d / 16) % 4,
// then the token within its group.  Lane (r, g) of the decode kernel then
// finds the 8 words it feeds to the matrix cores - tokens 4g..4g+3 of d rows
// 16 n + r, n = 0..7 - as two 16-byte pieces at g * 512 + s * 256 + r * 16
// (words n = 4 s .. 4 s + 3), so each of its two load instructions reads
// whole 256-byte runs of the tile.
__device__ __forceinline__ int byte_v_offset(int d, int tok) {
    return (tok >> 2) * 512 + (d >> 6) * 256 + (d & 15) * 16 + ((d >> 4) & 3) * 4 + (tok & 3);
}

// fp32 -> E4M3 code: nearest, ties to even mantissa, |x| >= 448 saturates to
// +-448, sign kept (so -0 and negative underflow give 0x80).  Written from
// the format: bias 7, subnormals m/8 * 2^-6, largest finite 1.75 * 2^8.
__device__ __forceinline__ uint32_t e4m3_code_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    const float af = __uint_as_float(a);
    if (!(af < 448.0f)) return sign | 0x7Eu;
    if (af < 0.015625f) {  // below 2^-6: subnormal codes 0..8, code = rint(|x| * 2^9)
        return sign | static_cast<uint32_t>(__builtin_rintf(af * 512.0f));
    }
    int e = static_cast<int>(a >> 23) - 127;  // -6 .. 8
    uint32_t keep = (a >> 20) & 7u;
    const uint32_t rest = a & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep += 1;
    if (keep == 8) {
        keep = 0;
        e += 1;
    }
    return sign | (static_cast<uint32_t>(e + 7) << 3) | keep;
}

}  // namespace pkv
