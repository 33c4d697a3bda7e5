// Internal helpers shared by the library's translation units (not installed).
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "pagedkv.h"

namespace pkv {

// Record a message for pkv_last_error() and return the status unchanged.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Argument checks shared by the device entry points (PKV_OK or an error).
int check_cache(const pkv_cache* c);
int check_attn(const pkv_cache* c, const pkv_attn_args* a);

// Wavefronts per kv head for a decode launch.
int32_t decode_parts(const pkv_cache* c, const pkv_attn_args* a);

// Workspace the decode part of a call needs (bytes; 0 when it has no rows).
size_t decode_workspace_bytes(const pkv_cache* c, const pkv_attn_args* a, int32_t rows);

// Shared-prefix pass of a decode call (a->shared_prefix_blocks > 0): every
// row's state over each of prefix_parts() ranges of the prefix into states
// [parts][rows][hq][128 + 4] (prefill.hip).
int prefix_parts(const pkv_cache* c, const pkv_attn_args* a, int32_t rows);
// Workspace of a prefill call's chunk rows (their key-range states; 0 when the
// tiles are not split), placed after the decode rows' part, 256-byte aligned.
size_t prefill_workspace_bytes(const pkv_cache* c, const pkv_attn_args* a);

}  // namespace pkv
