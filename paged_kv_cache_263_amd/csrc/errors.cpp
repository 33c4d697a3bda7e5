// Status strings and the per-thread last-error message of the C ABI.
#include <cstdio>

#include "internal.h"

namespace {
thread_local char g_last[512] = "";
}

namespace pkv {

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last, sizeof(g_last), fmt, ap);
    va_end(ap);
    return status;
}

}  // namespace pkv

extern "C" {

const char* pkv_strerror(int status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_INVALID: return "invalid argument";
        case PKV_ERR_OOM: return "out of KV blocks";
        case PKV_ERR_STATE: return "bad state (double free, refcount underflow or freed sequence)";
        case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
        case PKV_ERR_HIP: return "HIP runtime error";
        case PKV_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

const char* pkv_last_error(void) { return g_last; }

int pkv_version(void) { return 1; }

}  // extern "C"
