// Paged decode for callers that cannot allocate device memory: code under HIP
// graph capture, serving loops and harnesses that forbid hipMalloc.  It is
// paged_attn_decode with the workspace (row plan, partial results of rows cut
// between wavefronts, shared-prefix states) taken from a fixed array in device
// memory instead of a caller's buffer.  The kernels are the same ones.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code its name is only a stand-in for the symbol, not a device address, so
// host code never passes it to a kernel or a copy: on the first call on a
// device, with that device current, hipGetSymbolAddress gives the device
// address, which is kept per device and passed to the kernels as their
// workspace.
//
// Every call on one GPU shares that GPU's array: calls that overlap on one GPU
// (enqueued on different streams with no ordering between them) race on it.
// Calls on one stream, or ordered by events, are safe.  Nothing in the
// workspace needs to start at zero: every word the kernels read was written
// earlier in the same call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"

// The workspace array (see above).  Host code names it only in
// hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace pkv {

int launch_decode(const pkv_cache* c, const pkv_attn_args* a, int32_t rows, int32_t max_kv_len, const void* q,
                  void* out, const int32_t* table, const int32_t* kv_lens, void* workspace, size_t ws_bytes,
                  hipStream_t stream);

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES);

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's copy of the array (looked up once per
// device, with that device current).
int scratch_address(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (stream) {
        hipDevice_t sdev = 0;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev) return fail(PKV_ERR_INVALID, "the stream belongs to device %d, the current device is %d", sdev, dev);
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attn_decode_noalloc(const pkv_cache* c, const pkv_attn_args* a, void* stream) {
    int st = pkv::check_attn(c, a);
    if (st) return st;
    if (a->workspace || a->workspace_bytes)
        return pkv::fail(PKV_ERR_INVALID, "paged_attn_decode_noalloc takes no workspace (leave it NULL and 0)");
    const size_t need = pkv::decode_workspace_bytes(c, a, a->num_seqs);
    if (need > pkv::kScratchBytes)
        return pkv::fail(PKV_ERR_WORKSPACE, "this call needs %zu bytes of workspace, above the fixed %zu of the "
                         "no-allocation entry point (fewer rows or decode_parts, or use paged_attn_decode)",
                         need, pkv::kScratchBytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ptr = nullptr;
    if (a->num_seqs > 0) {
        st = pkv::scratch_address(s, &ptr);
        if (st) return st;
    }
    return pkv::launch_decode(c, a, a->num_seqs, a->max_kv_len, a->q, a->out, a->block_table, a->kv_lens, ptr,
                              pkv::kScratchBytes, s);
}
