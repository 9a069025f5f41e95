// attn_fwd_kv_noalloc: the split-KV forward with its workspace taken from a
// static device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation).  Same kernels, same plan, same result as
// attn_fwd_kv.
//
// The array is a file-scope __device__ object: every device the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never passes the array's name to a kernel (on the host that name is only a
// stand-in, not a device address); the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and is
// what the kernels receive.  Nothing in the array must start at zero: every
// partial the merge reads is written by the split kernel of the same call.

#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_launch.h"

__device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];   // device address of `scratch` on each device, once taken

// Device address of the current device's copy of `scratch` (taken on the first
// call on that device).
int scratch_of_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return ATTN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                                   int Nq, int Nk, int d, float scale, int mask_kind, int window, int q_offset,
                                   int dtype, void* stream) {
    const unsigned long long need = attn_fwd_kv_workspace_size(B, H, Nq, Nk, d);
    if (need > (unsigned long long)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0) {
        const int st = scratch_of_current_device(&ws);
        if (st != ATTN_OK) return st;
    }
    return attn_fwd_kv(q, k, v, out, lse, B, H, Nq, Nk, d, scale, mask_kind, window, q_offset, dtype, ws,
                       need > 0 ? (unsigned long long)ATTN_NOALLOC_SCRATCH_BYTES : 0ull, stream);
}
