// lightning_index_topk_noalloc: the indexer call of include/v4attn.h without a
// caller-provided workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation). Its scratch is one file-scope device array per GPU, holding
// what the workspace would: per (query, chunk) candidate counts, bounds and
// regions. It is zero-filled once per device, on the first call's stream.
//
// Host code never passes the array's name to a kernel: that name is a
// host-side stand-in. The device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only it is used.
//
// Every call on a GPU shares that GPU's array and leaves it initialised, as
// the other calls leave a workspace: calls that overlap in time on one GPU
// (different streams, or different host threads) race on it.

#include <mutex>

#include "common.hpp"

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)V4A_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_mu;
void *g_scratch[MAX_DEVICES];  // device address of `scratch` on each device (null until set up)

// The scratch's device address on the current device, set up (address taken,
// memory zero-filled on `stream`) on the first call there.
int scratch_ptr(hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return v4a::report(V4A_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES)
        return v4a::report(V4A_EINVAL, "device %d is beyond the %d devices the static scratch covers", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return v4a::report(V4A_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        const int r = v4a::fill_zero(p, SCRATCH_BYTES, stream);
        if (r) return r;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return V4A_OK;
}

}  // namespace

extern "C" int lightning_index_topk_noalloc(const v4a_index_args *a, v4a_stream stream) {
    size_t need = 0;
    int r = v4a::index_workspace(a, &need);
    if (r) return r;
    if (need > SCRATCH_BYTES)
        return v4a::report(V4A_EWORKSPACE,
                           "this call needs %zu bytes of scratch; the static scratch holds %zu "
                           "(use lightning_index_topk with a workspace)",
                           need, SCRATCH_BYTES);
    void *ptr = nullptr;
    if ((r = scratch_ptr((hipStream_t)stream, &ptr))) return r;
    return v4a::index_call(a, ptr, SCRATCH_BYTES, (hipStream_t)stream);
}
