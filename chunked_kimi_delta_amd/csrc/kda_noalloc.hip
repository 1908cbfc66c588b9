// kda_noalloc.hip -- kda_fwd_noalloc: the forward with its workspace in a static device array,
// for callers that cannot allocate device memory or pass a workspace (declared in
// include/kda_fwd.h).
//
// The array `scratch` is a file-scope __device__ variable: the runtime places one copy on every
// device the library's code object is loaded on, and it lives until the process ends. Its name
// in host code is only a host-side stand-in, so the device address of each copy is looked up
// once per device with hipGetSymbolAddress (with that device current) and that address is what
// the launches get.
#include <atomic>
#include <mutex>

#include "kda_fwd.h"
#include "kda_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_WORKSPACE_BYTES];

constexpr int MAX_DEV = 64;
std::atomic<void *> scratch_ptr[MAX_DEV];   // device address of `scratch`, per device ordinal
std::mutex scratch_mu;

// Device address of this device's `scratch`, or nullptr when the lookup fails.
void *device_scratch(int dev)
{
    if (dev < MAX_DEV) {
        void *p = scratch_ptr[dev].load(std::memory_order_acquire);
        if (p) return p;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    void *p = dev < MAX_DEV ? scratch_ptr[dev].load(std::memory_order_relaxed) : nullptr;
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();      // leave no sticky error for the caller's next call
        return nullptr;
    }
    if (dev < MAX_DEV) scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" kda_status kda_fwd_noalloc(const kda_fwd_args *args, void *stream)
{
    if (!args) return KDA_ERR_INVALID_ARG;
    // kda_fwd_workspace_bytes is 0 both for shapes that need no workspace and for arguments
    // kda_fwd rejects; kda_fwd below returns the rejection's own status
    if (kda_fwd_workspace_bytes(args) > KDA_NOALLOC_WORKSPACE_BYTES)
        return KDA_ERR_NOALLOC_TOO_LARGE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KDA_ERR_HIP;
    void *ws = device_scratch(dev);
    if (!ws) return KDA_ERR_HIP;
    return kda_fwd(args, ws, KDA_NOALLOC_WORKSPACE_BYTES, stream);
}
