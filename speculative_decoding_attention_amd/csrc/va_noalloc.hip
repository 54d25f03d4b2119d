// va_noalloc.hip -- the device array behind verify_attn_run_noalloc.
//
// verify_attn_run keeps the prefix ranges' partial outputs and log-sum-exps
// in a workspace the caller passes.  verify_attn_run_noalloc, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation), keeps them in `scratch` below: a
// file-scope device array of kNoAllocScratchBytes that every GPU the library
// runs on holds until the process ends.
//
// In host code the name `scratch` is a host-side stand-in, not a device
// address.  The address each device's copy lives at is taken once per device
// with hipGetSymbolAddress (that device current) and kept; host code passes
// only that address on, never the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "va_internal.h"

namespace va {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int noalloc_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_error("hipGetDevice: %s", hipGetErrorString(e));
        return VA_ERR_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("device %d beyond the %d devices the scratch table tracks", dev, kMaxDevices);
        return VA_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_error("hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
            return VA_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return VA_OK;
}

}  // namespace va
