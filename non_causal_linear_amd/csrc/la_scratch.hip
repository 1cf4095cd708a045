// Device scratch of la_fwd_noalloc, the entry point for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc). The forward's split partials go into a static device
// array instead of a caller workspace. Each GPU the library runs on holds its
// own copy of the array, from the moment the code object is loaded on that
// device until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: host
// code uses only the address hipGetSymbolAddress returns for the current
// device, kept per device below.

#include <hip/hip_runtime.h>

#include <mutex>

#include "la_internal.h"

namespace la {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t scratch_device_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace la
