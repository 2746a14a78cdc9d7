// Library-owned scratch memory for gdn_step_frame_noalloc: a file-scope device array that the
// loader places on every GPU the library runs on, so that a caller that cannot allocate device
// memory (HIP graph capture, tight serving loops, hosts that forbid hipMalloc) can still run a
// streaming step. Every call on one GPU shares that GPU's array.
//
// In host code `scratch` names a host-side stand-in, not a device address: the address of the
// current device's copy comes from hipGetSymbolAddress, looked up once per device (with that
// device current) on the first call there and kept for the life of the process.
#include <mutex>

#include "gdn_internal.h"

namespace gdn {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace gdn
