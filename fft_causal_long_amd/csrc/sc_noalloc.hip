// Scratch of the allocation-free entry point (sc_causal_conv_noalloc): a file-scope device
// array, so that the call needs no allocation at all.  Each GPU the library runs on holds
// its own copy from module load until the process ends.  In host code the array's name is
// only a host-side stand-in; the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and only that address is ever handed to a
// kernel or a copy.
#include <mutex>

#include "sc_internal.h"

namespace sc {

static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxStaticDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxStaticDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr, size_t* bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxStaticDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = STATIC_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace sc
