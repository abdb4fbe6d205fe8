// Built-in scratch for kda_prefill_noalloc: the prefill workspace of callers
// that cannot allocate device memory.  One array per device, in this code
// object's global memory, reserved when the code object is loaded on that
// device and held until the process ends.
//
// `scratch` below is a device variable: in host code its name denotes a
// host-side stand-in, not the device address.  The device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that pointer is ever handed to kernels.

#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
