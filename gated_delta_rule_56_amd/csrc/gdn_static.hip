// Device scratch of gdn_prefill_static: one array of GDN_STATIC_SCRATCH_BYTES on every GPU the
// library's code object is loaded on, held until the process ends, so that the call needs no
// allocation of its own.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

// Host code must not use this name as an address: on the host it is a stand-in, and each GPU
// holds its own copy at its own address. static_scratch() gives the current GPU's.
static __device__ __align__(256) unsigned char scratch[GDN_STATIC_SCRATCH_BYTES];

namespace gdn {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up
}  // namespace

hipError_t static_scratch(void **out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));  // with device dev current
        if (err != hipSuccess) return err;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gdn
