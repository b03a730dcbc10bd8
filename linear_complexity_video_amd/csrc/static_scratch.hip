// Library-held scratch for the entry point that allocates nothing
// (mate_bissd_scan_noalloc): one fixed array in device memory per GPU, loaded
// with the code object and kept until the process ends.
//
// In host code the array's name is only a host-side stand-in, not a device
// address, so the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "mate.h"

namespace mate {

namespace {

static __device__ __align__(256) unsigned char scratch[MATE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

} // namespace

hipError_t static_scratch(void **out)
{
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

} // namespace mate
