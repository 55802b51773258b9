// Static device scratch for the allocation-free backward entry point
// (fa_bwd_noalloc): the per-row D values that fa_bwd keeps in the caller's
// workspace live here instead, so that the call allocates nothing.
//
// `scratch` is a file-scope device array; every GPU the library runs on
// holds its own copy (16 MiB) from the first use until the process ends. In
// host code the name `scratch` is only a host-side stand-in for the symbol,
// so its device address is looked up with hipGetSymbolAddress once per
// device, with that device current, and only that address is ever handed to
// kernels. Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_kernels.h"

static __device__ __align__(256) float scratch[fa::kBwdScratchRows];

namespace fa {
namespace {

constexpr int kMaxDevices = 256;
std::mutex g_mu;
float* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t bwd_scratch(float** out)
{
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_addr[dev] = static_cast<float*>(p);
    }
    *out = g_addr[dev];
    return hipSuccess;
}

}  // namespace fa
