// Fixed device scratch for the entry point that allocates nothing (ssd_fwd_noalloc).
//
// Callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc) still need the forward's
// workspace: the fp64 chunk cumsums and the [b, n, h, p, r] chunk states.  It
// lives in one file-scope device array, which every GPU the library runs on
// holds (its own copy, at its own address) until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device address
// is taken once per device with hipGetSymbolAddress (with that device current)
// and cached; host code uses that pointer, never the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd.h"
#include "ssd_launch.hpp"

namespace ssd {

static_assert(SSD_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace ssd
