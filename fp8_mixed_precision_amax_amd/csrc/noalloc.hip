// Device-resident scratch of the linear forward that allocates nothing
// (fp8_linear_fwd_noalloc): for callers that cannot allocate device memory,
// such as code under HIP graph capture or tight serving loops.
//
// The array below lives in the code object, so every GPU the library is
// loaded on holds its own copy for the life of the process.  In host code
// its name is only a host-side stand-in: the device address of each GPU's
// copy comes from hipGetSymbolAddress, taken once per device (with that
// device current) and kept; host code passes that address to kernels and
// never the array's name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace fp8k {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

}  // namespace fp8k
