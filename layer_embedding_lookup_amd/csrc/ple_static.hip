// The library-owned scratch array behind ple_prefill_fused_noalloc: device
// memory for the fused prefill's intermediates (rows, kv, conv input) for
// callers that cannot allocate.  Every GPU the library runs on holds its own
// copy at its own address from the time the code object is loaded until the
// process ends.  The array's name is a host-side stand-in in host code: the
// device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is passed to kernels.
#include <mutex>

#include "ple_launch.h"

namespace ple {

static __device__ __align__(256) char scratch[PLE_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 256;
    static std::mutex mu;
    static void* addr[kMaxDevices];  // per device, set once
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace ple
