// noalloc.hip -- the scratch array behind mnb_gemm_accuracy4_noalloc, the
// entry point for callers that cannot allocate device memory.
//
// The array is a file-scope device variable: every device that loads the
// library holds its own copy until the process ends.  In host code the name
// `scratch` denotes a host-side stand-in, never the device memory, so it is
// never passed to a kernel or a copy: the device address comes from
// hipGetSymbolAddress, called once per device with that device current, and
// is cached per device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/mnb.h"
#include "mnb_internal.hpp"

namespace mnb {

namespace {

static __device__ __align__(256) unsigned char scratch[MNB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_addr[kMaxDevices];
std::mutex g_mu;

}  // namespace

hipError_t noalloc_scratch(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_mu);
        p = g_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return e;
            }
            if (!p) return hipErrorInvalidSymbol;
            g_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace mnb
