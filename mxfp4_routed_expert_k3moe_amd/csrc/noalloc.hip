// noalloc.hip -- the library's fixed device scratch for callers that cannot
// allocate (graph capture, serving loops that forbid hipMalloc).  One array of
// K3MOE_NOALLOC_SCRATCH_BYTES per device, held from module load to process end.
//
// The array's name is a host-side stand-in in host code, not a device address:
// its address on each device comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that pointer is handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "k3moe.h"
#include "launch.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[K3MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_ptr[kMaxDevices];
std::mutex g_mu;

}  // namespace

namespace k3moe {

hipError_t noalloc_scratch(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_mu);
        p = g_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            // the current device is `dev`: the address is that device's copy
            err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (err != hipSuccess) return err;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace k3moe
