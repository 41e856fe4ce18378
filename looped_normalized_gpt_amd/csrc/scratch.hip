// scratch.hip -- the device scratch of dory_forward_chunk_noalloc: a static
// array, so that callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) can run a forward.
//
// One copy of the array lives on every GPU the library runs on, from the first
// use until the process ends.  In host code the array's name is only a
// host-side stand-in: its device address on the current GPU is looked up once
// per device (at the first dory_create on that device) and kept here; kernels
// get that address, never the name.  Every no-allocation call on a GPU shares
// its array: calls that overlap on one GPU (any handle, any stream) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace dk {

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_addr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *ptr = g_addr[dev];
    return hipSuccess;
}

}  // namespace dk
