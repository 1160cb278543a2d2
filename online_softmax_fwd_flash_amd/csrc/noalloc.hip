// Fixed device scratch for flash_attn_bwd_noalloc: the backward's Dvec workspace (one float per
// query row and head) lives in a file-scope device array instead of memory allocated per call,
// for callers that cannot allocate.  Each device that runs the library holds its own copy of
// the array until the process ends.  Host code never uses the array's name as an address:
// the device address is looked up once per device (with that device current) and kept.
#include <atomic>

#include "kernels.h"

namespace fa {

namespace {

static_assert(kNoAllocDvecFloats % 64 == 0, "scratch size must keep 256-byte alignment");

__device__ __align__(256) float scratch[kNoAllocDvecFloats];

std::atomic<float*> g_scratch_ptr[kMaxDeviceSlots];

}  // namespace

hipError_t noalloc_dvec(size_t floats, float** out) {
    *out = nullptr;
    if (floats > (size_t)kNoAllocDvecFloats) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDeviceSlots) return hipErrorInvalidDevice;
    float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (addr == nullptr) return hipErrorInvalidSymbol;
        p = static_cast<float*>(addr);
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace fa
