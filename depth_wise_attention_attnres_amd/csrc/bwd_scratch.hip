// bwd_scratch.hip -- the backward's workspace held in a static device array,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code the
// name is only a stand-in, never a device address, so the address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// that pointer is what the kernels receive.  The backward's kernels overwrite
// every workspace region they read, so nothing needs clearing between calls;
// calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace attnres {

namespace {

static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t bwd_scratch(void** ptr) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = p;
    });
    if (g_err[dev] != hipSuccess) return g_err[dev];
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace attnres
