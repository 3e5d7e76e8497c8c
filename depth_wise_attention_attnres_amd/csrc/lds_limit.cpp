// lds_limit.cpp -- dynamic-LDS limits of the kernels that stage data in LDS,
// and the resident-workgroup counts that size persistent grids.
//
// A kernel's dynamic-LDS limit is an attribute of the function, shared by the
// whole process.  Setting it per call to what that call needs would let one
// host thread lower it between another thread's set and launch, so the limit
// is raised once per (kernel, device), to the device maximum, and never
// lowered; each call only checks that its own size fits.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <set>
#include <tuple>
#include <utility>

#include "launch.hpp"

namespace attnres {

namespace {

std::mutex g_mu;
std::set<std::pair<const void*, int>> g_raised;  // (kernel, device) pairs already raised

}  // namespace

int device_max_lds() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return 0;
    return v;
}

hipError_t prepare_dynamic_lds(const void* kernel, size_t bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int max_lds = 0;
    e = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    if (bytes > (size_t)max_lds) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_raised.count({kernel, dev}) != 0) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (e == hipSuccess) g_raised.insert({kernel, dev});
    return e;
}

// A persistent grid holds as many workgroups as the device runs at once; the
// count depends only on (kernel, device, threads, LDS), so it is queried once
// and cached under a lock (read-only afterwards).
hipError_t resident_workgroups(const void* kernel, int threads, size_t lds, int64_t* slots) {
    static std::mutex mu;
    static std::map<std::tuple<const void*, int, int, size_t>, int64_t> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const auto key = std::make_tuple(kernel, dev, threads, lds);
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto it = cache.find(key);
        if (it != cache.end()) {
            *slots = it->second;
            return hipSuccess;
        }
    }
    int ncu = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds)) != hipSuccess) return e;
    *slots = (int64_t)(ncu > 0 ? ncu : 1) * (per_cu > 0 ? per_cu : 1);
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = *slots;
    return hipSuccess;
}

}  // namespace attnres
