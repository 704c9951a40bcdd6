// launch_cache.cpp -- per-device launch facts cached once per process (see rtq_internal.h).
#include <hip/hip_runtime.h>

#include <mutex>
#include <tuple>
#include <map>

#include "rtq_internal.h"

namespace rtq {

namespace {
std::mutex g_mu;
std::map<int, int> g_cus;
std::map<std::tuple<int, const void*, int, size_t>, int> g_occ;
}  // namespace

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_cus.find(dev);
    if (it != g_cus.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    g_cus[dev] = cus;
    return cus;
}

hipError_t kernel_blocks_per_cu(const void* kernel, int threads, size_t lds, int* per_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const auto key = std::make_tuple(dev, kernel, threads, lds);
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_occ.find(key);
    if (it != g_occ.end()) {
        *per_cu = it->second;
        return hipSuccess;
    }
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    g_occ[key] = n;
    *per_cu = n;
    return hipSuccess;
}

}  // namespace rtq
