// pi_occupancy.hpp -- how many workgroups of a kernel the current device keeps resident at once,
// asked of the HIP runtime once per (device, kernel, block size, dynamic LDS) and remembered, so
// that a launch pays the query only the first time.  The persistent kernels size their grids from
// it: their workgroups wait on each other, so every one of them must be resident.
#pragma once

#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>

namespace pik {

// *cus = compute units of the current device, *per_cu = resident workgroups of `kern` per CU with
// `threads` threads and `lds` bytes of dynamic LDS.  0 on success, 1 if a query failed or the
// kernel cannot be resident at all.
inline int resident_slots(const void *kern, int threads, size_t lds, int *cus, int *per_cu) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void *, int, size_t>, std::pair<int, int>> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    const auto key = std::make_tuple(dev, kern, threads, lds);
    {
        std::lock_guard<std::mutex> g(mu);
        auto it = cache.find(key);
        if (it != cache.end()) {
            *cus = it->second.first;
            *per_cu = it->second.second;
            return 0;
        }
    }
    int c = 0, p = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&p, kern, threads, lds) != hipSuccess || p < 1 || c < 1) return 1;
    {
        std::lock_guard<std::mutex> g(mu);
        cache[key] = std::make_pair(c, p);
    }
    *cus = c;
    *per_cu = p;
    return 0;
}

}  // namespace pik
