// lds_limit.h -- per-device opt-in to a large dynamic-LDS allocation for a
// kernel (host code; included by the kernel sources that launch with more
// than 64 KB of dynamic LDS).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace skg {

// Raises `kernel`'s dynamic-LDS limit to `bytes` on the current device.  A
// function attribute belongs to one device, so this runs once per device:
// `done` is the caller's per-kernel bitmask of devices already set (devices
// past 63 set it on every call).
inline hipError_t allow_dynamic_lds(const void *kernel, size_t bytes,
                                    std::atomic<unsigned long long> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

}  // namespace skg
