// floors.hip -- measurement helpers (empty kernel, read stream, copy).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "skinny_floors.h"

namespace {

using skg::u32x4;

__global__ void empty_kernel() {}

constexpr int kReadMaxVecs = 8;

__global__ void __launch_bounds__(1024)
    read_kernel(const uint8_t *__restrict__ buf, int row_bytes, unsigned *__restrict__ sink) {
    const skg::Rsrc r = skg::make_rsrc(buf + (size_t)blockIdx.x * row_bytes, (unsigned)row_bytes);
    const int T = blockDim.x;
    const int nvec = row_bytes >> 4;
    u32x4 v[kReadMaxVecs];
#pragma unroll
    for (int i = 0; i < kReadMaxVecs; ++i) {
        const int idx = threadIdx.x + i * T;
        v[i] = skg::load16<skg::kCacheStream>(r, idx < nvec ? (unsigned)idx * 16u : skg::kOOB);
    }
    unsigned h = 0;
#pragma unroll
    for (int i = 0; i < kReadMaxVecs; ++i) h ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (h == 0x9E3779B9u) sink[blockIdx.x] = h;
}

__global__ void __launch_bounds__(256)
    copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" int skinny_floor_empty(int grid, int threads, hipStream_t stream) {
    if (grid < 1 || threads < 1 || threads > 1024) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(threads), 0, stream);
    return (int)hipGetLastError();
}

extern "C" int skinny_floor_read(const void *buf, int rows, int row_bytes, int threads,
                                 unsigned *sink, hipStream_t stream) {
    if (!buf || !sink || rows < 1 || row_bytes < 16 || row_bytes % 16 || threads < 64 ||
        threads > 1024 || threads % 64 || row_bytes > 16 * kReadMaxVecs * threads ||
        (uintptr_t)buf % 16)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(rows), dim3(threads), 0, stream, (const uint8_t *)buf,
                       row_bytes, sink);
    return (int)hipGetLastError();
}

extern "C" int skinny_floor_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    if (!src || !dst || bytes % 16 || (uintptr_t)src % 16 || (uintptr_t)dst % 16)
        return (int)hipErrorInvalidValue;
    const size_t n = bytes / 16;
    if (n == 0) return 0;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const u32x4 *)src, (u32x4 *)dst, n);
    return (int)hipGetLastError();
}
