// floors.hip -- measurement helpers (empty kernel, read stream, copy).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"
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

// A flat read of `bytes` bytes: workgroup b reads the 32 KB [32768 b,
// 32768 (b + 1)) (the last one less), 256 threads with 8 loads of 16 bytes
// each, every load issued before any is consumed.
__global__ void __launch_bounds__(256)
    read_flat_kernel(const uint8_t *__restrict__ buf, size_t bytes, unsigned *__restrict__ sink) {
    const size_t base = (size_t)blockIdx.x * 32768;
    const size_t left = bytes - base;
    const skg::Rsrc r = skg::make_rsrc(buf + base, (unsigned)(left < 32768 ? left : 32768));
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = skg::load16<skg::kCacheStream>(r, (unsigned)(threadIdx.x + i * 256) * 16u);
    unsigned h = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) h ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (h == 0x9E3779B9u) sink[blockIdx.x] = h;
}

__global__ void __launch_bounds__(256)
    copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) dst[i] = src[i];
}

// The bf16 dot kernel's operand intake with no arithmetic: workgroup b
// loads the C rows of W and all M rows of x exactly as the dot kernel does
// (thread t takes the 16-byte vectors t, t + T, ... of each row; every load
// in flight before any is consumed; W streaming, x default), then folds the
// words with xor.  Its time is the floor of the dot kernel's loads alone.
template <int M, int C, int V>
__global__ void __launch_bounds__(skg::dot_max_threads(M, C, V, true))
    intake_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, int N, int K,
                  unsigned *__restrict__ sink) {
    const int T = blockDim.x;
    const int t = threadIdx.x;
    const int n0 = blockIdx.x * C;
    const int ncols = min(C, N - n0);
    const unsigned rowb = (unsigned)K * 2u;
    const skg::Rsrc wr = skg::make_rsrc(W + (size_t)n0 * K, (unsigned)ncols * rowb);
    const skg::Rsrc xr = skg::make_rsrc(x, (unsigned)M * rowb);
    const int K8 = K >> 3;
    u32x4 wv[C][V];
    u32x4 xv[M][V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int v = t + i * T;
        const unsigned off = v < K8 ? (unsigned)v * 16u : skg::kOOB;
#pragma unroll
        for (int c = 0; c < C; ++c)
            wv[c][i] = skg::load16<skg::kCacheStream>(wr, off + (unsigned)c * rowb);
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int v = t + i * T;
        const unsigned off = v < K8 ? (unsigned)v * 16u : skg::kOOB;
#pragma unroll
        for (int m = 0; m < M; ++m)
            xv[m][i] = skg::load16<skg::kCacheDefault>(xr, off + (unsigned)m * rowb);
    }
    unsigned h = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
        for (int c = 0; c < C; ++c) h ^= wv[c][i].x ^ wv[c][i].y ^ wv[c][i].z ^ wv[c][i].w;
#pragma unroll
        for (int m = 0; m < M; ++m) h ^= xv[m][i].x ^ xv[m][i].y ^ xv[m][i].z ^ xv[m][i].w;
    }
    if (h == 0x9E3779B9u) sink[blockIdx.x] = h;
}

typedef void (*IntakeFn)(const uint16_t *, const uint16_t *, int, int, unsigned *);

template <int M, int C, int V>
constexpr IntakeFn intake_entry() {
    if constexpr (skg::dot_regs(M, C, V, true) <= skg::kDotRegsMax)
        return &intake_kernel<M, C, V>;
    else
        return nullptr;
}

template <int M, int C>
IntakeFn intake_v(int V) {
    switch (V) {
    case 1: return intake_entry<M, C, 1>();
    case 2: return intake_entry<M, C, 2>();
    case 3: return intake_entry<M, C, 3>();
    case 4: return intake_entry<M, C, 4>();
    case 6: return intake_entry<M, C, 6>();
    case 7: return intake_entry<M, C, 7>();
    case 8: return intake_entry<M, C, 8>();
    case 12: return intake_entry<M, C, 12>();
    case 14: return intake_entry<M, C, 14>();
    case 16: return intake_entry<M, C, 16>();
    default: return nullptr;
    }
}

template <int M>
IntakeFn intake_c(int C, int V) {
    switch (C) {
    case 1: return intake_v<M, 1>(V);
    case 2: return intake_v<M, 2>(V);
    case 3: return intake_v<M, 3>(V);
    case 4: return intake_v<M, 4>(V);
    default: return nullptr;
    }
}

IntakeFn intake_pick(int M, int C, int V) {
    switch (M) {
    case 1: return intake_c<1>(C, V);
    case 2: return intake_c<2>(C, V);
    case 3: return intake_c<3>(C, V);
    case 4: return intake_c<4>(C, V);
    case 5: return intake_c<5>(C, V);
    case 6: return intake_c<6>(C, V);
    case 7: return intake_c<7>(C, V);
    case 8: return intake_c<8>(C, V);
    case 9: return intake_c<9>(C, V);
    case 10: return intake_c<10>(C, V);
    case 11: return intake_c<11>(C, V);
    case 12: return intake_c<12>(C, V);
    case 13: return intake_c<13>(C, V);
    case 14: return intake_c<14>(C, V);
    case 15: return intake_c<15>(C, V);
    case 16: return intake_c<16>(C, V);
    default: return nullptr;
    }
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

extern "C" int skinny_floor_read_flat(const void *buf, size_t bytes, unsigned *sink,
                                      hipStream_t stream) {
    if (!buf || !sink || bytes < 16 || bytes % 16 || (uintptr_t)buf % 16 ||
        bytes > ((size_t)1 << 40))
        return (int)hipErrorInvalidValue;
    const size_t grid = (bytes + 32767) / 32768;
    hipLaunchKernelGGL(read_flat_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t *)buf, bytes, sink);
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

extern "C" int skinny_floor_intake(const void *x, const void *W, int M, int N, int K, int cols,
                                   int threads, int vecs, unsigned *sink, hipStream_t stream) {
    if (!x || !W || !sink || M < 1 || M > 16 || N < 1 || K < 8 || K % 8 || threads < 64 ||
        threads > 1024 || threads % 64 || (uintptr_t)x % 16 || (uintptr_t)W % 16 ||
        (long)vecs * threads < K / 8 || (long)N * K * 2 > 0x7FFFFFFFL)
        return (int)hipErrorInvalidValue;
    IntakeFn f = intake_pick(M, cols, vecs);
    if (!f || threads > skg::dot_max_threads(M, cols, vecs, true)) return (int)hipErrorInvalidValue;
    const int grid = (N + cols - 1) / cols;
    hipLaunchKernelGGL(f, dim3(grid), dim3(threads), 0, stream, (const uint16_t *)x,
                       (const uint16_t *)W, N, K, sink);
    return (int)hipGetLastError();
}
