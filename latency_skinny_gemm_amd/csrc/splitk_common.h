// splitk_common.h -- the ordered cross-workgroup reduction shared by the
// split-K kernels (device code; included by the kernel sources only).
#pragma once

#include "device_common.h"
#include "internal.h"

namespace skg {

// Grid position of a tiled workgroup b: row block mb (M > 128 only), K chunk
// s and column group j, in a grid of MB * G workgroups (G = S * column
// groups).  Where G is a multiple of 8 the MB row blocks of one (s, j) take
// workgroup ids 8 apart, so they run on one XCD (workgroup i runs on XCD
// i % 8) and that XCD's L2 fetches their shared W tile once; otherwise mb
// is fastest.  s is fastest among the (s, j) pairs in both cases.
struct TiledPos {
    int mb, s, j;
};
__device__ __forceinline__ TiledPos tiled_position(int b, int MB, int S, int G) {
    int mb, sj;
    if (MB > 1 && G % 8 == 0) {
        const int q = b / (8 * MB), r = b % (8 * MB);
        mb = r / 8;
        sj = q * 8 + r % 8;
    } else {
        mb = b % MB;
        sj = b / MB;
    }
    return TiledPos{mb, sj % S, sj / S};
}

// A split's fp32 partial ws[s][m][n].  With the last-arriver reduction
// (coherent) each store is an agent-scope relaxed atomic store, which
// writes through to the device's coherence point (global_store ... sc1):
// once it has completed, a workgroup on any XCD reads it with agent-scope
// loads, and no cache of the device has to be written back or invalidated.
// For the second-kernel reduction, which reads after a kernel boundary,
// plain stores.
__device__ __forceinline__ void put_partial(float *ws, size_t i, float v, bool coherent) {
    if (coherent)
        __hip_atomic_store(ws + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        ws[i] = v;
}

// The workspace ws[S][M][N] seen through one buffer resource, for 16-byte
// coherent (sc1) accesses: usable when N % 4 == 0 (16-byte aligned rows)
// and the S*M*N floats span less than 2^31 bytes (every byte offset is a
// valid 32-bit buffer offset below kOOB).
struct PartialsVec {
    Rsrc r;
    bool ok;
};
__device__ __forceinline__ PartialsVec partials_vec(float *ws, int M, int N, int S) {
    const unsigned long long bytes = (unsigned long long)S * (unsigned)M * (unsigned)N * 4ull;
    const bool ok = (N & 3) == 0 && bytes < 0x80000000ull;
    return PartialsVec{make_rsrc(ws, ok ? (unsigned)bytes : 0u), ok};
}

// Four consecutive partials (ws + i 16-byte aligned).  Coherent: one
// 16-byte sc1 store where the buffer view covers the workspace, else four
// dword atomic stores (the same coherence per dword).
__device__ __forceinline__ void put_partial4(float *ws, size_t i, f32x4 v, bool coherent,
                                             const PartialsVec &pv) {
    if (coherent && pv.ok) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), pv.r,
                                               (unsigned)(i * 4u), 0, kCacheCoherent);
    } else if (coherent) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __hip_atomic_store(ws + i + q, v[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *reinterpret_cast<f32x4 *>(ws + i) = v;
    }
}

// Called by every thread of a workgroup that has just written its fp32
// partial for the columns [col0, col0 + ncols) of tile j with
// put_partial(..., coherent = true).  Every wave waits until its partial
// stores have completed at device scope, then a barrier, then thread 0
// counts the workgroup in with one agent-scope relaxed atomic add on the
// tile's ticket.  The workgroup that counts last has seen every other
// workgroup's add, each made after that workgroup's stores completed, so
// its agent-scope loads of the partials return the stored values.  No
// fence writes back or invalidates an L2: the ordering comes from the
// explicit wait, the barrier and the atomic, all at device scope.  That
// workgroup sums the S partials in ascending s, applies the FP8 per-tensor
// scale product `scale` when `scaled` (once; the caller computes it),
// adds the bias and rounds once; it
// re-arms the ticket (the next kernel on the stream sees the zero after
// the kernel boundary).  No workgroup waits on another.
// E and G size the batch of 16-byte partial loads each thread keeps in
// flight (E * G loads, 4 * E * (G + 1) VGPRs): the kernels launched with up
// to 1024 threads take a smaller batch than the 256-thread tiled kernels.
template <int E = 8, int G = 4>
__device__ __forceinline__ void last_arriver_reduce(float *__restrict__ ws,
                                                    unsigned *__restrict__ tickets,
                                                    const uint16_t *__restrict__ bias,
                                                    void *__restrict__ out, int out_f32, int M, int N,
                                                    int S, int j, int col0, int ncols,
                                                    unsigned *is_last, bool scaled = false,
                                                    float scale = 1.0f) {
    wait_all_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(&tickets[j], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *is_last = (prev == (unsigned)S - 1u) ? 1u : 0u;
        if (*is_last)  // every partial of tile j has arrived: rearm for the next call
            __hip_atomic_store(&tickets[j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!*is_last) return;
    const PartialsVec pv = partials_vec(ws, M, N, S);
    const Rsrc br = bias_rsrc(bias, N);
    if (pv.ok && ((col0 | ncols) & 3) == 0) {
        // Four columns per item, 16-byte sc1 loads: each thread puts E items
        // x G splits of loads in flight before adding any of them, so the
        // tile costs about ceil(items / (E * threads)) * ceil(S / G) memory
        // latencies.  Each column still adds its S partials in ascending s
        // from 0.0f: the same bits as the loop below and the second kernel.
        const int C4 = ncols >> 2, items = M * C4;
        const unsigned plane = (unsigned)M * (unsigned)N * 4u;  // bytes per split
        for (int e0 = threadIdx.x; e0 < items; e0 += E * (int)blockDim.x) {
            unsigned off[E];
#pragma unroll
            for (int q = 0; q < E; ++q) {
                const int e = e0 + q * (int)blockDim.x;
                const int m = e / C4;
                off[q] = e < items ? ((unsigned)m * (unsigned)N + (unsigned)(col0 + 4 * (e - m * C4))) * 4u
                                   : kOOB;
            }
            // the items' bias values go out ahead of their partials
            unsigned bb[E][4];
#pragma unroll
            for (int q = 0; q < E; ++q) {
                const int e = e0 + q * (int)blockDim.x;
                const int m = e / C4;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    bb[q][k] = load_bias_bits(br, col0 + 4 * (e - m * C4) + k, e < items);
            }
            f32x4 acc[E];
#pragma unroll
            for (int q = 0; q < E; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < S; s0 += G) {
                f32x4 t[E][G];
#pragma unroll
                for (int q = 0; q < E; ++q)
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        const bool live = off[q] != kOOB && s0 + i < S;
                        t[q][i] = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       pv.r, live ? off[q] + (unsigned)(s0 + i) * plane : kOOB, 0,
                                       kCacheCoherent));
                    }
#pragma unroll
                for (int q = 0; q < E; ++q)
#pragma unroll
                    for (int i = 0; i < G; ++i)
                        if (s0 + i < S) acc[q] += t[q][i];
            }
#pragma unroll
            for (int q = 0; q < E; ++q) {
                const int e = e0 + q * (int)blockDim.x;
                if (e >= items) continue;
                const int m = e / C4;
                const int n = col0 + 4 * (e - m * C4);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float v = acc[q][k];
                    if (scaled) v *= scale;
                    if (bias) v += bf16_to_f32(bb[q][k]);
                    store_out(out, (size_t)m * N + n + k, v, out_f32);
                }
            }
        }
        return;
    }
    const int elems = M * ncols;
    for (int e = threadIdx.x; e < elems; e += blockDim.x) {
        const int m = e / ncols;
        const int n = col0 + (e - m * ncols);
        const unsigned bb = load_bias_bits(br, n);  // ahead of the partials
        float v = ordered_sum<8>(S, [&](int ss) {
            return __hip_atomic_load(ws + ((size_t)ss * M + m) * N + n, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        });
        if (scaled) v *= scale;
        if (bias) v += bf16_to_f32(bb);
        store_out(out, (size_t)m * N + n, v, out_f32);
    }
}

}  // namespace skg
