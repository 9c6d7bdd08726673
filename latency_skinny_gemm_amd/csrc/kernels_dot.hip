// kernels_dot.hip -- dot-product kernel for tiny M (gfx950).
//
// The "vllm PR #42562" page (impl. item 1 and the LLBf16Dotprod snippet)
// gives the idea: one workgroup per output column (expert), the whole K
// loop unrolled at compile time, 128-bit vector loads of W, a per-token fp32
// multiply-add, and a shuffle + shared-memory reduction.  Here, on 64-wide
// waves:
//  * workgroup b owns C consecutive columns n0 = b*C ...; thread t owns the
//    16-byte vectors t, t+T, t+2T, ... of K (V of them), so each wave-wide
//    load instruction covers 1 KB of one W row, coalesced;
//  * every load of W (streaming, non-temporal) and of x is issued before
//    the first multiply: the whole per-workgroup slice is in flight at once;
//  * vectors past K read as zeros through the buffer resource's range
//    check, so there is no scalar tail loop (K % 8 == 0 always holds);
//  * the multiply-add is either fp32 FMA on widened bf16 (one IEEE rounding
//    per product) or, with SKG_FLAG_DOT2, gfx950's bf16 dot instruction
//    (two products per instruction on packed operands, no widening);
//  * the per-thread sums of all C*M outputs are reduced over the wave
//    together by a reduce-scatter (two lane-swap levels and four DPP
//    levels, each halving the values a lane holds), then over the waves
//    through LDS in wave order, then bias is added in fp32 and the sum is
//    rounded once to bf16.
// Every reduction order is fixed: the result is bitwise reproducible for a
// given plan and input.
#include <atomic>

#include "device_common.h"
#include "internal.h"
#include "lds_limit.h"

namespace skg {

// W1: the workgroup is one wave (its own instantiation, so the multi-wave
// kernels compile exactly as without it).
// WF (SKG_FLAG_DOT_WFIRST): the issue order of the loads.  Without it the
// compiler orders them (it interleaves the W and x loads of successive
// vectors and starts the first products while later x loads are still
// being issued); with it every W load (the HBM stream, the longest latency)
// and the bias load go first, pinned by a scheduling barrier, and the x
// loads (from L2) and the products follow in the compiler's order.  Which
// is faster depends on the shape (measured: W first gains up to 16 % at
// 384 columns and 15-16 rows, and loses up to 7 % at 1-7 rows), so the
// planner's table picks per shape.  The bias is loaded at the start with
// WF and after the reductions without it: any other instruction in the
// loads' scheduling region changed the compiler's order there (measured
// 2-7 % slower at 5-12 rows).
template <int M, int C, int V, bool DOT2, bool W1, bool WF>
__global__ void __launch_bounds__((W1 ? 64 : dot_max_threads(M, C, V, DOT2)))
    dot_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
               const uint16_t *__restrict__ bias, void *__restrict__ out, int N, int K,
               int out_f32) {
    const int T = blockDim.x;
    const int t = threadIdx.x;
    const int n0 = blockIdx.x * C;
    const int ncols = min(C, N - n0);
    const unsigned rowb = (unsigned)K * 2u;
    const Rsrc wr = make_rsrc(W + (size_t)n0 * K, (unsigned)ncols * rowb);
    const Rsrc xr = make_rsrc(x, (unsigned)M * rowb);
    const int K8 = K >> 3;

    // The C*M sums end in a reduce-scatter over the wave (lane l ends with
    // the total of index l >> (6 - L), index c*M + m) and then, across
    // waves, in thread t < C*M.  So the thread that stores index i, and the
    // bias column n0 + i / M it adds, are known from the start (WF loads it
    // then).
    constexpr int CM = C * M;
    constexpr int L = CM <= 1 ? 0 : CM <= 2 ? 1 : CM <= 4 ? 2 : CM <= 8 ? 3 : CM <= 16 ? 4 : CM <= 32 ? 5 : 6;
    static_assert(CM <= 64, "one value index per lane at most");
    const int eidx = W1 ? (t & 63) >> (6 - L) : t;
    auto load_bias = [&]() {
        return load_bias_bits(bias_rsrc(bias, N), n0 + eidx / M, eidx < CM);
    };

    u32x4 wv[C][V];
    u32x4 xv[M][V];
    unsigned bb = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int v = t + i * T;
        const unsigned off = v < K8 ? (unsigned)v * 16u : kOOB;
#pragma unroll
        for (int c = 0; c < C; ++c) wv[c][i] = load16<kCacheStream>(wr, off + (unsigned)c * rowb);
    }
    if constexpr (WF) {
        bb = load_bias();
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int v = t + i * T;
        const unsigned off = v < K8 ? (unsigned)v * 16u : kOOB;
#pragma unroll
        for (int m = 0; m < M; ++m) xv[m][i] = load16<kCacheDefault>(xr, off + (unsigned)m * rowb);
    }

    float acc[C][M];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[c][m] = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int m = 0; m < M; ++m)
                acc[c][m] = DOT2 ? dot8_dot2(xv[m][i], wv[c][i], acc[c][m])
                                 : dot8_fma(xv[m][i], wv[c][i], acc[c][m]);

    // Reduce-scatter the C*M per-lane sums over the wave (padded with zeros
    // to a power of two): lane l ends with the wave's total of index
    // l >> (6 - L), index c*M + m; the first lane of each index group owns it.
    float part[1 << L];
#pragma unroll
    for (int i = 0; i < (1 << L); ++i) part[i] = i < CM ? acc[i / M][i % M] : 0.0f;
    const float total = wave_reduce_scatter<L>(part);
    const int lane = t & 63;
    const int idx = lane >> (6 - L);
    const bool owner = (lane & ((1 << (6 - L)) - 1)) == 0 && idx < CM;

    __shared__ float red[kMaxThreads / 64][CM];
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int nw = T >> 6;
    if constexpr (W1) {
        // One wave: its totals are final, so each owner lane stores its
        // output with no LDS round trip and no barrier.  The sum starts from
        // 0 as the cross-wave sum below does: same bits.
        if (owner) {
            const int c = idx / M, m = idx - (idx / M) * M;
            const int n = n0 + c;
            if (n < N) {
                float s = 0.0f + total;
                if (bias) s += bf16_to_f32(WF ? bb : bias[n]);
                store_out(out, (size_t)m * N + n, s, out_f32);
            }
        }
        return;
    }
    if (owner) red[wave][idx] = total;
    __syncthreads();
    if (t < CM) {
        const int c = t / M;
        const int m = t - c * M;
        const int n = n0 + c;
        float s = ordered_sum<8>(nw, [&](int w) { return red[w][t]; });
        if (n < N) {
            if (bias) s += bf16_to_f32(WF ? bb : bias[n]);
            store_out(out, (size_t)m * N + n, s, out_f32);
        }
    }
}

// The dot kernel with x in LDS (SKG_FLAG_DOT_XLDS), for K = 512 * V exactly
// (every lane has V whole vectors of every row: no K tail).  A workgroup of
// nw waves covers CW * nw consecutive columns; wave w owns CW of them over
// the whole K, lane l the 16-byte vectors l, l + 64, ... (V of them) of
// each.  Order of work:
//  1. x (all M rows, in its own row-major layout) is copied to LDS by
//     buffer-to-LDS loads, 16 bytes a lane, 1 KB a wave per pass;
//  2. every W load of the wave (CW * V, streaming) is issued;
//  3. s_waitcnt vmcnt(CW * V): loads complete in issue order, so this waits
//     for the x loads only and leaves the W loads in flight; a barrier then
//     makes every wave's part of x visible;
//  4. the products: for each vector step, each row's x vector is read from
//     LDS once and used for the CW columns, as the W vectors arrive;
//  5. a wave reduce-scatter of the CW * M sums, and the owner lanes store.
// x is read from L2 once per workgroup (not once per C columns), and no
// cross-wave reduction is needed.  Lane l's sums and the reduction tree are
// those of the one-wave dot kernel, so at equal V the bits are the same.
template <int M, int CW, int V>
__global__ void __launch_bounds__(xlds_max_threads(M, CW, V))
    dotx_kernel(const uint16_t *x, const uint16_t *W, const uint16_t *__restrict__ bias,
                void *__restrict__ out, int N, int K, int out_f32) {
    extern __shared__ __attribute__((aligned(16))) unsigned char xs[];
    const int T = blockDim.x;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int nw = T >> 6;
    const int n0 = (blockIdx.x * nw + wave) * CW;  // this wave's first column
    const int ncols = n0 < N ? min(CW, N - n0) : 0;
    const unsigned rowb = (unsigned)K * 2u;
    constexpr int K8 = V * 64;                     // K / 8
    const Rsrc xr = make_rsrc(x, (unsigned)M * rowb);
    const Rsrc wr = make_rsrc(W + (size_t)(ncols ? n0 : 0) * K, (unsigned)ncols * rowb);

    // 0. the bias of the column this lane stores (index idx of step 5's
    // reduce-scatter), ahead of every operand load (no load without a bias)
    constexpr int CM = CW * M;
    constexpr int L = CM <= 1 ? 0 : CM <= 2 ? 1 : CM <= 4 ? 2 : CM <= 8 ? 3 : CM <= 16 ? 4 : CM <= 32 ? 5 : 6;
    static_assert(CM <= 64, "one value index per lane at most");
    const int idx = lane >> (6 - L);
    unsigned bb = 0;
    if (bias) bb = load_bias_bits(bias_rsrc(bias, N), n0 + idx / M, idx < CM && idx / M < ncols);

    // 1. x -> LDS: wave w moves chunks q0 ... q0 + 63 for q0 = 64w, 64w + T,
    // ... below M * K8 (both sides contiguous; M * K8 is a multiple of 64)
#pragma unroll 1
    for (int q0 = wave * 64; q0 < M * K8; q0 += T)
        lds_load16<kCacheDefault>(xr, xs + (size_t)q0 * 16u, (unsigned)(q0 + lane) * 16u);
    // The W loads must follow the x loads and precede the wait: the count
    // in step 3 depends on it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 2. W, step-major (the order the products consume them); columns past
    // N read zeros through the range check
    u32x4 wv[V][CW];
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
        for (int c = 0; c < CW; ++c)
            wv[i][c] = load16<kCacheStream>(wr, (unsigned)(i * 64 + lane) * 16u + (unsigned)c * rowb);
    __builtin_amdgcn_sched_barrier(0);

    // 3. this wave's x loads are done once at most its CW*V W loads remain;
    // then every wave's
    wait_vmcnt_lds<CW * V>();
    barrier_nofence();

    // 4. products
    float acc[CW][M];
#pragma unroll
    for (int c = 0; c < CW; ++c)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[c][m] = 0.0f;
    const unsigned char *xl = xs + (size_t)lane * 16u;
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const u32x4 xv = *reinterpret_cast<const u32x4 *>(xl + (size_t)(m * K8 + i * 64) * 16u);
#pragma unroll
            for (int c = 0; c < CW; ++c) acc[c][m] = dot8_dot2(xv, wv[i][c], acc[c][m]);
        }

    // 5. reduce-scatter over the wave; lane l owns index l >> (6 - L), c*M + m
    float part[1 << L];
#pragma unroll
    for (int i = 0; i < (1 << L); ++i) part[i] = i < CM ? acc[i / M][i % M] : 0.0f;
    const float total = wave_reduce_scatter<L>(part);
    if ((lane & ((1 << (6 - L)) - 1)) == 0 && idx < CM) {
        const int c = idx / M, m = idx - (idx / M) * M;
        if (c < ncols) {
            const int n = n0 + c;
            float s = 0.0f + total;  // as the one-wave dot kernel: same bits
            if (bias) s += bf16_to_f32(bb);
            store_out(out, (size_t)m * N + n, s, out_f32);
        }
    }
}

namespace {

typedef int (*DotLaunch)(const SkgPlan &, const void *, const void *, const void *, void *, int,
                         int, int, hipStream_t);

template <int M, int C, int V, bool DOT2, bool WF>
int launch_dot_t(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                 int N, int K, int out_f32, hipStream_t stream) {
    if constexpr (M <= kDotOneWaveMaxM) {
        if (p.threads == 64) {
            hipLaunchKernelGGL((dot_kernel<M, C, V, DOT2, true, WF>), dim3(p.grid), dim3(64), 0,
                               stream, (const uint16_t *)x, (const uint16_t *)W,
                               (const uint16_t *)bias, out, N, K, out_f32);
            return (int)hipGetLastError();
        }
    }
    hipLaunchKernelGGL((dot_kernel<M, C, V, DOT2, false, WF>), dim3(p.grid), dim3(p.threads), 0,
                       stream, (const uint16_t *)x, (const uint16_t *)W, (const uint16_t *)bias,
                       out, N, K, out_f32);
    return (int)hipGetLastError();
}

// Instantiated only where the per-thread registers fit (the planner applies
// the same bound and never asks for the others); the W-first order only
// with the dot instruction (the planner rejects it without).
template <int M, int C, int V, bool DOT2, bool WF>
constexpr DotLaunch dot_entry() {
    if constexpr (dot_regs(M, C, V, DOT2) <= kDotRegsMax && (DOT2 || !WF))
        return &launch_dot_t<M, C, V, DOT2, WF>;
    else
        return nullptr;
}

template <int M, int C, bool DOT2, bool WF>
DotLaunch pick_v(int V) {
    switch (V) {
    case 1: return dot_entry<M, C, 1, DOT2, WF>();
    case 2: return dot_entry<M, C, 2, DOT2, WF>();
    case 3: return dot_entry<M, C, 3, DOT2, WF>();
    case 4: return dot_entry<M, C, 4, DOT2, WF>();
    case 6: return dot_entry<M, C, 6, DOT2, WF>();
    case 7: return dot_entry<M, C, 7, DOT2, WF>();
    case 8: return dot_entry<M, C, 8, DOT2, WF>();
    case 12: return dot_entry<M, C, 12, DOT2, WF>();
    case 14: return dot_entry<M, C, 14, DOT2, WF>();
    case 16: return dot_entry<M, C, 16, DOT2, WF>();
    default: return nullptr;
    }
}

template <int M, int C>
DotLaunch pick_f(int V, bool dot2, bool wf) {
    if (!dot2) return wf ? nullptr : pick_v<M, C, false, false>(V);
    return wf ? pick_v<M, C, true, true>(V) : pick_v<M, C, true, false>(V);
}

template <int M>
DotLaunch pick_c(int C, int V, bool dot2, bool wf) {
    switch (C) {
    case 1: return pick_f<M, 1>(V, dot2, wf);
    case 2: return pick_f<M, 2>(V, dot2, wf);
    case 3: return pick_f<M, 3>(V, dot2, wf);
    case 4: return pick_f<M, 4>(V, dot2, wf);
    default: return nullptr;
    }
}

DotLaunch pick(int M, int C, int V, bool dot2, bool wf) {
    switch (M) {
    case 1: return pick_c<1>(C, V, dot2, wf);
    case 2: return pick_c<2>(C, V, dot2, wf);
    case 3: return pick_c<3>(C, V, dot2, wf);
    case 4: return pick_c<4>(C, V, dot2, wf);
    case 5: return pick_c<5>(C, V, dot2, wf);
    case 6: return pick_c<6>(C, V, dot2, wf);
    case 7: return pick_c<7>(C, V, dot2, wf);
    case 8: return pick_c<8>(C, V, dot2, wf);
    case 9: return pick_c<9>(C, V, dot2, wf);
    case 10: return pick_c<10>(C, V, dot2, wf);
    case 11: return pick_c<11>(C, V, dot2, wf);
    case 12: return pick_c<12>(C, V, dot2, wf);
    case 13: return pick_c<13>(C, V, dot2, wf);
    case 14: return pick_c<14>(C, V, dot2, wf);
    case 15: return pick_c<15>(C, V, dot2, wf);
    case 16: return pick_c<16>(C, V, dot2, wf);
    default: return nullptr;
    }
}

template <int M, int CW, int V>
int launch_dotx_t(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                  int N, int K, int out_f32, hipStream_t stream) {
    const int K8 = K / 8;
    if (K8 != V * 64) return (int)hipErrorInvalidConfiguration;  // the kernel's contract
    const size_t lds = (size_t)xlds_lds_bytes(M, K8);
    static std::atomic<unsigned long long> lds_set{0};
    if (lds > 64 * 1024) {
        const hipError_t attr = allow_dynamic_lds(
            reinterpret_cast<const void *>(&dotx_kernel<M, CW, V>), lds, lds_set);
        if (attr != hipSuccess) return (int)attr;
    }
    hipLaunchKernelGGL((dotx_kernel<M, CW, V>), dim3(p.grid), dim3(p.threads), lds, stream,
                       (const uint16_t *)x, (const uint16_t *)W, (const uint16_t *)bias, out, N, K,
                       out_f32);
    return (int)hipGetLastError();
}

template <int M, int CW, int V>
constexpr DotLaunch dotx_entry() {
    if constexpr (xlds_built(M, CW, V))
        return &launch_dotx_t<M, CW, V>;
    else
        return nullptr;
}

template <int M, int CW>
DotLaunch pickx_v(int V) {
    switch (V) {
    case 4: return dotx_entry<M, CW, 4>();
    case 6: return dotx_entry<M, CW, 6>();
    case 8: return dotx_entry<M, CW, 8>();
    case 12: return dotx_entry<M, CW, 12>();
    case 14: return dotx_entry<M, CW, 14>();
    case 16: return dotx_entry<M, CW, 16>();
    default: return nullptr;
    }
}

template <int M>
DotLaunch pickx_c(int CW, int V) {
    if (CW == 1) return pickx_v<M, 1>(V);
    if (CW == 2) return pickx_v<M, 2>(V);
    if (CW == 4) return pickx_v<M, 4>(V);
    return nullptr;
}

DotLaunch pickx(int M, int CW, int V) {
    switch (M) {
    case 1: return pickx_c<1>(CW, V);
    case 2: return pickx_c<2>(CW, V);
    case 3: return pickx_c<3>(CW, V);
    case 4: return pickx_c<4>(CW, V);
    case 5: return pickx_c<5>(CW, V);
    case 6: return pickx_c<6>(CW, V);
    case 7: return pickx_c<7>(CW, V);
    case 8: return pickx_c<8>(CW, V);
    case 9: return pickx_c<9>(CW, V);
    case 10: return pickx_c<10>(CW, V);
    case 11: return pickx_c<11>(CW, V);
    case 12: return pickx_c<12>(CW, V);
    case 13: return pickx_c<13>(CW, V);
    case 14: return pickx_c<14>(CW, V);
    case 15: return pickx_c<15>(CW, V);
    case 16: return pickx_c<16>(CW, V);
    default: return nullptr;
    }
}

}  // namespace

int launch_dot(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
               int out_f32, int M, int N, int K, hipStream_t stream) {
    DotLaunch f = (p.flags & SKG_FLAG_DOT_XLDS)
                      ? pickx(M, p.cols / (p.threads / 64), p.depth)
                      : pick(M, p.cols, p.depth, (p.flags & SKG_FLAG_DOT2) != 0,
                             (p.flags & SKG_FLAG_DOT_WFIRST) != 0);
    if (!f) return (int)hipErrorInvalidConfiguration;
    return f(p, x, W, bias, out, N, K, out_f32, stream);
}

}  // namespace skg
