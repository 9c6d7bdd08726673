// kernels_splitk.hip -- split-K MFMA kernel and its ordered reduction (gfx950).
//
// The "vllm PR #42562" page (impl. item 2, the LLBf16SplitK snippet and the
// review notes) splits K over the CTAs of a cluster, pads M to a 16-row MMA
// tile, accumulates in fp32 and reduces the partials through distributed
// shared memory after a cluster barrier.  gfx950 has no clusters and no
// DSMEM; here:
//  * workgroup (j, s) owns columns [16*NB*j, 16*NB*(j+1)) and the K chunk
//    [s*k_chunk, (s+1)*k_chunk); each wave takes a contiguous run of the
//    chunk's 32-wide K steps;
//  * each step is one v_mfma_f32_16x16x32_bf16 per (m-tile, column block):
//    A = x rows (M padded to 16 with zeros), B = W rows.  A lane's 8-element
//    B operand is 16 contiguous bytes of one W row, so W goes from HBM
//    straight into the MFMA operand registers with coalesced 16-byte loads
//    (64 contiguous bytes per row per step);
//  * a wave keeps 2 x D steps of loads in flight (two register stages used
//    alternately), so the W stream never waits on an MFMA;
//  * rows past M, columns past N and K past the chunk read as zeros through
//    the buffer resources' range check;
//  * the waves' 16x16 fp32 tiles are summed through LDS in wave order;
//  * with S > 1 each workgroup writes its fp32 partial to the workspace
//    ws[s][m][n]; the partials are then summed in ascending s by either the
//    last workgroup of the tile to finish (partials stored at device scope,
//    a device-scope ticket counter and device-scope loads, no cache
//    write-back; no workgroup ever waits on another) or by a second kernel.  Both add the same numbers in the same order, so the
//    output does not depend on which workgroup finishes last.
#include "device_common.h"
#include "internal.h"
#include "splitk_common.h"

namespace skg {

template <int MT, int NB, int D>
__global__ void __launch_bounds__((splitk_max_threads(MT, NB, D)))
    splitk_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
                  const uint16_t *__restrict__ bias, void *__restrict__ out,
                  float *__restrict__ ws, unsigned *__restrict__ tickets, int M, int N, int K,
                  int S, int k_chunk, int reduce, int out_f32) {
    extern __shared__ float lds[];
    __shared__ unsigned is_last;

    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.x % S;  // split index fastest: the S workgroups of
    const int j = blockIdx.x / S;  // a tile share one x chunk per XCD
    const int col0 = j * NB * 16;
    const int ncols = min(NB * 16, N - col0);
    const unsigned rowb = (unsigned)K * 2u;
    const Rsrc wr = make_rsrc(W + (size_t)col0 * K, (unsigned)ncols * rowb);
    const Rsrc xr = make_rsrc(x, (unsigned)M * rowb);
    const int kbeg = s * k_chunk;
    const int kend = min(K, kbeg + k_chunk);
    const int nsteps = (kend - kbeg + 31) >> 5;
    // each wave takes a contiguous run of steps, so the two 64-byte halves
    // of a 128-byte W line are read by the same wave, back to back
    const int spw = (nsteps + nw - 1) / nw;
    const int first_step = wave * spw;
    const int my_steps = max(0, min(spw, nsteps - first_step));
    const int nchunks = (my_steps + D - 1) / D;
    const unsigned r16 = (unsigned)(lane & 15);
    const int kq = (lane >> 4) * 8;

    // (S == 1) the bias of the lane's column in each of the NB column
    // blocks, loaded ahead of the operand stream for the epilogue
    unsigned bb[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) bb[nb] = 0;
    if (bias && S == 1) {
        const Rsrc br = bias_rsrc(bias, N);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bb[nb] = load_bias_bits(br, col0 + nb * 16 + (lane & 15));
    }

    f32x4 acc[NB][MT];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wa[D][NB], xa[D][MT], wb[D][NB], xb[D][MT];

    auto load_stage = [&](u32x4(&wbuf)[D][NB], u32x4(&xbuf)[D][MT], int chunk) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = chunk * D + d;
            const int k = kbeg + (first_step + i) * 32 + kq;
            const unsigned koff = ((i < my_steps) & (k < kend)) ? (unsigned)k * 2u : kOOB;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                wbuf[d][nb] = load16<kCacheStream>(wr, koff + ((unsigned)nb * 16u + r16) * rowb);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                xbuf[d][mt] = load16<kCacheDefault>(xr, koff + ((unsigned)mt * 16u + r16) * rowb);
        }
    };
    auto mma_stage = [&](u32x4(&wbuf)[D][NB], u32x4(&xbuf)[D][MT]) {
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, xbuf[d][mt]),
                        __builtin_bit_cast(bf16x8, wbuf[d][nb]), acc[nb][mt], 0, 0, 0);
    };

    if (nchunks <= 1) {
        load_stage(wa, xa, 0);
        mma_stage(wa, xa);
    } else {
        load_stage(wa, xa, 0);
        for (int c = 0; c < nchunks; c += 2) {
            load_stage(wb, xb, c + 1);  // past the end: all zeros, no traffic
            mma_stage(wa, xa);
            load_stage(wa, xa, c + 2);
            mma_stage(wb, xb);
        }
    }

    // ---- sum the waves' tiles through LDS, in wave order
    // layout: [wave][q = (nb*MT + mt)*4 + i][lane]
    constexpr int Q = NB * MT * 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lds[(wave * Q + (nb * MT + mt) * 4 + i) * 64 + lane] = acc[nb][mt][i];
    __syncthreads();

    // MFMA 16x16 output layout: lane l, register i holds row 4*(l/16)+i,
    // column l%16 of the tile; rows are m (from x), columns n (from W).
    for (int q = wave; q < Q; q += nw) {
        float v = ordered_sum<8>(nw, [&](int w) { return lds[(w * Q + q) * 64 + lane]; });
        const int nb = q / (MT * 4);
        const int mt = (q >> 2) % MT;
        const int i = q & 3;
        const int n = col0 + nb * 16 + (lane & 15);
        const int m = mt * 16 + (lane >> 4) * 4 + i;
        if (m < M && n < N) {
            if (S == 1) {
                unsigned b = bb[0];  // bb[nb], without indexing registers at run time
#pragma unroll
                for (int k = 1; k < NB; ++k) b = nb == k ? bb[k] : b;
                if (bias) v += bf16_to_f32(b);
                store_out(out, (size_t)m * N + n, v, out_f32);
            } else {
                put_partial(ws, ((size_t)s * M + m) * N + n, v, reduce == SKG_REDUCE_LAST);
            }
        }
    }
    if (S == 1 || reduce != SKG_REDUCE_LAST) return;

    last_arriver_reduce<2, 4>(ws, tickets, bias, out, out_f32, M, N, S, j, col0, ncols, &is_last);
}

// Second-pass reduction: the same sum in the same order as the in-kernel
// one, one output element per thread.
__global__ void __launch_bounds__(256)
    splitk_reduce_kernel(const float *__restrict__ ws, const uint16_t *__restrict__ bias,
                         void *__restrict__ out, int M, int N, int S,
                         const float *__restrict__ sx, const float *__restrict__ sw, int out_f32) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= M * N) return;
    const int m = e / N;
    const int n = e - m * N;
    // bias and scales first: their loads overlap the partials' loads (none
    // is issued for a null pointer)
    unsigned bb = 0;
    if (bias) bb = load_bias_bits(bias_rsrc(bias, N), n);
    float sxv = 1.0f, swv = 1.0f;
    if (sx) {
        sxv = load_scale(sx);
        swv = load_scale(sw);
    }
    float v = ordered_sum<8>(S, [&](int ss) { return ws[((size_t)ss * M + m) * N + n]; });
    if (sx) v *= sxv * swv;  // FP8 per-tensor scale product, applied once
    if (bias) v += bf16_to_f32(bb);
    store_out(out, e, v, out_f32);
}

// The same reduction, four consecutive outputs per thread (N % 4 == 0, so
// the four share a row and every partial load is 16 bytes).  Each of the
// four sums adds the partials in ascending s, as above: identical bits.
__global__ void __launch_bounds__(256)
    splitk_reduce4_kernel(const float *__restrict__ ws, const uint16_t *__restrict__ bias,
                          void *__restrict__ out, int M, int N, int S,
                          const float *__restrict__ sx, const float *__restrict__ sw,
                          int out_f32) {
    const int e = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (e >= M * N) return;
    const size_t plane = (size_t)M * N;
    const int n = e % N;
    // bias and scales first: their loads overlap the partials' loads
    // instead of following them one round trip each (none is issued for a
    // null pointer)
    unsigned bb[4] = {0, 0, 0, 0};
    if (bias) {
        const Rsrc br = bias_rsrc(bias, N);
#pragma unroll
        for (int q = 0; q < 4; ++q) bb[q] = load_bias_bits(br, n + q);
    }
    float sxv = 1.0f, swv = 1.0f;
    if (sx) {
        sxv = load_scale(sx);
        swv = load_scale(sw);
    }
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < S; i0 += 8) {
        f32x4 t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            t[i] = (i0 + i < S) ? *reinterpret_cast<const f32x4 *>(ws + (i0 + i) * plane + e)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i0 + i < S) v += t[i];
    }
    const float scale = sxv * swv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float r = v[q];
        if (sx) r *= scale;
        if (bias) r += bf16_to_f32(bb[q]);
        store_out(out, e + q, r, out_f32);
    }
}

namespace {

typedef int (*SplitKLaunch)(const SkgPlan &, const void *, const void *, const void *, void *,
                            int, float *, unsigned *, int, int, int, hipStream_t);

template <int MT, int NB, int D>
int launch_splitk_t(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                    int out_f32, float *ws, unsigned *tickets, int M, int N, int K,
                    hipStream_t stream) {
    const size_t lds_bytes = (size_t)(p.threads / 64) * NB * MT * 4 * 64 * sizeof(float);
    hipLaunchKernelGGL((splitk_kernel<MT, NB, D>), dim3(p.grid), dim3(p.threads), lds_bytes,
                       stream, (const uint16_t *)x, (const uint16_t *)W, (const uint16_t *)bias,
                       out, ws, tickets, M, N, K, p.splits, p.k_chunk, p.reduce, out_f32);
    return (int)hipGetLastError();
}

template <int MT, int NB, int D>
constexpr SplitKLaunch splitk_entry() {
    if constexpr (splitk_built(MT, NB, D))
        return &launch_splitk_t<MT, NB, D>;
    else
        return nullptr;
}

template <int MT, int NB>
SplitKLaunch pick_d(int D) {
    switch (D) {
    case 1: return splitk_entry<MT, NB, 1>();
    case 2: return splitk_entry<MT, NB, 2>();
    case 4: return splitk_entry<MT, NB, 4>();
    case 8: return splitk_entry<MT, NB, 8>();
    default: return nullptr;
    }
}

template <int MT>
SplitKLaunch pick_nb(int NB, int D) {
    return NB == 1 ? pick_d<MT, 1>(D) : NB == 2 ? pick_d<MT, 2>(D) : NB == 4 ? pick_d<MT, 4>(D)
                                                                              : nullptr;
}

SplitKLaunch pick(int MT, int NB, int D) {
    switch (MT) {
    case 1: return pick_nb<1>(NB, D);
    case 2: return pick_nb<2>(NB, D);
    case 3: return pick_nb<3>(NB, D);
    case 4: return pick_nb<4>(NB, D);
    case 5: return pick_nb<5>(NB, D);
    case 6: return pick_nb<6>(NB, D);
    case 7: return pick_nb<7>(NB, D);
    case 8: return pick_nb<8>(NB, D);
    default: return nullptr;
    }
}

}  // namespace

int launch_splitk_reduce(const float *ws, const void *bias, void *out, int out_f32, int M, int N,
                         int S, hipStream_t stream, const float *sx, const float *sw) {
    const int elems = M * N;
    if ((N & 3) == 0)
        hipLaunchKernelGGL(splitk_reduce4_kernel, dim3((elems / 4 + 255) / 256), dim3(256), 0,
                           stream, ws, (const uint16_t *)bias, out, M, N, S, sx, sw, out_f32);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((elems + 255) / 256), dim3(256), 0, stream,
                           ws, (const uint16_t *)bias, out, M, N, S, sx, sw, out_f32);
    return (int)hipGetLastError();
}

int launch_splitk(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                  int out_f32, float *ws, unsigned *tickets, int M, int N, int K,
                  hipStream_t stream) {
    SplitKLaunch f = pick(p.m_tiles, p.cols, p.depth);
    if (!f) return (int)hipErrorInvalidConfiguration;
    int rc = f(p, x, W, bias, out, out_f32, ws, tickets, M, N, K, stream);
    if (rc != (int)hipSuccess || p.splits == 1 || p.reduce != SKG_REDUCE_KERNEL) return rc;
    return launch_splitk_reduce(ws, bias, out, out_f32, M, N, p.splits, stream);
}

}  // namespace skg
