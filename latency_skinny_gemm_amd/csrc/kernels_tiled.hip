// kernels_tiled.hip -- split-K MFMA kernel with LDS-staged operand tiles,
// for larger M x N (the dense decode linear, M up to 128).
//
// The "vllm PR #42562" page's split-K kernel stages A and B tiles through
// shared memory in a multi-stage pipeline and pads M to the MMA tile.  Here
// that staging pays off once one workgroup covers many columns and all of
// M: every W row and every x row of a K step is loaded once per workgroup
// and read from LDS by the waves that need it, so x is re-read once per
// 16*NB columns instead of once per 16.
//  * workgroup (j, s): columns [16*NB*j, 16*NB*(j+1)), all M rows (MT
//    16-row tiles, rows past M read as zeros), K chunk s;
//  * 4 waves arranged WM x WN (WM*WN = 4); wave (wm, wn) owns MTW m-tiles by
//    NBW column blocks of the output and never shares a tile, so there is no
//    cross-wave reduction;
//  * per 32-wide K step the workgroup loads MT x-blocks and NB W-blocks of
//    1 KB each.  A block is stored in LDS exactly in v_mfma_f32_16x16x32_bf16
//    operand order (lane p holds row p%16, bytes 16*(p/16)..+16 of the
//    step's 64 bytes), so every fragment read is one linear, conflict-free
//    ds_read_b128;
//  * D steps form a chunk; chunks alternate between two register sets
//    (global loads in flight) and two LDS buffers, one barrier per chunk;
//  * K splits (S > 1) reuse the ordered reductions of the split-K kernel.
#include "device_common.h"
#include "internal.h"
#include "splitk_common.h"

namespace skg {

template <int MTW, int NBW, int WM, int D>
__global__ void __launch_bounds__(256)
    tiled_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
                 const uint16_t *__restrict__ bias, uint16_t *__restrict__ out,
                 float *__restrict__ ws, unsigned *__restrict__ tickets, int M, int N, int K,
                 int S, int k_chunk, int reduce) {
    constexpr int WN = 4 / WM;
    constexpr int MT = MTW * WM;          // 16-row tiles the workgroup covers
    constexpr int NB = NBW * WN;          // 16-column blocks the workgroup covers
    constexpr int BLK = MT + NB;          // 1 KB blocks per K step
    constexpr int PAIRS = BLK * 64;       // (block, lane) pairs per step
    constexpr int R = (PAIRS + 255) / 256;  // pairs per thread per step
    constexpr int STEP_BYTES = BLK * 1024;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    __shared__ unsigned is_last;

    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lane = t & 63;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int s = blockIdx.x % S;
    const int j = blockIdx.x / S;
    const int col0 = j * NB * 16;
    const int ncols = min(NB * 16, N - col0);
    const unsigned rowb = (unsigned)K * 2u;
    const Rsrc wr = make_rsrc(W + (size_t)col0 * K, (unsigned)ncols * rowb);
    const Rsrc xr = make_rsrc(x, (unsigned)M * rowb);
    const int kbeg = s * k_chunk;
    const int kend = min(K, kbeg + k_chunk);
    const int nsteps = (kend - kbeg + 31) >> 5;
    const int nch = (nsteps + D - 1) / D;

    // per-thread load slots: pair q = t + 256*r -> (block, p); the block's
    // row and the lane's 16-byte column inside the step's 64 bytes
    unsigned row_off[R];   // byte offset of the row in its buffer resource
    bool is_w[R], valid[R];
    unsigned kbyte[R];     // 16*(p/16)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int q = t + 256 * r;
        valid[r] = q < PAIRS;
        const int blk = q >> 6, p = q & 63;
        is_w[r] = blk >= MT;
        const int row = (is_w[r] ? blk - MT : blk) * 16 + (p & 15);
        row_off[r] = (unsigned)row * rowb;
        kbyte[r] = (unsigned)(p >> 4) * 16u;
    }

    auto load_chunk = [&](u32x4(&regs)[D][R], int c) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int st = c * D + d;
            const int k0 = kbeg + st * 32;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const unsigned kb = (unsigned)k0 * 2u + kbyte[r];
                const bool ok = valid[r] & (st < nsteps) & ((int)(kb >> 1) < kend);
                const unsigned off = ok ? row_off[r] + kb : kOOB;
                regs[d][r] = is_w[r] ? load16<kCacheStream>(wr, off) : load16<kCacheDefault>(xr, off);
            }
        }
    };
    auto store_chunk = [&](unsigned char *buf, u32x4(&regs)[D][R]) {
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (valid[r])
                    *reinterpret_cast<u32x4 *>(buf + d * STEP_BYTES + (t + 256 * r) * 16) = regs[d][r];
    };

    f32x4 acc[MTW][NBW];
#pragma unroll
    for (int a = 0; a < MTW; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_chunk = [&](const unsigned char *buf) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const unsigned char *stp = buf + d * STEP_BYTES;
            u32x4 af[MTW], bf[NBW];
#pragma unroll
            for (int a = 0; a < MTW; ++a)
                af[a] = *reinterpret_cast<const u32x4 *>(stp + (wm * MTW + a) * 1024 + lane * 16);
#pragma unroll
            for (int b = 0; b < NBW; ++b)
                bf[b] = *reinterpret_cast<const u32x4 *>(stp + (MT + wn * NBW + b) * 1024 + lane * 16);
#pragma unroll
            for (int a = 0; a < MTW; ++a)
#pragma unroll
                for (int b = 0; b < NBW; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, af[a]), __builtin_bit_cast(bf16x8, bf[b]),
                        acc[a][b], 0, 0, 0);
        }
    };

    unsigned char *lds0 = lds_raw;
    unsigned char *lds1 = lds_raw + D * STEP_BYTES;
    u32x4 ra[D][R], rb[D][R];
    load_chunk(ra, 0);
    for (int c = 0; c < nch; c += 2) {
        // nch is the same for every wave of the workgroup: the branches below
        // are uniform and every wave reaches every barrier
        load_chunk(rb, c + 1);  // past the end: zeros, no memory traffic
        store_chunk(lds0, ra);
        __syncthreads();
        compute_chunk(lds0);
        if (c + 1 < nch) {
            load_chunk(ra, c + 2);
            store_chunk(lds1, rb);
            __syncthreads();
            compute_chunk(lds1);
        }
    }

    // ---- epilogue: MFMA 16x16 layout, lane l register i -> row 4*(l/16)+i,
    // column l%16 of the tile
#pragma unroll
    for (int a = 0; a < MTW; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = (wm * MTW + a) * 16 + (lane >> 4) * 4 + i;
                const int n = col0 + (wn * NBW + b) * 16 + (lane & 15);
                if (m < M && n < N) {
                    float v = acc[a][b][i];
                    if (S == 1) {
                        if (bias) v += bf16_to_f32(bias[n]);
                        out[(size_t)m * N + n] = f32_to_bf16_rne(v);
                    } else {
                        ws[((size_t)s * M + m) * N + n] = v;
                    }
                }
            }
    if (S == 1 || reduce != SKG_REDUCE_LAST) return;
    last_arriver_reduce(ws, tickets, bias, out, M, N, S, j, col0, ncols, &is_last);
}

namespace {

typedef int (*TiledLaunch)(const SkgPlan &, const void *, const void *, const void *, void *,
                           float *, unsigned *, int, int, int, hipStream_t);

template <int MTW, int NBW, int WM, int D>
int launch_tiled_t(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                   float *ws, unsigned *tickets, int M, int N, int K, hipStream_t stream) {
    constexpr int BLK = MTW * WM + NBW * (4 / WM);
    const size_t lds_bytes = (size_t)2 * D * BLK * 1024;
    hipLaunchKernelGGL((tiled_kernel<MTW, NBW, WM, D>), dim3(p.grid), dim3(256), lds_bytes,
                       stream, (const uint16_t *)x, (const uint16_t *)W, (const uint16_t *)bias,
                       (uint16_t *)out, ws, tickets, M, N, K, p.splits, p.k_chunk, p.reduce);
    return (int)hipGetLastError();
}

template <int MTW, int NBW, int WM, int D>
constexpr TiledLaunch tiled_entry() {
    if constexpr (tiled_built(MTW, NBW, WM, D))
        return &launch_tiled_t<MTW, NBW, WM, D>;
    else
        return nullptr;
}

template <int MTW, int NBW, int WM>
TiledLaunch pick_d(int D) {
    switch (D) {
    case 1: return tiled_entry<MTW, NBW, WM, 1>();
    case 2: return tiled_entry<MTW, NBW, WM, 2>();
    case 4: return tiled_entry<MTW, NBW, WM, 4>();
    default: return nullptr;
    }
}

template <int MTW, int WM>
TiledLaunch pick_nbw(int NBW, int D) {
    switch (NBW) {
    case 1: return pick_d<MTW, 1, WM>(D);
    case 2: return pick_d<MTW, 2, WM>(D);
    case 4: return pick_d<MTW, 4, WM>(D);
    case 8: return pick_d<MTW, 8, WM>(D);
    default: return nullptr;
    }
}

template <int WM>
TiledLaunch pick_mtw(int MTW, int NBW, int D) {
    switch (MTW) {
    case 1: return pick_nbw<1, WM>(NBW, D);
    case 2: return pick_nbw<2, WM>(NBW, D);
    case 4: return pick_nbw<4, WM>(NBW, D);
    default: return nullptr;
    }
}

TiledLaunch pick(int MTW, int NBW, int WM, int D) {
    switch (WM) {
    case 1: return pick_mtw<1>(MTW, NBW, D);
    case 2: return pick_mtw<2>(MTW, NBW, D);
    case 4: return pick_mtw<4>(MTW, NBW, D);
    default: return nullptr;
    }
}

}  // namespace

int launch_tiled(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                 float *ws, unsigned *tickets, int M, int N, int K, hipStream_t stream) {
    int MTW = 0, NBW = 0, WM = 0;
    tiled_shape(p, M, &MTW, &NBW, &WM);
    TiledLaunch f = pick(MTW, NBW, WM, p.depth);
    if (!f) return (int)hipErrorInvalidConfiguration;
    int rc = f(p, x, W, bias, out, ws, tickets, M, N, K, stream);
    if (rc != (int)hipSuccess || p.splits == 1 || p.reduce != SKG_REDUCE_KERNEL) return rc;
    return launch_splitk_reduce(ws, bias, out, M, N, p.splits, stream);
}

}  // namespace skg
