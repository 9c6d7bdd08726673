// kernels_tiled.hip -- split-K MFMA kernel whose x and W tiles stream into a
// ring of LDS stages by direct buffer-to-LDS loads, for larger M x N (the
// dense decode linear, M up to 128).
//
// The "vllm PR #42562" page's split-K kernel stages A and B tiles through
// shared memory in a multi-stage pipeline and pads M to the MMA tile.  On
// gfx950 the staging needs no registers: buffer_load_dwordx4 with the LDS
// bit writes lane p's 16 bytes to LDS at (wave-uniform base) + 16*p, and an
// out-of-range lane writes zeros (both measured on the MI355X).  So:
//  * workgroup (mb, j, s): columns [16*NB*j, 16*NB*(j+1)), rows of row
//    block mb (MT 16-row tiles, MT a power of two; one block covers M up to
//    128, more rows take blocks of 128; rows past M read as zeros), K chunk s;
//    the split index is fastest in the grid, so with S a multiple of 8 every
//    XCD (workgroup i runs on XCD i % 8) holds one K chunk of x in its L2;
//  * a K step is 32 wide; per step the workgroup needs MT x-blocks and NB
//    W-blocks of 1 KB (16 rows x 64 bytes).  Lane p of the load that fills
//    a block reads row p%16, bytes 16*(p/16)..+16 of the step, so the block
//    lands in LDS exactly in v_mfma_f32_16x16x32_bf16 operand order and
//    every fragment read is one linear, conflict-free ds_read_b128;
//  * a stage holds U steps; NS stages form a ring.  Stage i+NS-1 goes into
//    the slot of stage i-1 as soon as every wave has read that slot (the
//    barrier before stage i's MFMAs), so NS-1 stages are in flight while
//    one is multiplied.  Each wave waits for its own loads of the stage with
//    s_waitcnt vmcnt (the count of its loads issued after them is fixed at
//    compile time) and for its own LDS reads, then one s_barrier makes every
//    wave's loads visible.
//    The same barrier also orders the next overwrite of a slot after every
//    wave's reads of it, so there is one barrier per stage and no fence;
//  * 4 waves arranged WM x WN own disjoint MT/WM x NB/WN tiles of the
//    output: no cross-wave reduction;
//  * K splits (S > 1) reuse the ordered reductions of the split-K kernel.
#include "device_common.h"
#include "internal.h"
#include "lds_limit.h"
#include "splitk_common.h"

namespace skg {

namespace {

// Chunk swizzle of row r (0..15) in a block whose rows hold 4*U chunks of
// 16 bytes: rows 64*U bytes apart share a 256-byte bank window 4/U at a
// time, so the XOR key is the row's index among those that share it.
template <int U>
__device__ __forceinline__ int swz(int r) {
    return (r / (4 / U)) & (4 * U - 1);
}

}  // namespace

template <int MT, int NB, int WM, int NS, int U>
__global__ void __launch_bounds__(256)
    tiled_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
                 const uint16_t *__restrict__ bias, void *__restrict__ out,
                 float *__restrict__ ws, unsigned *__restrict__ tickets, int M, int N, int K,
                 int S, int k_chunk, int reduce, int out_f32, int MB) {
    constexpr int WN = 4 / WM;
    constexpr int MTW = MT / WM;          // m-tiles per wave
    constexpr int NBW = NB / WN;          // column blocks per wave
    constexpr int BLK = MT + NB;          // blocks of U KB per stage
    constexpr int STAGE = BLK * U * 1024; // bytes per stage
    static_assert(MT % WM == 0 && NB % WN == 0, "wave arrangement");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    __shared__ unsigned is_last;

    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lane = t & 63;
    const int wm = wave / WN;
    const int wn = wave % WN;
    // workgroup (mb, j, s): row block mb of MT*16 rows (M > 128 only),
    // column group j, K chunk s
    const TiledPos pos_ = tiled_position(blockIdx.x, MB, S, gridDim.x / MB);
    const int mb = pos_.mb, s = pos_.s, j = pos_.j;
    const int row0 = mb * MT * 16;
    const int Mb = min(MT * 16, M - row0);  // rows of this block
    const int col0 = j * NB * 16;
    const int ncols = min(NB * 16, N - col0);
    const unsigned rowb = (unsigned)K * 2u;
    const Rsrc wr = make_rsrc(W + (size_t)col0 * K, (unsigned)ncols * rowb);
    const Rsrc xr = make_rsrc(x + (size_t)row0 * K, (unsigned)Mb * rowb);
    const int kbeg = s * k_chunk;
    const int nsteps = (min(K, kbeg + k_chunk) - kbeg) >> 5;  // K, k_chunk: multiples of 32
    const int nstages = (nsteps + U - 1) / U;

    // The epilogue's bias (S == 1), loaded now: thread t stores columns
    // col0 + 4 * (t % C4) + 0..3 of its rows.  Without a bias no load is
    // issued (the extra loads cost about 1 % at these shapes).
    constexpr int C4 = NB * 4;  // 4-column groups per row
    static_assert(256 % C4 == 0, "a thread keeps its column group");
    unsigned bb[4] = {0, 0, 0, 0};
    if (bias && S == 1) {
        const Rsrc br = bias_rsrc(bias, N);
        const int c = (t % C4) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) bb[q] = load_bias_bits(br, col0 + c + q);
    }

    // Stage layout: MT x-blocks then NB W-blocks; a block is 16 rows of the
    // stage's 64*U bytes (U steps), U KB, row-major.  Inside a row the
    // 16-byte chunk c sits at position c ^ swz(r), so the 16 rows that one
    // MFMA fragment read touches hit 16 different 16-byte bank groups.
    // A load instruction fills 1 KB of a block: 16/U whole rows of 64*U
    // contiguous bytes (lane p writes position 64*i + p of the block, i.e.
    // row (64*i + p) / (4*U), and reads the chunk that belongs there).
    // Wave w issues x instructions q = w + 4*i (q < MT*U) and W instructions
    // likewise (q < NB*U); slots past those load zeros into the spare 1 KB
    // after the ring, so every wave issues XPW + WPW loads per stage.
    constexpr int CPR = 4 * U;            // 16-byte chunks per row and stage
    constexpr int XB = MT * U, WB = NB * U;
    constexpr int XPW = (XB + 3) / 4, WPW = (WB + 3) / 4;
    constexpr int BPW = XPW + WPW;
    unsigned xoff[XPW], woff[WPW];        // byte offset of the lane's chunk at K = 0
    int xstep[XPW], wstep[WPW];           // step of the stage that the chunk belongs to
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
        const int q = wave + 4 * i;
        const int lin = (q % U) * 64 + lane;
        const int r = lin / CPR, c = (lin % CPR) ^ swz<U>(r);
        const int row = (q / U) * 16 + r;
        xoff[i] = (q < XB && row < Mb) ? (unsigned)row * rowb + (unsigned)c * 16u : kOOB;
        xstep[i] = c >> 2;
    }
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
        const int q = wave + 4 * i;
        const int lin = (q % U) * 64 + lane;
        const int r = lin / CPR, c = (lin % CPR) ^ swz<U>(r);
        const int row = (q / U) * 16 + r;
        woff[i] = (q < WB && row < ncols) ? (unsigned)row * rowb + (unsigned)c * 16u : kOOB;
        wstep[i] = c >> 2;
    }

    // Each column group walks its chunk's stages in a rotated order: the
    // workgroups of one XCD then read different K ranges of x (and of their
    // W rows) at any moment instead of the same lines in lockstep.
    const int rot = j % nstages;
    auto issue = [&](int slot, int stage) {
        // stages past the chunk read zeros (no memory traffic)
        int pos = stage + rot;
        if (pos >= nstages) pos -= nstages;
        if (stage >= nstages) pos = nstages;  // no live step
        const unsigned k0b = (unsigned)(kbeg + pos * U * 32) * 2u;
        unsigned char *base = lds_raw + slot * STAGE;
#pragma unroll
        for (int i = 0; i < XPW; ++i) {
            const int q = wave + 4 * i;
            const bool live = pos * U + xstep[i] < nsteps;
            unsigned char *dst = q < XB ? base + (q / U) * (U * 1024) + (q % U) * 1024
                                        : lds_raw + NS * STAGE;
            lds_load16<kCacheDefault>(xr, dst, live ? xoff[i] + k0b : kOOB);
        }
#pragma unroll
        for (int i = 0; i < WPW; ++i) {
            const int q = wave + 4 * i;
            const bool live = pos * U + wstep[i] < nsteps;
            unsigned char *dst = q < WB ? base + (MT + q / U) * (U * 1024) + (q % U) * 1024
                                        : lds_raw + NS * STAGE;
            lds_load16<kCacheStream>(wr, dst, live ? woff[i] + k0b : kOOB);
        }
    };

    f32x4 acc[MTW][NBW];
#pragma unroll
    for (int a = 0; a < MTW; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment of step u: lane l takes row l % 16, chunk 4*u + l / 16
    const int fr = lane & 15;
    auto compute = [&](int slot) {
        const unsigned char *stg = lds_raw + slot * STAGE;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int fo = fr * (CPR * 16) + (((4 * u + (lane >> 4)) ^ swz<U>(fr)) * 16);
            u32x4 af[MTW], bf[NBW];
#pragma unroll
            for (int a = 0; a < MTW; ++a)
                af[a] = *reinterpret_cast<const u32x4 *>(stg + (wm * MTW + a) * (U * 1024) + fo);
#pragma unroll
            for (int b = 0; b < NBW; ++b)
                bf[b] = *reinterpret_cast<const u32x4 *>(stg + (MT + wn * NBW + b) * (U * 1024) +
                                                         fo);
#pragma unroll
            for (int a = 0; a < MTW; ++a)
#pragma unroll
                for (int b = 0; b < NBW; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, af[a]), __builtin_bit_cast(bf16x8, bf[b]),
                        acc[a][b], 0, 0, 0);
        }
    };

#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, st);
    for (int st = 0; st < nstages; ++st) {
        // nstages is the same for every wave: every wave reaches every barrier
        wait_vmcnt_lds<(NS - 2) * BPW>();
        barrier_nofence();
        // The refill goes to the slot consumed in the previous iteration:
        // every wave's reads of it returned (lgkmcnt(0)) before the barrier,
        // so it is issued before this stage's MFMAs and NS - 1 stages stay
        // in flight while they run.  The wait above still counts NS - 2
        // stages issued after the one it waits for.
        issue((st + NS - 1) % NS, st + NS - 1);
        compute(st % NS);
    }
    wait_vmcnt_lds<0>();  // no load to LDS outlives the loop

    // ---- epilogue.  The output tile goes through the (now idle) ring as
    // fp32 [MT*16][NB*16 + 4], so that global stores cover whole rows:
    // 16-byte stores of the fp32 partials, or 4 bf16 outputs per thread.
    // MFMA 16x16 layout: lane l register i -> row 4*(l/16)+i, column l%16
    // of the tile.  The row stride of NB*16 + 4 floats puts the 4 rows that
    // one LDS store touches in different banks.
    constexpr int TS = NB * 16 + 4;
    float *tile = reinterpret_cast<float *>(lds_raw);
    __syncthreads();  // every wave has left the ring
#pragma unroll
    for (int a = 0; a < MTW; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                tile[((wm * MTW + a) * 16 + (lane >> 4) * 4 + i) * TS + (wn * NBW + b) * 16 +
                     (lane & 15)] = acc[a][b][i];
    __syncthreads();
    const bool vec = (N & 3) == 0;  // 16-byte aligned workspace rows
    const bool coherent = reduce == SKG_REDUCE_LAST;  // partials read by the last arriver
    const PartialsVec pv = partials_vec(ws, M, N, S);
    for (int e = t; e < Mb * C4; e += 256) {
        const int r = e / C4, c = (e % C4) * 4;
        if (c >= ncols) continue;
        const f32x4 v = *reinterpret_cast<const f32x4 *>(tile + r * TS + c);
        const int n = col0 + c;
        const size_t m = (size_t)(row0 + r);
        if (S == 1) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (c + q < ncols)
                    store_out(out, m * N + n + q, bias ? v[q] + bf16_to_f32(bb[q]) : v[q],
                              out_f32);
        } else if (vec && c + 4 <= ncols) {
            put_partial4(ws, ((size_t)s * M + m) * N + n, v, coherent, pv);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (c + q < ncols) put_partial(ws, ((size_t)s * M + m) * N + n + q, v[q], coherent);
        }
    }
    // (the planner gives REDUCE_LAST only with one row block)
    if (S == 1 || reduce != SKG_REDUCE_LAST) return;
    last_arriver_reduce(ws, tickets, bias, out, out_f32, M, N, S, j, col0, ncols, &is_last);
}

namespace {

typedef int (*TiledLaunch)(const SkgPlan &, const void *, const void *, const void *, void *,
                           int, float *, unsigned *, int, int, int, hipStream_t);

template <int MT, int NB, int WM, int NS, int U>
int launch_tiled_t(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                   int out_f32, float *ws, unsigned *tickets, int M, int N, int K,
                   hipStream_t stream) {
    const size_t lds_bytes = tiled_lds_bytes(MT, NB, NS, U);
    // rings above 64 KB: allow the kernel that much dynamic LDS (once per device)
    static std::atomic<unsigned long long> lds_set{0};
    const hipError_t attr = allow_dynamic_lds(
        reinterpret_cast<const void *>(&tiled_kernel<MT, NB, WM, NS, U>), lds_bytes, lds_set);
    if (attr != hipSuccess) return (int)attr;
    hipLaunchKernelGGL((tiled_kernel<MT, NB, WM, NS, U>), dim3(p.grid), dim3(256), lds_bytes,
                       stream, (const uint16_t *)x, (const uint16_t *)W, (const uint16_t *)bias,
                       out, ws, tickets, M, N, K, p.splits, p.k_chunk, p.reduce, out_f32,
                       tiled_row_blocks(M, MT));
    return (int)hipGetLastError();
}

template <int MT, int NB, int WM, int NS, int U>
constexpr TiledLaunch tiled_entry() {
    if constexpr (tiled_built(MT, NB, WM, NS, U))
        return &launch_tiled_t<MT, NB, WM, NS, U>;
    else
        return nullptr;
}

template <int MT, int NB, int WM, int U>
TiledLaunch pick_ns(int NS) {
    switch (NS) {
    case 2: return tiled_entry<MT, NB, WM, 2, U>();
    case 3: return tiled_entry<MT, NB, WM, 3, U>();
    case 4: return tiled_entry<MT, NB, WM, 4, U>();
    case 5: return tiled_entry<MT, NB, WM, 5, U>();
    case 6: return tiled_entry<MT, NB, WM, 6, U>();
    case 8: return tiled_entry<MT, NB, WM, 8, U>();
    default: return nullptr;
    }
}

template <int MT, int NB, int WM>
TiledLaunch pick_u(int NS, int U) {
    return U == 4 ? pick_ns<MT, NB, WM, 4>(NS) : U == 2 ? pick_ns<MT, NB, WM, 2>(NS) : nullptr;
}

template <int MT, int NB>
TiledLaunch pick_wm(int WM, int NS, int U) {
    switch (WM) {
    case 1: return pick_u<MT, NB, 1>(NS, U);
    case 2: return pick_u<MT, NB, 2>(NS, U);
    case 4: return pick_u<MT, NB, 4>(NS, U);
    default: return nullptr;
    }
}

template <int MT>
TiledLaunch pick_nb(int NB, int WM, int NS, int U) {
    switch (NB) {
    case 1: return pick_wm<MT, 1>(WM, NS, U);
    case 2: return pick_wm<MT, 2>(WM, NS, U);
    case 4: return pick_wm<MT, 4>(WM, NS, U);
    case 8: return pick_wm<MT, 8>(WM, NS, U);
    case 16: return pick_wm<MT, 16>(WM, NS, U);
    default: return nullptr;
    }
}

TiledLaunch pick(int MT, int NB, int WM, int NS, int U) {
    switch (MT) {
    case 1: return pick_nb<1>(NB, WM, NS, U);
    case 2: return pick_nb<2>(NB, WM, NS, U);
    case 4: return pick_nb<4>(NB, WM, NS, U);
    case 8: return pick_nb<8>(NB, WM, NS, U);
    default: return nullptr;
    }
}

}  // namespace

int launch_tiled(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                 int out_f32, float *ws, unsigned *tickets, int M, int N, int K,
                 hipStream_t stream) {
    const int U = (p.flags & SKG_FLAG_TILED_WIDE) ? 4 : 2;
    TiledLaunch f = pick(p.m_tiles, p.cols, p.waves_m, p.depth, U);
    if (!f) return (int)hipErrorInvalidConfiguration;
    int rc = f(p, x, W, bias, out, out_f32, ws, tickets, M, N, K, stream);
    if (rc != (int)hipSuccess || p.splits == 1 || p.reduce != SKG_REDUCE_KERNEL) return rc;
    return launch_splitk_reduce(ws, bias, out, out_f32, M, N, p.splits, stream);
}

}  // namespace skg
