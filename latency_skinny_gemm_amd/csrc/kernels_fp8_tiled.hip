// kernels_fp8_tiled.hip -- the LDS-ring tiled kernel for FP8 (OCP e4m3fn)
// operands: per-tensor or MX (e8m0 per 32 K) scales, larger M x N.
//
// Semantics as the other FP8 kernels ("sglang PR #28333" page for the
// per-tensor form, the scale product applied once at the end; "sglang PR
// #34042" page for MX block scaling, applied here by the MFMA itself).
// Structure as the bf16 tiled kernel: workgroup (mb, j, s) owns 16*NB
// columns, the rows of row block mb (MT tiles, rows past M read as zeros)
// and K chunk s; a ring of
// NS LDS stages fed by buffer-to-LDS loads; one vmcnt wait and one barrier
// per stage; the output tile leaves through LDS as whole rows.
//  * a K step is 128 wide (one v_mfma_scale_f32_16x16x128_f8f6f4); a stage
//    holds U steps, so 128*U contiguous bytes of each row;
//  * a block is 16 rows x 128*U bytes, row-major, the 16-byte chunk c of row
//    r at position c ^ swz(r) (the 16 rows of one fragment read land in 16
//    bank groups); a load instruction fills 1 KB with 8/U whole row pieces;
//  * the MFMA operand of lane l (measured on the MI355X): row l % 16, the
//    chunks at K offsets 16g and 64 + 16g of the step (g = l / 16), and the
//    e8m0 byte of the step's 32-element block g;
//  * MX mode loads the e8m0 bytes of the workgroup's whole K chunk once,
//    before the ring, in 16-byte pieces into an area after it (loads
//    complete in issue order, so the wait for the first stage covers
//    them).  Streaming 4 bytes of each row per stage cost 1.7 us at M = 128,
//    K = N = 4096: every such load touched a cache line per two lanes.
//    Rows past M or N read zero codes and a zero exponent, which contribute
//    exactly 0; blocks past the chunk's end take exponent 127 (x 1) against
//    their zero codes.
#include "device_common.h"
#include "internal.h"
#include "lds_limit.h"
#include "splitk_common.h"

namespace skg {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
// chunk swizzle for rows of CPR 16-byte chunks (rows sharing a 256-byte
// bank window get different keys)
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    return (r / (16 / CPR)) & (CPR - 1);
}

}  // namespace

template <int MT, int NB, int WM, int NS, int U, bool MX>
__global__ void __launch_bounds__(256)
    fp8_tiled_kernel(const uint8_t *__restrict__ x, const uint8_t *__restrict__ W,
                     const uint16_t *__restrict__ bias, const float *__restrict__ sx,
                     const float *__restrict__ sw, const uint8_t *__restrict__ xe,
                     const uint8_t *__restrict__ we, void *__restrict__ out,
                     float *__restrict__ ws, unsigned *__restrict__ tickets, int M, int N, int K,
                     int S, int k_chunk, int reduce, int out_f32, int MB) {
    constexpr int WN = 4 / WM;
    constexpr int MTW = MT / WM;
    constexpr int NBW = NB / WN;
    constexpr int CPR = 8 * U;                 // 16-byte chunks per row and stage
    constexpr int BLKB = 16 * 128 * U;         // bytes per block
    constexpr int STAGE = (MT + NB) * BLKB;
    constexpr int XI = MT * 2 * U, WI = NB * 2 * U;   // data instructions per stage
    constexpr int XPW = (XI + 3) / 4, WPW = (WI + 3) / 4;
    constexpr int BPW = XPW + WPW;
    static_assert(MT % WM == 0 && NB % WN == 0, "wave arrangement");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    __shared__ unsigned is_last;
    unsigned char *const pad = lds_raw + NS * STAGE;  // 1 KB that padding loads fill

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
    const unsigned rowb = (unsigned)K;
    const unsigned srow = (unsigned)(K >> 5);
    const Rsrc wr = make_rsrc(W + (size_t)col0 * K, (unsigned)ncols * rowb);
    const Rsrc xr = make_rsrc(x + (size_t)row0 * K, (unsigned)Mb * rowb);
    const Rsrc xer = make_rsrc(xe + (MX ? (size_t)row0 * srow : 0), MX ? (unsigned)Mb * srow : 0u);
    const Rsrc wer = make_rsrc(we + (MX ? (size_t)col0 * srow : 0), MX ? (unsigned)ncols * srow : 0u);
    const int kbeg = s * k_chunk;
    const int nsteps = (min(K, kbeg + k_chunk) - kbeg) >> 7;  // K, k_chunk: multiples of 128
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

    // data loads: instruction q fills part q % (2U) of block q / (2U)
    unsigned xoff[XPW], woff[WPW];
    int xstep[XPW], wstep[WPW];
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
        const int q = wave + 4 * i;
        const int lin = (q % (2 * U)) * 64 + lane;
        const int r = lin / CPR, c = (lin % CPR) ^ swz<CPR>(r);
        const int row = (q / (2 * U)) * 16 + r;
        xoff[i] = (q < XI && row < Mb) ? (unsigned)row * rowb + (unsigned)c * 16u : kOOB;
        xstep[i] = c >> 3;
    }
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
        const int q = wave + 4 * i;
        const int lin = (q % (2 * U)) * 64 + lane;
        const int r = lin / CPR, c = (lin % CPR) ^ swz<CPR>(r);
        const int row = (q / (2 * U)) * 16 + r;
        woff[i] = (q < WI && row < ncols) ? (unsigned)row * rowb + (unsigned)c * 16u : kOOB;
        wstep[i] = c >> 3;
    }
    // MX: the chunk's scale bytes.  Slot q (16 bytes) of an area is piece
    // q % (SR / 16) of row q / (SR / 16); the pieces past a row's k_chunk / 32
    // bytes (the row's padding) load zeros.  Each area is a whole number of
    // KB, so no instruction writes past its own.
    const int kch = min(K, kbeg + k_chunk) - kbeg;  // this chunk's K
    const int SR = fp8_tiled_scale_stride(k_chunk);
    unsigned char *const xsa = pad + 1024;
    unsigned char *const wsa = xsa + fp8_tiled_scale_area(MT * 16, k_chunk);
    if constexpr (MX) {
        const int spr = SR / 16;                  // slots per row
        const int live = (k_chunk / 32 + 15) / 16;  // slots of a row that hold bytes
        const unsigned kb = (unsigned)kbeg / 32u;
        auto load_area = [&](Rsrc r, unsigned char *area, int rows, int real_rows) {
            const int slots = rows * spr;
            for (int b = wave * 64; b < slots; b += 256) {  // wave-uniform trip count
                const int q = b + lane, row = q / spr, c = q - row * spr;
                const bool ok = q < slots && c < live && row < real_rows;
                lds_load16<kCacheDefault>(r, area + b * 16,
                                          ok ? (unsigned)row * srow + kb + 16u * (unsigned)c : kOOB);
            }
        };
        load_area(xer, xsa, MT * 16, Mb);
        load_area(wer, wsa, NB * 16, ncols);
    }

    const int rot = j % nstages;
    auto issue = [&](int slot, int stage) {
        int pos = stage + rot;
        if (pos >= nstages) pos -= nstages;
        if (stage >= nstages) pos = nstages;  // no live step: zero-byte loads
        const unsigned k0 = (unsigned)(kbeg + pos * U * 128);
        unsigned char *base = lds_raw + slot * STAGE;
#pragma unroll
        for (int i = 0; i < XPW; ++i) {
            const int q = wave + 4 * i;
            const bool live = pos * U + xstep[i] < nsteps;
            unsigned char *dst = q < XI ? base + (q / (2 * U)) * BLKB + (q % (2 * U)) * 1024 : pad;
            lds_load16<kCacheDefault>(xr, dst, live ? xoff[i] + k0 : kOOB);
        }
#pragma unroll
        for (int i = 0; i < WPW; ++i) {
            const int q = wave + 4 * i;
            const bool live = pos * U + wstep[i] < nsteps;
            unsigned char *dst =
                q < WI ? base + (MT + q / (2 * U)) * BLKB + (q % (2 * U)) * 1024 : pad;
            lds_load16<kCacheStream>(wr, dst, live ? woff[i] + k0 : kOOB);
        }
    };

    f32x4 acc[MTW][NBW];
#pragma unroll
    for (int a = 0; a < MTW; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int fr = lane & 15, fg = lane >> 4;
    auto compute = [&](int slot, int pos) {
        const unsigned char *stg = lds_raw + slot * STAGE;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int o0 = fr * (CPR * 16) + (((8 * u + fg) ^ swz<CPR>(fr)) * 16);
            const int o1 = fr * (CPR * 16) + (((8 * u + 4 + fg) ^ swz<CPR>(fr)) * 16);
            i32x8 af[MTW], bf[NBW];
            int as[MTW], bs[NBW];
            // this lane's 32-element block of the chunk, and whether it lies
            // inside the chunk's K
            const int blk32 = 4 * (pos * U + u) + fg;
            const bool sl = 32 * blk32 < kch;
            const int sc = sl ? blk32 : 0;  // every scale read stays inside its row
#pragma unroll
            for (int a = 0; a < MTW; ++a) {
                const unsigned char *blk = stg + (wm * MTW + a) * BLKB;
                const u32x4 p0 = *reinterpret_cast<const u32x4 *>(blk + o0);
                const u32x4 p1 = *reinterpret_cast<const u32x4 *>(blk + o1);
                af[a] = i32x8{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w,
                              (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
                if constexpr (MX) {
                    const int v = xsa[((wm * MTW + a) * 16 + fr) * SR + sc];  // always in range
                    as[a] = sl ? v : 127;
                } else {
                    as[a] = 127;
                }
            }
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const unsigned char *blk = stg + (MT + wn * NBW + b) * BLKB;
                const u32x4 p0 = *reinterpret_cast<const u32x4 *>(blk + o0);
                const u32x4 p1 = *reinterpret_cast<const u32x4 *>(blk + o1);
                bf[b] = i32x8{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w,
                              (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
                if constexpr (MX) {
                    const int v = wsa[((wn * NBW + b) * 16 + fr) * SR + sc];
                    bs[b] = sl ? v : 127;
                } else {
                    bs[b] = 127;
                }
            }
#pragma unroll
            for (int a = 0; a < MTW; ++a)
#pragma unroll
                for (int b = 0; b < NBW; ++b)
                    // formats 0/0: e4m3 on both sides; scale byte 0 of each lane
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        af[a], bf[b], acc[a][b], 0, 0, 0, as[a], 0, bs[b]);
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
        const int cpos = st + rot < nstages ? st + rot : st + rot - nstages;  // as issue()
        compute(st % NS, cpos);
    }
    wait_vmcnt_lds<0>();  // no load to LDS outlives the loop

    // ---- epilogue through LDS, as in the bf16 tiled kernel; per-tensor
    // mode applies sx*sw once (here when S == 1, else in the reduction)
    constexpr int TS = NB * 16 + 4;
    float *tile = reinterpret_cast<float *>(lds_raw);
    __syncthreads();
#pragma unroll
    for (int a = 0; a < MTW; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                tile[((wm * MTW + a) * 16 + fg * 4 + i) * TS + (wn * NBW + b) * 16 + fr] =
                    acc[a][b][i];
    __syncthreads();
    const float scale = MX ? 1.0f : sx[0] * sw[0];
    const bool vec = (N & 3) == 0;
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
                if (c + q < ncols) {
                    float o = MX ? v[q] : v[q] * scale;
                    if (bias) o += bf16_to_f32(bb[q]);
                    store_out(out, m * N + n + q, o, out_f32);
                }
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
    last_arriver_reduce(ws, tickets, bias, out, out_f32, M, N, S, j, col0, ncols, &is_last, !MX,
                        scale);
}

namespace {

typedef int (*Fp8TiledLaunch)(const SkgPlan &, const Fp8Args &, float *, unsigned *, int, int,
                              int, hipStream_t);

template <int MT, int NB, int WM, int NS, int U, bool MX>
int launch_fp8_tiled_t(const SkgPlan &p, const Fp8Args &a, float *ws, unsigned *tickets, int M,
                       int N, int K, hipStream_t stream) {
    // MX adds the chunk's scale bytes (the planner checked the total); the
    // limit is raised once per device to the most any chunk may take
    const size_t lds_bytes = MX ? fp8_tiled_mx_lds_bytes(MT, NB, NS, U, p.k_chunk)
                                : fp8_tiled_lds_bytes(MT, NB, NS, U);
    if (lds_bytes > (size_t)kTiledMaxLds) return (int)hipErrorInvalidConfiguration;
    static std::atomic<unsigned long long> lds_set{0};  // devices whose limit is set
    const hipError_t attr = allow_dynamic_lds(
        reinterpret_cast<const void *>(&fp8_tiled_kernel<MT, NB, WM, NS, U, MX>),
        MX ? (size_t)kTiledMaxLds : lds_bytes, lds_set);
    if (attr != hipSuccess) return (int)attr;
    hipLaunchKernelGGL((fp8_tiled_kernel<MT, NB, WM, NS, U, MX>), dim3(p.grid), dim3(256),
                       lds_bytes, stream, (const uint8_t *)a.x, (const uint8_t *)a.W,
                       (const uint16_t *)a.bias, a.sx, a.sw, a.xe, a.we, a.out, ws, tickets, M, N,
                       K, p.splits, p.k_chunk, p.reduce, a.out_f32, tiled_row_blocks(M, MT));
    return (int)hipGetLastError();
}

template <int MT, int NB, int WM, int NS, int U, bool MX>
constexpr Fp8TiledLaunch fp8_tiled_entry() {
    if constexpr (fp8_tiled_built(MT, NB, WM, NS, U))
        return &launch_fp8_tiled_t<MT, NB, WM, NS, U, MX>;
    else
        return nullptr;
}

template <int MT, int NB, int WM, int U, bool MX>
Fp8TiledLaunch pick_ns(int NS) {
    switch (NS) {
    case 2: return fp8_tiled_entry<MT, NB, WM, 2, U, MX>();
    case 3: return fp8_tiled_entry<MT, NB, WM, 3, U, MX>();
    case 4: return fp8_tiled_entry<MT, NB, WM, 4, U, MX>();
    case 5: return fp8_tiled_entry<MT, NB, WM, 5, U, MX>();
    case 6: return fp8_tiled_entry<MT, NB, WM, 6, U, MX>();
    case 8: return fp8_tiled_entry<MT, NB, WM, 8, U, MX>();
    default: return nullptr;
    }
}

template <int MT, int NB, int WM, bool MX>
Fp8TiledLaunch pick_u(int NS, int U) {
    return U == 2 ? pick_ns<MT, NB, WM, 2, MX>(NS) : U == 1 ? pick_ns<MT, NB, WM, 1, MX>(NS)
                                                            : nullptr;
}

template <int MT, int NB, bool MX>
Fp8TiledLaunch pick_wm(int WM, int NS, int U) {
    switch (WM) {
    case 1: return pick_u<MT, NB, 1, MX>(NS, U);
    case 2: return pick_u<MT, NB, 2, MX>(NS, U);
    case 4: return pick_u<MT, NB, 4, MX>(NS, U);
    default: return nullptr;
    }
}

template <int MT, bool MX>
Fp8TiledLaunch pick_nb(int NB, int WM, int NS, int U) {
    switch (NB) {
    case 1: return pick_wm<MT, 1, MX>(WM, NS, U);
    case 2: return pick_wm<MT, 2, MX>(WM, NS, U);
    case 4: return pick_wm<MT, 4, MX>(WM, NS, U);
    case 8: return pick_wm<MT, 8, MX>(WM, NS, U);
    case 16: return pick_wm<MT, 16, MX>(WM, NS, U);
    default: return nullptr;
    }
}

template <bool MX>
Fp8TiledLaunch pick(int MT, int NB, int WM, int NS, int U) {
    switch (MT) {
    case 1: return pick_nb<1, MX>(NB, WM, NS, U);
    case 2: return pick_nb<2, MX>(NB, WM, NS, U);
    case 4: return pick_nb<4, MX>(NB, WM, NS, U);
    case 8: return pick_nb<8, MX>(NB, WM, NS, U);
    default: return nullptr;
    }
}

}  // namespace

int launch_fp8_tiled(const SkgPlan &p, const Fp8Args &a, float *ws, unsigned *tickets, int M,
                     int N, int K, hipStream_t stream) {
    const bool mx = a.mode == SKG_FP8_MX32;
    const int U = (p.flags & SKG_FLAG_TILED_WIDE) ? 2 : 1;
    Fp8TiledLaunch f = mx ? pick<true>(p.m_tiles, p.cols, p.waves_m, p.depth, U)
                          : pick<false>(p.m_tiles, p.cols, p.waves_m, p.depth, U);
    if (!f) return (int)hipErrorInvalidConfiguration;
    int rc = f(p, a, ws, tickets, M, N, K, stream);
    if (rc != (int)hipSuccess || p.splits == 1 || p.reduce != SKG_REDUCE_KERNEL) return rc;
    return launch_splitk_reduce(ws, a.bias, a.out, a.out_f32, M, N, p.splits, stream,
                                mx ? nullptr : a.sx, mx ? nullptr : a.sw);
}

}  // namespace skg
