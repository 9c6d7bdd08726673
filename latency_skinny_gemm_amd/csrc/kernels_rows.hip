// kernels_rows.hip -- MFMA kernel for M <= 64 whose x and W stream through an
// LDS ring as whole row segments, K split over the waves of one workgroup.
//
// The "vllm PR #42562" page's split-K kernel stages A and B tiles through
// shared memory and pads M to the MMA tile; its K split is over blocks,
// which needs a reduction across workgroups.  On gfx950 the dense decode
// linear at small M can do without that:
//  * workgroup b owns R consecutive output columns (R = 16, one MFMA tile
//    width, or 8, 10, 12 to spread a smaller N over more CUs) and the whole
//    K, so N = 4096 gives 256 workgroups and nothing is reduced across
//    workgroups;
//  * a stage is KS = 512 (or 256) K elements: each of the R W rows and of
//    the M x rows contributes one segment of 2*KS bytes, and one
//    buffer-to-LDS load moves 1 KB (lane p: 16 bytes), so every load reads
//    1 KB of one row or 512 bytes of each of two rows.  (Loading W straight
//    into MFMA operand order would read 16 rows x 64 bytes per instruction,
//    which streams about 30 % slower on this GPU; pieces of 128 bytes and
//    up stream alike.)
//  * LDS rows are 2*KS bytes; inside row r the 16-byte chunk c sits at
//    position c ^ (r mod 16) (the load's lane p fetches the chunk that
//    belongs at position p), so the 16 rows that one MFMA fragment read
//    touches hit 16 different 16-byte bank groups: conflict-free
//    ds_read_b128;
//  * NS stages form a ring (the discipline of the tiled kernel: stage i+NS-1
//    refills the slot of stage i-1 after the barrier that precedes stage
//    i's products; each wave waits for its own loads by counting them);
//  * a stage has KS/32 MFMA steps; wave w of NW takes steps w, w+NW, ...
//    and keeps one 16x16 fp32 partial tile per 16 rows of x; the NW
//    partials are summed in wave order through LDS at the end, bias added
//    in fp32, one rounding.
// Rows of x past M (up to MP, the rows the kernel is built for) load zeros
// and are never stored.  A fragment lane whose row is past M (x) or past R
// (W) reads a real row (row mod M, mod R): it only feeds outputs that are
// never stored.  W rows past N and K past the end load zeros (range check).
// Every order is fixed: the result is bitwise reproducible for a plan.
#include <atomic>

#include "device_common.h"
#include "internal.h"
#include "lds_limit.h"

namespace skg {

template <int MP, int NW, int NS, int R, int KS>
__global__ void __launch_bounds__(NW * 64)
    rows_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
                const uint16_t *__restrict__ bias, void *__restrict__ out, int M, int N, int K,
                int out_f32) {
    constexpr int SB = 2 * KS;                  // bytes of a stage row
    constexpr int CPR = SB / 16;                // 16-byte chunks per row
    constexpr int RPL = rows_per_load(KS);      // rows per load instruction
    constexpr int XR = (MP + RPL - 1) / RPL * RPL;
    constexpr int WL = R / RPL, XL = XR / RPL;  // load instructions per stage
    constexpr int WPW = rows_w_loads(NW, R, KS), XPW = rows_x_loads(MP, NW, KS);
    constexpr int LPW = WPW + XPW;              // loads per wave per stage
    constexpr int STAGE = rows_stage_bytes(MP, R, KS);
    constexpr int JUNK = (R + XR) * SB;         // the KB that takes the padding loads
    constexpr int MT = (MP + 15) / 16;          // 16-row tiles of x
    constexpr int STEPS = KS / 32;              // MFMA steps per stage
    static_assert(STEPS % NW == 0, "whole steps per wave");
    static_assert(NW * MT * 16 * 17 * 4 <= NS * STAGE, "the epilogue's tiles fit the ring");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int n0 = blockIdx.x * R;
    const int ncols = min(R, N - n0);
    // The bias of the epilogue's first column for thread t, n0 + t % R,
    // loaded ahead of the ring (the only column it stores when NW * 64 is a
    // multiple of R or M * R <= NW * 64).  Without a bias no load is issued.
    const Rsrc br = bias_rsrc(bias, N);
    unsigned bb = 0;
    if (bias) bb = load_bias_bits(br, n0 + t % R, t % R < ncols);
    const unsigned rowb = (unsigned)K * 2u;
    const Rsrc wr = make_rsrc(W + (size_t)n0 * K, (unsigned)ncols * rowb);
    const Rsrc xr = make_rsrc(x, (unsigned)M * rowb);
    const int nstages = (K + KS - 1) / KS;

    // Load instruction j of a block: lane p fills position p % CPR of row
    // j*RPL + p / CPR, i.e. that row's chunk (p % CPR) ^ (LDS row mod 16).
    // Wave w issues W instructions w + NW*i (i < WPW) and x instructions
    // likewise; those past the block load zeros into the padding KB, so that
    // every wave issues LPW loads per stage.
    const int lrow = lane / CPR, lpos = lane % CPR;
    unsigned wsrc[WPW], xsrc[XPW];
    int wdst[WPW], xdst[XPW], wk[WPW], xk[XPW];
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
        const int j = wave + NW * i;
        const int r = j * RPL + lrow;
        const int c = lpos ^ (r & 15);
        wk[i] = 8 * c;
        wdst[i] = j < WL ? j * RPL * SB : JUNK;
        wsrc[i] = j < WL && r < ncols ? (unsigned)r * rowb + 16u * (unsigned)c : kOOB;
    }
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
        const int j = wave + NW * i;
        const int m = j * RPL + lrow;
        const int c = lpos ^ ((R + m) & 15);
        xk[i] = 8 * c;
        xdst[i] = j < XL ? (R + j * RPL) * SB : JUNK;
        xsrc[i] = j < XL && m < M ? (unsigned)m * rowb + 16u * (unsigned)c : kOOB;
    }

    // Workgroups walk the K stages in a rotated order, so those that share
    // an XCD do not read the same x lines in lockstep.
    const int rot = blockIdx.x % nstages;
    auto issue = [&](int slot, int stage) {
        int pos = stage + rot;
        if (pos >= nstages) pos -= nstages;
        // stages past the end load zeros (no memory traffic); so do the
        // 16-byte pieces at or past K
        const int k0 = stage < nstages ? pos * KS : K;
        const unsigned kb = (unsigned)k0 * 2u;
        unsigned char *base = lds + slot * STAGE;
#pragma unroll
        for (int i = 0; i < WPW; ++i)
            lds_load16<kCacheStream>(wr, base + wdst[i],
                                     wsrc[i] != kOOB && k0 + wk[i] < K ? wsrc[i] + kb : kOOB);
#pragma unroll
        for (int i = 0; i < XPW; ++i)
            lds_load16<kCacheDefault>(xr, base + xdst[i],
                                      xsrc[i] != kOOB && k0 + xk[i] < K ? xsrc[i] + kb : kOOB);
    };

    // fragments: lane l reads row l % 16 (x: of tile a, W: of the R rows,
    // wrapped) at 16-byte chunk 4u + l/16 of step u
    const int fr = lane & 15, g = lane >> 4;
    const int rb = fr % R;
    int abase[MT], akey[MT];
#pragma unroll
    for (int a = 0; a < MT; ++a) {
        const int ra = R + (16 * a + fr) % M;
        abase[a] = ra * SB;
        akey[a] = ra & 15;
    }
    f32x4 acc[MT];
#pragma unroll
    for (int a = 0; a < MT; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int slot) {
        const unsigned char *stg = lds + slot * STAGE;
#pragma unroll
        for (int q = 0; q < STEPS / NW; ++q) {
            const int kc = 4 * (wave + NW * q) + g;
            const u32x4 b = *reinterpret_cast<const u32x4 *>(stg + rb * SB + 16 * (kc ^ (rb & 15)));
#pragma unroll
            for (int a = 0; a < MT; ++a) {
                const u32x4 av =
                    *reinterpret_cast<const u32x4 *>(stg + abase[a] + 16 * (kc ^ akey[a]));
                acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                                 __builtin_bit_cast(bf16x8, b),
                                                                 acc[a], 0, 0, 0);
            }
        }
    };

#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, st);
    for (int st = 0; st < nstages; ++st) {
        // nstages is the same for every wave: every wave reaches every barrier
        wait_vmcnt_lds<(NS - 2) * LPW>();
        barrier_nofence();
        // refill the slot read in the previous iteration (every wave's reads
        // of it returned before the barrier); NS - 1 stages stay in flight
        issue((st + NS - 1) % NS, st + NS - 1);
        compute(st % NS);
    }
    wait_vmcnt_lds<0>();  // no load to LDS outlives the loop

    // ---- epilogue: the NW partial tiles through the idle ring, summed in
    // wave order.  MFMA 16x16 layout: lane l register i -> row 4*(l/16)+i,
    // column l%16.  Row stride 17 floats.
    float *red = reinterpret_cast<float *>(lds);
    __syncthreads();  // every wave has left the ring
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[((wave * MT + a) * 16 + g * 4 + i) * 17 + fr] = acc[a][i];
    __syncthreads();
    for (int e = t; e < M * R; e += NW * 64) {
        const int m = e / R, c = e - (e / R) * R;
        if (c >= ncols) continue;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += red[((w * MT + m / 16) * 16 + m % 16) * 17 + c];
        const int n = n0 + c;
        const unsigned b = ((NW * 64) % R == 0 || e == t) ? bb : load_bias_bits(br, n);
        if (bias) s += bf16_to_f32(b);
        store_out(out, (size_t)m * N + n, s, out_f32);
    }
}

namespace {

typedef int (*RowsLaunch)(const SkgPlan &, const void *, const void *, const void *, void *, int,
                          int, int, int, hipStream_t);

template <int MP, int NW, int NS, int R, int KS>
int launch_rows_t(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                  int out_f32, int M, int N, int K, hipStream_t stream) {
    const size_t lds = (size_t)rows_lds_bytes(MP, NS, R, KS);
    static std::atomic<unsigned long long> lds_set{0};
    if (lds > 64 * 1024) {
        const hipError_t attr = allow_dynamic_lds(
            reinterpret_cast<const void *>(&rows_kernel<MP, NW, NS, R, KS>), lds, lds_set);
        if (attr != hipSuccess) return (int)attr;
    }
    hipLaunchKernelGGL((rows_kernel<MP, NW, NS, R, KS>), dim3(p.grid), dim3(NW * 64), lds, stream,
                       (const uint16_t *)x, (const uint16_t *)W, (const uint16_t *)bias, out, M, N,
                       K, out_f32);
    return (int)hipGetLastError();
}

template <int MP, int NW, int NS, int R, int KS>
constexpr RowsLaunch rows_entry() {
    if constexpr (rows_built(MP, NW, NS, R, KS))
        return &launch_rows_t<MP, NW, NS, R, KS>;
    else
        return nullptr;
}

template <int MP, int NW, int R, int KS>
RowsLaunch pick_ns(int NS) {
    switch (NS) {
    case 3: return rows_entry<MP, NW, 3, R, KS>();
    case 4: return rows_entry<MP, NW, 4, R, KS>();
    case 5: return rows_entry<MP, NW, 5, R, KS>();
    case 6: return rows_entry<MP, NW, 6, R, KS>();
    default: return nullptr;
    }
}

template <int MP, int NW, int KS>
RowsLaunch pick_r(int NS, int R) {
    switch (R) {
    case 8: return pick_ns<MP, NW, 8, KS>(NS);
    case 10: return pick_ns<MP, NW, 10, KS>(NS);
    case 12: return pick_ns<MP, NW, 12, KS>(NS);
    case 16: return pick_ns<MP, NW, 16, KS>(NS);
    default: return nullptr;
    }
}

template <int MP, int KS>
RowsLaunch pick_shape(int NW, int NS, int R) {
    if (NW == 4) return pick_r<MP, 4, KS>(NS, R);
    if (NW == 8) return pick_r<MP, 8, KS>(NS, R);
    return nullptr;
}

template <int MP>
RowsLaunch pick_ks(int NW, int NS, int R, int KS) {
    if (KS == 512) return pick_shape<MP, 512>(NW, NS, R);
    if (KS == 256) return pick_shape<MP, 256>(NW, NS, R);
    return nullptr;
}

RowsLaunch pick(int MP, int NW, int NS, int R, int KS) {
    switch (MP) {
    case 1: return pick_ks<1>(NW, NS, R, KS);
    case 2: return pick_ks<2>(NW, NS, R, KS);
    case 3: return pick_ks<3>(NW, NS, R, KS);
    case 4: return pick_ks<4>(NW, NS, R, KS);
    case 5: return pick_ks<5>(NW, NS, R, KS);
    case 6: return pick_ks<6>(NW, NS, R, KS);
    case 7: return pick_ks<7>(NW, NS, R, KS);
    case 8: return pick_ks<8>(NW, NS, R, KS);
    case 9: return pick_ks<9>(NW, NS, R, KS);
    case 10: return pick_ks<10>(NW, NS, R, KS);
    case 11: return pick_ks<11>(NW, NS, R, KS);
    case 12: return pick_ks<12>(NW, NS, R, KS);
    case 13: return pick_ks<13>(NW, NS, R, KS);
    case 14: return pick_ks<14>(NW, NS, R, KS);
    case 15: return pick_ks<15>(NW, NS, R, KS);
    case 16: return pick_ks<16>(NW, NS, R, KS);
    case 24: return pick_ks<24>(NW, NS, R, KS);
    case 32: return pick_ks<32>(NW, NS, R, KS);
    case 48: return pick_ks<48>(NW, NS, R, KS);
    case 64: return pick_ks<64>(NW, NS, R, KS);
    default: return nullptr;
    }
}

}  // namespace

int launch_rows(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                int out_f32, int M, int N, int K, hipStream_t stream) {
    const int KS = (p.flags & SKG_FLAG_ROWS_HALF) ? 256 : 512;
    RowsLaunch f = pick(rows_mp(M), p.threads / 64, p.depth, p.cols, KS);
    if (!f) return (int)hipErrorInvalidConfiguration;
    return f(p, x, W, bias, out, out_f32, M, N, K, stream);
}

}  // namespace skg
