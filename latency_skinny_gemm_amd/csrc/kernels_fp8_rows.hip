// kernels_fp8_rows.hip -- the whole-row MFMA ring kernel for FP8 e4m3 (per-
// tensor or MX scales), M <= 32.
//
// The bf16 ring kernel (kernels_rows.hip) with 128-wide K steps on
// v_mfma_scale_f32_16x16x128_f8f6f4 ("sglang PR #28333" page for the
// per-tensor scales, "sglang PR #34042" page for the MX block scales):
//  * workgroup b owns R = 16 (or 8) output columns and the whole K; its NW
//    waves take the MFMA steps of each stage round-robin and keep one 16x16
//    fp32 tile per 16 rows of x; the tiles are summed in wave order at the
//    end;
//  * a stage is SB = 1024 (or 512) K elements, i.e. SB bytes of every W and
//    x row, one LDS row each, moved by 1 KB buffer-to-LDS loads (one whole
//    row segment, or two half ones) with the XOR chunk swizzle of the bf16
//    kernel;
//  * a lane's operand for step u is the 16-byte chunks 8u + g and 8u + 4 + g
//    of its row (g = lane / 16), the layout measured for this instruction;
//  * MX: the stage's e8m0 bytes (SB / 32 per row) stream into the same
//    ring, one 1 KB load per operand block, issued by waves 0..; a wave
//    without one loads zeros into the spare KB, so every wave issues the
//    same count.  Lane (row r, group g) supplies the byte of block 4u + g
//    of row r.  K must then be a multiple of 512: a scale chunk of 16 bytes
//    never straddles the end of a row's scales;
//  * per-tensor: the instruction's scales are 2^0 and sx * sw multiplies
//    the wave-ordered sum once, then bias is added, one rounding.
// Rows of x past M (up to MP, a power of two) load zeros and are never
// stored; fragment lanes past M or R read a real row, which only feeds
// outputs that are never stored.  W rows past N and K past the end load
// zeros (range check), so do their scale bytes (2^-127 times zero).
#include <atomic>

#include "device_common.h"
#include "internal.h"
#include "lds_limit.h"

namespace skg {

namespace {
typedef int i32x8 __attribute__((ext_vector_type(8)));
}  // namespace

template <int MP, int NW, int NS, int R, int SB, bool MX>
__global__ void __launch_bounds__(NW * 64)
    fp8_rows_kernel(const uint8_t *__restrict__ x, const uint8_t *__restrict__ W,
                    const uint16_t *__restrict__ bias, const float *__restrict__ sx,
                    const float *__restrict__ sw, const uint8_t *__restrict__ xe,
                    const uint8_t *__restrict__ we, void *__restrict__ out, int M, int N, int K,
                    int out_f32) {
    constexpr int CPR = SB / 16;                   // 16-byte chunks per row
    constexpr int RPL = 1024 / SB;                 // rows per load instruction
    constexpr int XR = (MP + RPL - 1) / RPL * RPL;
    constexpr int WL = R / RPL, XL = XR / RPL;     // code loads per stage
    constexpr int WPW = (WL + NW - 1) / NW, XPW = (XL + NW - 1) / NW;
    constexpr int SPR = SB / 32;                   // scale bytes per row per stage
    constexpr int CS = SPR / 16;                   // 16-byte scale chunks per row
    constexpr int RPS = 64 / CS;                   // scale rows per load
    constexpr int WSL = (R + RPS - 1) / RPS, XSL = (XR + RPS - 1) / RPS;
    static_assert(!MX || WSL + XSL <= NW, "one scale load per wave at most");
    constexpr int LPW = WPW + XPW + (MX ? 1 : 0);  // loads per wave per stage
    constexpr int CODES = (R + XR) * SB;           // code rows of a stage
    constexpr int JUNK = CODES;                    // the KB that takes padding loads
    constexpr int WSC = CODES + 1024;              // W scale block (WSL KB)
    constexpr int XSC = WSC + WSL * 1024;          // x scale block (XSL KB)
    constexpr int STAGE = fp8_rows_stage_bytes(MP, R, SB, MX);
    constexpr int MT = (MP + 15) / 16;
    constexpr int STEPS = SB / 128;                // MFMA steps per stage
    static_assert(STEPS % NW == 0, "whole steps per wave");
    static_assert(NW * MT * 16 * 17 * 4 <= NS * STAGE, "the epilogue's tiles fit the ring");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int n0 = blockIdx.x * R;
    const int ncols = min(R, N - n0);
    // The epilogue's bias, loaded ahead of the ring: column n0 + t % R is
    // the only one thread t stores (NW * 64 is a multiple of R).  Without a
    // bias no load is issued.
    static_assert((NW * 64) % R == 0, "a thread keeps its column");
    unsigned bb = 0;
    if (bias) bb = load_bias_bits(bias_rsrc(bias, N), n0 + t % R, t % R < ncols);
    const unsigned rowb = (unsigned)K;
    const Rsrc wr = make_rsrc(W + (size_t)n0 * K, (unsigned)ncols * rowb);
    const Rsrc xr = make_rsrc(x, (unsigned)M * rowb);
    const int nstages = (K + SB - 1) / SB;

    // code loads: lane p fills position p % CPR of row j*RPL + p / CPR with
    // that row's chunk (p % CPR) ^ (LDS row mod 16)
    const int lrow = lane / CPR, lpos = lane % CPR;
    unsigned wsrc[WPW], xsrc[XPW];
    int wdst[WPW], xdst[XPW], wk[WPW], xk[XPW];
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
        const int j = wave + NW * i;
        const int r = j * RPL + lrow;
        const int c = lpos ^ (r & 15);
        wk[i] = 16 * c;
        wdst[i] = j < WL ? j * RPL * SB : JUNK;
        wsrc[i] = j < WL && r < ncols ? (unsigned)r * rowb + 16u * (unsigned)c : kOOB;
    }
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
        const int j = wave + NW * i;
        const int m = j * RPL + lrow;
        const int c = lpos ^ ((R + m) & 15);
        xk[i] = 16 * c;
        xdst[i] = j < XL ? (R + j * RPL) * SB : JUNK;
        xsrc[i] = j < XL && m < M ? (unsigned)m * rowb + 16u * (unsigned)c : kOOB;
    }
    // scale loads (MX): wave w < WSL moves W scale rows RPS*w.., waves
    // WSL.. the x ones; lane p: row p / CS, 16-byte chunk p % CS
    const unsigned srow = (unsigned)K / 32u;
    Rsrc sr = make_rsrc(we, 0);
    unsigned ssrc = kOOB;
    int sdst = JUNK, sk = 0;
    if constexpr (MX) {
        const int srl = lane / CS, sc = lane % CS;
        sk = 16 * sc;
        if (wave < WSL) {
            const int r = wave * RPS + srl;
            sr = make_rsrc(we + (size_t)n0 * srow, (unsigned)ncols * srow);
            ssrc = r < ncols ? (unsigned)r * srow + 16u * (unsigned)sc : kOOB;
            sdst = WSC + wave * 1024;
        } else if (wave < WSL + XSL) {
            const int m = (wave - WSL) * RPS + srl;
            sr = make_rsrc(xe, (unsigned)M * srow);
            ssrc = m < M ? (unsigned)m * srow + 16u * (unsigned)sc : kOOB;
            sdst = XSC + (wave - WSL) * 1024;
        }
    }

    const int rot = blockIdx.x % nstages;
    auto issue = [&](int slot, int stage) {
        int pos = stage + rot;
        if (pos >= nstages) pos -= nstages;
        // stages past the end load zeros (no memory traffic); so do the
        // 16-byte pieces at or past K
        const int k0 = stage < nstages ? pos * SB : K;
        unsigned char *base = lds + slot * STAGE;
#pragma unroll
        for (int i = 0; i < WPW; ++i)
            lds_load16<kCacheStream>(wr, base + wdst[i],
                                     wsrc[i] != kOOB && k0 + wk[i] < K ? wsrc[i] + k0 : kOOB);
#pragma unroll
        for (int i = 0; i < XPW; ++i)
            lds_load16<kCacheDefault>(xr, base + xdst[i],
                                      xsrc[i] != kOOB && k0 + xk[i] < K ? xsrc[i] + k0 : kOOB);
        if constexpr (MX) {
            // the stage's scale bytes start at k0 / 32; a chunk lies wholly
            // before or wholly past the row's K / 32 (K % 512 == 0)
            const unsigned kb = (unsigned)k0 / 32u;
            lds_load16<kCacheDefault>(sr, base + sdst,
                                      ssrc != kOOB && kb + (unsigned)sk < srow ? ssrc + kb : kOOB);
        }
    };

    // fragments: lane l reads row l % 16 (x: of tile a, W: of the R rows,
    // wrapped), chunks 8u + g and 8u + 4 + g of step u
    const int fr = lane & 15, g = lane >> 4;
    const int rb = fr % R;
    int abase[MT], akey[MT], asrow[MT];
#pragma unroll
    for (int a = 0; a < MT; ++a) {
        const int m = (16 * a + fr) % M;
        abase[a] = (R + m) * SB;
        akey[a] = (R + m) & 15;
        asrow[a] = m * SPR;
    }
    f32x4 acc[MT];
#pragma unroll
    for (int a = 0; a < MT; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto frag = [&](const unsigned char *row, int key, int u) {
        const u32x4 p0 = *reinterpret_cast<const u32x4 *>(row + 16 * ((8 * u + g) ^ key));
        const u32x4 p1 = *reinterpret_cast<const u32x4 *>(row + 16 * ((8 * u + 4 + g) ^ key));
        return i32x8{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w,
                     (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
    };
    auto compute = [&](int slot) {
        const unsigned char *stg = lds + slot * STAGE;
#pragma unroll
        for (int q = 0; q < STEPS / NW; ++q) {
            const int u = wave + NW * q;
            const i32x8 b = frag(stg + rb * SB, rb & 15, u);
            const int bs = MX ? (int)stg[WSC + rb * SPR + 4 * u + g] : 127;
#pragma unroll
            for (int a = 0; a < MT; ++a) {
                const i32x8 av = frag(stg + abase[a], akey[a], u);
                const int as = MX ? (int)stg[XSC + asrow[a] + 4 * u + g] : 127;
                // formats 0/0: e4m3 on both sides; scale byte 0 of each lane
                acc[a] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, acc[a], 0, 0,
                                                                          0, as, 0, bs);
            }
        }
    };

#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, st);
    for (int st = 0; st < nstages; ++st) {
        // nstages is the same for every wave: every wave reaches every barrier
        wait_vmcnt_lds<(NS - 2) * LPW>();
        barrier_nofence();
        issue((st + NS - 1) % NS, st + NS - 1);
        compute(st % NS);
    }
    wait_vmcnt_lds<0>();  // no load to LDS outlives the loop

    // ---- epilogue: the NW partial tiles through the idle ring, summed in
    // wave order; per-tensor mode applies sx * sw once, then bias
    float *red = reinterpret_cast<float *>(lds);
    __syncthreads();
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[((wave * MT + a) * 16 + g * 4 + i) * 17 + fr] = acc[a][i];
    __syncthreads();
    const float scale = MX ? 1.0f : sx[0] * sw[0];
    for (int e = t; e < M * R; e += NW * 64) {
        const int m = e / R, c = e - (e / R) * R;
        if (c >= ncols) continue;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += red[((w * MT + m / 16) * 16 + m % 16) * 17 + c];
        if (!MX) s *= scale;
        const int n = n0 + c;
        if (bias) s += bf16_to_f32(bb);
        store_out(out, (size_t)m * N + n, s, out_f32);
    }
}

namespace {

typedef int (*Fp8RowsLaunch)(const SkgPlan &, const Fp8Args &, int, int, int, hipStream_t);

template <int MP, int NW, int NS, int R, int SB, bool MX>
int launch_fp8_rows_t(const SkgPlan &p, const Fp8Args &a, int M, int N, int K,
                      hipStream_t stream) {
    const size_t lds = (size_t)fp8_rows_lds_bytes(MP, NS, R, SB, MX);
    static std::atomic<unsigned long long> lds_set{0};
    if (lds > 64 * 1024) {
        const hipError_t attr = allow_dynamic_lds(
            reinterpret_cast<const void *>(&fp8_rows_kernel<MP, NW, NS, R, SB, MX>), lds, lds_set);
        if (attr != hipSuccess) return (int)attr;
    }
    hipLaunchKernelGGL((fp8_rows_kernel<MP, NW, NS, R, SB, MX>), dim3(p.grid), dim3(NW * 64), lds,
                       stream, (const uint8_t *)a.x, (const uint8_t *)a.W,
                       (const uint16_t *)a.bias, a.sx, a.sw, a.xe, a.we, a.out, M, N, K,
                       a.out_f32);
    return (int)hipGetLastError();
}

template <int MP, int NW, int NS, int R, int SB, bool MX>
constexpr Fp8RowsLaunch fp8_rows_entry() {
    if constexpr (fp8_rows_built(MP, NW, NS, R, SB, MX))
        return &launch_fp8_rows_t<MP, NW, NS, R, SB, MX>;
    else
        return nullptr;
}

template <int MP, int NW, int R, int SB, bool MX>
Fp8RowsLaunch pick_ns(int NS) {
    switch (NS) {
    case 3: return fp8_rows_entry<MP, NW, 3, R, SB, MX>();
    case 4: return fp8_rows_entry<MP, NW, 4, R, SB, MX>();
    case 5: return fp8_rows_entry<MP, NW, 5, R, SB, MX>();
    case 6: return fp8_rows_entry<MP, NW, 6, R, SB, MX>();
    default: return nullptr;
    }
}

template <int MP, int SB, bool MX>
Fp8RowsLaunch pick_shape(int NW, int NS, int R) {
    if (NW == 4) return R == 16 ? pick_ns<MP, 4, 16, SB, MX>(NS) : R == 8 ? pick_ns<MP, 4, 8, SB, MX>(NS) : nullptr;
    if (NW == 8) return R == 16 ? pick_ns<MP, 8, 16, SB, MX>(NS) : R == 8 ? pick_ns<MP, 8, 8, SB, MX>(NS) : nullptr;
    return nullptr;
}

template <int MP, bool MX>
Fp8RowsLaunch pick_sb(int NW, int NS, int R, int SB) {
    if (SB == 1024) return pick_shape<MP, 1024, MX>(NW, NS, R);
    if (SB == 512) return pick_shape<MP, 512, MX>(NW, NS, R);
    return nullptr;
}

template <bool MX>
Fp8RowsLaunch pick(int MP, int NW, int NS, int R, int SB) {
    switch (MP) {
    case 1: return pick_sb<1, MX>(NW, NS, R, SB);
    case 2: return pick_sb<2, MX>(NW, NS, R, SB);
    case 4: return pick_sb<4, MX>(NW, NS, R, SB);
    case 8: return pick_sb<8, MX>(NW, NS, R, SB);
    case 16: return pick_sb<16, MX>(NW, NS, R, SB);
    case 32: return pick_sb<32, MX>(NW, NS, R, SB);
    default: return nullptr;
    }
}

}  // namespace

int launch_fp8_rows(const SkgPlan &p, const Fp8Args &a, int M, int N, int K, hipStream_t stream) {
    const bool mx = a.mode == SKG_FP8_MX32;
    if (mx && K % kFp8RowsMxK != 0) return (int)hipErrorInvalidConfiguration;  // planner checks it
    const int SB = (p.flags & SKG_FLAG_ROWS_HALF) ? 512 : 1024;
    const int NW = p.threads / 64, MP = fp8_rows_mp(M);
    Fp8RowsLaunch f = mx ? pick<true>(MP, NW, p.depth, p.cols, SB)
                         : pick<false>(MP, NW, p.depth, p.cols, SB);
    if (!f) return (int)hipErrorInvalidConfiguration;
    return f(p, a, M, N, K, stream);
}

}  // namespace skg
