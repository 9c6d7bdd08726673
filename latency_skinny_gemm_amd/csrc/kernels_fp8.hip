// kernels_fp8.hip -- FP8 (OCP e4m3fn) small-M GEMM kernels for gfx950.
//
// Semantics ("sglang PR #28333" page, key source snippet and motivation;
// "sglang PR #34042" page, MX block scaling):
//   per-tensor:  out = bf16( sx*sw * sum_k xq*wq  + bias ),  the scale product
//                applied once, in the epilogue;
//   MX (32):     out = bf16( sum_b 2^(ex[m,b]-127) 2^(ew[n,b]-127) sum_{k in b} xq*wq + bias ),
//                one e8m0 exponent per 32 consecutive K of every row.
// Accumulation is fp32 throughout.
//
// Dot kernel (M <= 16): the bf16 dot kernel's structure (one workgroup per
// column, 16-byte vectors = 16 fp8 values, every load issued up front,
// DPP + LDS reduction), widening e4m3 pairs to fp32 in hardware
// (v_cvt_pk_f32_fp8) and accumulating with fp32 FMA.  In MX mode each
// 16-element partial is scaled by the exact power of two 2^(ex+ew-254)
// (ldexp) before it joins the accumulator.
//
// MFMA kernel: the split-K kernel's structure with
// v_mfma_scale_f32_16x16x128_f8f6f4.  A lane's operand is two 16-element
// chunks of one row (two 16-byte loads) and its e8m0 byte scales one
// 32-element block of the step (the lane layout is measured, see the
// kernel); the hardware applies the scales.  Per-tensor mode passes the
// unit exponent 127 and multiplies by sx*sw once at the end.
#include "device_common.h"
#include "internal.h"
#include "splitk_common.h"

namespace skg {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// OCP e8m0 pair -> the fp32 scale 2^(ex + ew - 254) applied with ldexp
// (exact unless the result leaves fp32's range); 0xFF in either is NaN.
__device__ __forceinline__ float mx_scale_apply(float p, unsigned ex, unsigned ew) {
    if (ex == 0xFFu || ew == 0xFFu) return __builtin_nanf("");
    return __builtin_amdgcn_ldexpf(p, (int)ex + (int)ew - 254);
}

// 16 e4m3 products of two 16-byte vectors added to acc, k ascending.  Each
// byte pair is widened to fp32 with v_cvt_pk_f32_fp8 (exact: e4m3 is a
// subset of fp32) and multiplied-added in fp32 (the product of two e4m3
// values is exact in fp32, so each step rounds once).
__device__ __forceinline__ float fma_word_fp8(unsigned a, unsigned b, float acc) {
    const auto a01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a, false);
    const auto b01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false);
    const auto a23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a, true);
    const auto b23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, true);
    acc = __builtin_fmaf(a01[0], b01[0], acc);
    acc = __builtin_fmaf(a01[1], b01[1], acc);
    acc = __builtin_fmaf(a23[0], b23[0], acc);
    acc = __builtin_fmaf(a23[1], b23[1], acc);
    return acc;
}
__device__ __forceinline__ float dot16_fp8(u32x4 a, u32x4 b, float acc) {
    acc = fma_word_fp8(a.x, b.x, acc);
    acc = fma_word_fp8(a.y, b.y, acc);
    acc = fma_word_fp8(a.z, b.z, acc);
    acc = fma_word_fp8(a.w, b.w, acc);
    return acc;
}

__device__ __forceinline__ unsigned load_byte(Rsrc r, unsigned off) {
    return (unsigned)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// ------------------------------------------------------------------ dot
// QX: x arrives as bf16 and is quantised statically with sx on load (the
// fused form of the "sglang PR #28333" page's static quant kernel): each
// 16-element vector is two 16-byte bf16 loads, turned into 16 e4m3 codes
// exactly as the standalone quantisation kernel does.
// C output columns per workgroup share each x load.  W1: the workgroup is
// one wave (its own instantiation, so the multi-wave kernels compile exactly
// as without it).
template <int M, int C, int V, bool MX, bool QX, bool W1>
__global__ void __launch_bounds__((W1 ? 64 : fp8_dot_max_threads(M, C, V, MX, QX)))
    fp8_dot_kernel(const void *__restrict__ x, const uint8_t *__restrict__ W,
                   const uint16_t *__restrict__ bias, const float *__restrict__ sx,
                   const float *__restrict__ sw, const uint8_t *__restrict__ xe,
                   const uint8_t *__restrict__ we, void *__restrict__ out, int N, int K,
                   int out_f32) {
    static_assert(!(MX && QX), "static quantisation is per-tensor");
    const int T = blockDim.x;
    const int t = threadIdx.x;
    const int n0 = blockIdx.x * C;
    const int ncols = min(C, N - n0);
    const unsigned rowb = (unsigned)K;  // one byte per element
    const Rsrc wr = make_rsrc(W + (size_t)n0 * K, (unsigned)ncols * rowb);
    const unsigned xrowb = QX ? 2u * rowb : rowb;  // bf16 or e4m3 x rows
    const Rsrc xr = make_rsrc(x, (unsigned)M * xrowb);
    const int K16 = K >> 4;
    const unsigned srow = (unsigned)(K >> 5);  // scale bytes per row (MX)
    const Rsrc xer = make_rsrc(xe, MX ? (unsigned)M * srow : 0u);
    const Rsrc wer = make_rsrc(we + (MX ? (size_t)n0 * srow : 0), MX ? (unsigned)ncols * srow : 0u);

    u32x4 wv[C][V], xv[M][V];
    unsigned wsc[C][V], xsc[M][V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int v = t + i * T;
        const unsigned off = v < K16 ? (unsigned)v * 16u : kOOB;
#pragma unroll
        for (int c = 0; c < C; ++c) wv[c][i] = load16<kCacheStream>(wr, off + (unsigned)c * rowb);
    }
    if constexpr (QX) {
        const float inv = 1.0f / sx[0];  // correctly rounded (no fast-math)
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int v = t + i * T;
            const unsigned off = v < K16 ? (unsigned)v * 32u : kOOB;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4 lo = load16<kCacheDefault>(xr, off + (unsigned)m * xrowb);
                const u32x4 hi = load16<kCacheDefault>(xr, off + 16u + (unsigned)m * xrowb);
                xv[m][i] = quant16_e4m3(lo, hi, inv);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int v = t + i * T;
            const unsigned off = v < K16 ? (unsigned)v * 16u : kOOB;
#pragma unroll
            for (int m = 0; m < M; ++m)
                xv[m][i] = load16<kCacheDefault>(xr, off + (unsigned)m * rowb);
        }
    }
    if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int v = t + i * T;
            const unsigned blk = v < K16 ? (unsigned)(v >> 1) : kOOB;  // 32-element block
#pragma unroll
            for (int c = 0; c < C; ++c) wsc[c][i] = load_byte(wer, blk + (unsigned)c * srow);
#pragma unroll
            for (int m = 0; m < M; ++m) xsc[m][i] = load_byte(xer, blk + (unsigned)m * srow);
        }
    }

    float acc[C][M];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[c][m] = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int v = t + i * T;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if constexpr (MX) {
                    const float p = dot16_fp8(xv[m][i], wv[c][i], 0.0f);
                    if (v < K16) acc[c][m] += mx_scale_apply(p, xsc[m][i], wsc[c][i]);
                } else {
                    acc[c][m] = dot16_fp8(xv[m][i], wv[c][i], acc[c][m]);
                }
            }
    }

    // the C*M sums over the wave by one reduce-scatter (lane l ends with the
    // total of index l >> (6 - L), index c*M + m), then over the waves in
    // wave order
    constexpr int CM = C * M;
    constexpr int L = CM <= 1 ? 0 : CM <= 2 ? 1 : CM <= 4 ? 2 : CM <= 8 ? 3 : CM <= 16 ? 4 : CM <= 32 ? 5 : 6;
    static_assert(CM <= 64, "one value index per lane at most");
    float part[1 << L];
#pragma unroll
    for (int i = 0; i < (1 << L); ++i) part[i] = i < CM ? acc[i / M][i % M] : 0.0f;
    const float total = wave_reduce_scatter<L>(part);
    const int lane = t & 63;
    const int idx = lane >> (6 - L);
    const bool owner = (lane & ((1 << (6 - L)) - 1)) == 0 && idx < CM;

    __shared__ float red[kMaxThreads / 64][CM];
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int nw = T >> 6;
    if constexpr (W1) {
        // One wave: its totals are final, so each owner lane stores its
        // output with no LDS round trip and no barrier (the same bits as the
        // cross-wave sum below, which starts from 0 too).
        if (owner) {
            const int c = idx / M, m = idx - (idx / M) * M;
            const int n = n0 + c;
            if (n < N) {
                float s = 0.0f + total;
                if (!MX) s *= sx[0] * sw[0];
                if (bias) s += bf16_to_f32(bias[n]);
                store_out(out, (size_t)m * N + n, s, out_f32);
            }
        }
        return;
    }
    if (owner) red[wave][idx] = total;
    __syncthreads();
    if (t < C * M) {
        const int c = t / M, m = t - (t / M) * M;
        const int n = n0 + c;
        float s = ordered_sum<8>(nw, [&](int w) { return red[w][t]; });
        if (n < N) {
            if (!MX) s *= sx[0] * sw[0];
            if (bias) s += bf16_to_f32(bias[n]);
            store_out(out, (size_t)m * N + n, s, out_f32);
        }
    }
}

// ------------------------------------------------------------------ MFMA split-K
// QX: x arrives as bf16 and is quantised statically with sx, as in the dot
// kernel: the stage keeps the raw bf16 (four 16-byte loads per step and
// m-tile) and each 16-element chunk becomes 16 e4m3 codes just before its
// MFMAs, with the same conversion as the standalone quantisation kernel.
template <int MT, int NB, int D, bool MX, bool QX>
__global__ void __launch_bounds__((QX ? 256 : fp8_mfma_max_threads(MT, NB, D, MX)))
    fp8_mfma_kernel(const void *__restrict__ x, const uint8_t *__restrict__ W,
                    const uint16_t *__restrict__ bias, const float *__restrict__ sx,
                    const float *__restrict__ sw, const uint8_t *__restrict__ xe,
                    const uint8_t *__restrict__ we, void *__restrict__ out,
                    float *__restrict__ ws, unsigned *__restrict__ tickets, int M, int N, int K,
                    int S, int k_chunk, int reduce, int out_f32) {
    extern __shared__ float lds[];
    __shared__ unsigned is_last;

    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.x % S;
    const int j = blockIdx.x / S;
    const int col0 = j * NB * 16;
    const int ncols = min(NB * 16, N - col0);
    static_assert(!(MX && QX), "static quantisation is per-tensor");
    const unsigned rowb = (unsigned)K;
    const unsigned xrowb = QX ? 2u * rowb : rowb;  // bf16 or e4m3 x rows
    const unsigned srow = (unsigned)(K >> 5);
    const Rsrc wr = make_rsrc(W + (size_t)col0 * K, (unsigned)ncols * rowb);
    const Rsrc xr = make_rsrc(x, (unsigned)M * xrowb);
    const Rsrc xer = make_rsrc(xe, MX ? (unsigned)M * srow : 0u);
    const Rsrc wer = make_rsrc(we + (MX ? (size_t)col0 * srow : 0), MX ? (unsigned)ncols * srow : 0u);
    const int kbeg = s * k_chunk;
    const int kend = min(K, kbeg + k_chunk);
    const int nsteps = (kend - kbeg + 127) >> 7;  // 128-wide K steps
    const int spw = (nsteps + nw - 1) / nw;
    const int first_step = wave * spw;
    const int my_steps = max(0, min(spw, nsteps - first_step));
    const int nchunks = (my_steps + D - 1) / D;
    const unsigned r16 = (unsigned)(lane & 15);
    // Operand layout of the 16x16x128 f8f6f4 MFMA (measured on MI355X): lane
    // group g = lane/16 holds two 16-element chunks of its row, K offsets
    // 16g and 64 + 16g of the 128-wide step, and its scale byte applies to
    // the step's 32-element block g (K offsets 32g .. 32g+31).
    const int g16 = (lane >> 4) * 16;
    const int gblk = lane >> 4;

    f32x4 acc[NB][MT];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // a stage: D steps of (two 16-byte halves per operand block, x as bf16
    // taking four) + MX scales
    constexpr int XH = QX ? 4 : 2;
    const float inv = QX ? 1.0f / sx[0] : 0.0f;  // correctly rounded (no fast-math)
    u32x4 wa[D][NB][2], xa[D][MT][XH], wb[D][NB][2], xb[D][MT][XH];
    unsigned wsa[D][NB], xsa[D][MT], wsb[D][NB], xsb[D][MT];

    auto load_stage = [&](u32x4(&wbuf)[D][NB][2], u32x4(&xbuf)[D][MT][XH], unsigned(&wsc)[D][NB],
                          unsigned(&xsc)[D][MT], int chunk) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = chunk * D + d;
            const int k0 = kbeg + (first_step + i) * 128;  // the step's first K
            const bool live = i < my_steps;
            // each 16-element chunk and the scale's block have their own
            // bound (K may end inside the step; per-tensor K may end halfway
            // through a 32-element block)
            const bool ok0 = live & (k0 + g16 < kend);
            const bool ok1 = live & (k0 + 64 + g16 < kend);
            const bool okb = live & (k0 + 32 * gblk < kend);
            const unsigned koff = ok0 ? (unsigned)(k0 + g16) : kOOB;
            const unsigned koff1 = ok1 ? (unsigned)(k0 + 64 + g16) : kOOB;
            const unsigned boff = okb ? (unsigned)(k0 / 32 + gblk) : kOOB;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const unsigned ro = ((unsigned)nb * 16u + r16) * rowb;
                wbuf[d][nb][0] = load16<kCacheStream>(wr, koff + ro);
                wbuf[d][nb][1] = load16<kCacheStream>(wr, koff1 + ro);
                if constexpr (MX) {
                    const unsigned e = load_byte(wer, boff + ((unsigned)nb * 16u + r16) * srow);
                    wsc[d][nb] = okb ? e : 127u;
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const unsigned ro = ((unsigned)mt * 16u + r16) * xrowb;
                if constexpr (QX) {
                    const unsigned q0 = ok0 ? (unsigned)(k0 + g16) * 2u : kOOB;
                    const unsigned q1 = ok1 ? (unsigned)(k0 + 64 + g16) * 2u : kOOB;
                    xbuf[d][mt][0] = load16<kCacheDefault>(xr, q0 + ro);
                    xbuf[d][mt][1] = load16<kCacheDefault>(xr, q0 + 16u + ro);
                    xbuf[d][mt][2] = load16<kCacheDefault>(xr, q1 + ro);
                    xbuf[d][mt][3] = load16<kCacheDefault>(xr, q1 + 16u + ro);
                } else {
                    xbuf[d][mt][0] = load16<kCacheDefault>(xr, koff + ro);
                    xbuf[d][mt][1] = load16<kCacheDefault>(xr, koff1 + ro);
                }
                if constexpr (MX) {
                    // rows past M read as zero data; give them the unit scale
                    const unsigned e = load_byte(xer, boff + ((unsigned)mt * 16u + r16) * srow);
                    xsc[d][mt] = (okb && (int)(mt * 16 + r16) < M) ? e : 127u;
                }
            }
        }
    };
    auto mma_stage = [&](u32x4(&wbuf)[D][NB][2], u32x4(&xbuf)[D][MT][XH], unsigned(&wsc)[D][NB],
                         unsigned(&xsc)[D][MT]) {
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                u32x4 a0, a1;
                if constexpr (QX) {
                    a0 = quant16_e4m3(xbuf[d][mt][0], xbuf[d][mt][1], inv);
                    a1 = quant16_e4m3(xbuf[d][mt][2], xbuf[d][mt][3], inv);
                } else {
                    a0 = xbuf[d][mt][0];
                    a1 = xbuf[d][mt][1];
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const u32x4 b0 = wbuf[d][nb][0], b1 = wbuf[d][nb][1];
                    const i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                     (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                                     (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                    const int sa = MX ? (int)xsc[d][mt] : 127;
                    const int sb = MX ? (int)wsc[d][nb] : 127;
                    // formats 0/0: both operands fp8 e4m3; scale byte 0 of each lane
                    acc[nb][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a, b, acc[nb][mt], 0, 0, 0, sa, 0, sb);
                }
            }
    };

    if (nchunks <= 1) {
        load_stage(wa, xa, wsa, xsa, 0);
        mma_stage(wa, xa, wsa, xsa);
    } else {
        load_stage(wa, xa, wsa, xsa, 0);
        for (int c = 0; c < nchunks; c += 2) {
            load_stage(wb, xb, wsb, xsb, c + 1);  // past the end: zeros, unit scales
            mma_stage(wa, xa, wsa, xsa);
            load_stage(wa, xa, wsa, xsa, c + 2);
            mma_stage(wb, xb, wsb, xsb);
        }
    }

    constexpr int Q = NB * MT * 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lds[(wave * Q + (nb * MT + mt) * 4 + i) * 64 + lane] = acc[nb][mt][i];
    __syncthreads();
    const float scale = MX ? 1.0f : sx[0] * sw[0];
    for (int q = wave; q < Q; q += nw) {
        float v = ordered_sum<8>(nw, [&](int w) { return lds[(w * Q + q) * 64 + lane]; });
        const int nb = q / (MT * 4);
        const int mt = (q >> 2) % MT;
        const int i = q & 3;
        const int n = col0 + nb * 16 + (lane & 15);
        const int m = mt * 16 + (lane >> 4) * 4 + i;
        if (m < M && n < N) {
            if (S == 1) {
                v *= scale;
                if (bias) v += bf16_to_f32(bias[n]);
                store_out(out, (size_t)m * N + n, v, out_f32);
            } else {
                put_partial(ws, ((size_t)s * M + m) * N + n, v, reduce == SKG_REDUCE_LAST);
            }
        }
    }
    if (S == 1 || reduce != SKG_REDUCE_LAST) return;
    last_arriver_reduce<2, 4>(ws, tickets, bias, out, out_f32, M, N, S, j, col0, ncols, &is_last,
                              !MX, scale);
}

namespace {

typedef int (*Fp8DotLaunch)(const SkgPlan &, const Fp8Args &, int, int, hipStream_t);
typedef int (*Fp8MfmaLaunch)(const SkgPlan &, const Fp8Args &, float *, unsigned *, int, int, int,
                             hipStream_t);

template <int M, int C, int V, bool MX, bool QX>
int launch_fp8_dot_t(const SkgPlan &p, const Fp8Args &a, int N, int K, hipStream_t stream) {
    if constexpr (M <= kDotOneWaveMaxM) {
        if (p.threads == 64) {
            hipLaunchKernelGGL((fp8_dot_kernel<M, C, V, MX, QX, true>), dim3(p.grid), dim3(64), 0,
                               stream, a.x, (const uint8_t *)a.W, (const uint16_t *)a.bias, a.sx,
                               a.sw, a.xe, a.we, a.out, N, K, a.out_f32);
            return (int)hipGetLastError();
        }
    }
    hipLaunchKernelGGL((fp8_dot_kernel<M, C, V, MX, QX, false>), dim3(p.grid), dim3(p.threads), 0,
                       stream, a.x, (const uint8_t *)a.W, (const uint16_t *)a.bias, a.sx, a.sw,
                       a.xe, a.we, a.out, N, K, a.out_f32);
    return (int)hipGetLastError();
}

template <int M, int C, int V, bool MX, bool QX>
constexpr Fp8DotLaunch fp8_dot_entry() {
    if constexpr (QX ? (!MX && fp8q_dot_regs(M, C, V) <= kDotRegsMax)
                     : fp8_dot_regs(M, C, V, MX) <= kDotRegsMax)
        return &launch_fp8_dot_t<M, C, V, MX, QX>;
    else
        return nullptr;
}

template <int M, int C, bool MX, bool QX>
Fp8DotLaunch fp8_dot_v(int V) {
    switch (V) {
    case 1: return fp8_dot_entry<M, C, 1, MX, QX>();
    case 2: return fp8_dot_entry<M, C, 2, MX, QX>();
    case 4: return fp8_dot_entry<M, C, 4, MX, QX>();
    default: return nullptr;
    }
}

template <int M, bool MX, bool QX>
Fp8DotLaunch fp8_dot_c(int C, int V) {
    switch (C) {
    case 1: return fp8_dot_v<M, 1, MX, QX>(V);
    case 2: return fp8_dot_v<M, 2, MX, QX>(V);
    case 4: return fp8_dot_v<M, 4, MX, QX>(V);
    default: return nullptr;
    }
}

template <bool MX, bool QX>
Fp8DotLaunch fp8_dot_m(int M, int C, int V) {
    switch (M) {
    case 1: return fp8_dot_c<1, MX, QX>(C, V);
    case 2: return fp8_dot_c<2, MX, QX>(C, V);
    case 3: return fp8_dot_c<3, MX, QX>(C, V);
    case 4: return fp8_dot_c<4, MX, QX>(C, V);
    case 5: return fp8_dot_c<5, MX, QX>(C, V);
    case 6: return fp8_dot_c<6, MX, QX>(C, V);
    case 7: return fp8_dot_c<7, MX, QX>(C, V);
    case 8: return fp8_dot_c<8, MX, QX>(C, V);
    case 9: return fp8_dot_c<9, MX, QX>(C, V);
    case 10: return fp8_dot_c<10, MX, QX>(C, V);
    case 11: return fp8_dot_c<11, MX, QX>(C, V);
    case 12: return fp8_dot_c<12, MX, QX>(C, V);
    case 13: return fp8_dot_c<13, MX, QX>(C, V);
    case 14: return fp8_dot_c<14, MX, QX>(C, V);
    case 15: return fp8_dot_c<15, MX, QX>(C, V);
    case 16: return fp8_dot_c<16, MX, QX>(C, V);
    default: return nullptr;
    }
}

template <int MT, int NB, int D, bool MX, bool QX>
int launch_fp8_mfma_t(const SkgPlan &p, const Fp8Args &a, float *ws, unsigned *tickets, int M,
                      int N, int K, hipStream_t stream) {
    const size_t lds_bytes = (size_t)(p.threads / 64) * NB * MT * 4 * 64 * sizeof(float);
    hipLaunchKernelGGL((fp8_mfma_kernel<MT, NB, D, MX, QX>), dim3(p.grid), dim3(p.threads),
                       lds_bytes, stream, a.x, (const uint8_t *)a.W, (const uint16_t *)a.bias,
                       a.sx, a.sw, a.xe, a.we, a.out, ws, tickets, M, N, K, p.splits,
                       p.k_chunk, p.reduce, a.out_f32);
    return (int)hipGetLastError();
}

template <int MT, int NB, int D, bool MX, bool QX>
constexpr Fp8MfmaLaunch fp8_mfma_entry() {
    if constexpr (QX ? fp8q_mfma_built(MT, NB, D) : fp8_mfma_built(MT, NB, D))
        return &launch_fp8_mfma_t<MT, NB, D, MX, QX>;
    else
        return nullptr;
}

template <int MT, int NB, bool MX, bool QX>
Fp8MfmaLaunch fp8_mfma_d(int D) {
    switch (D) {
    case 1: return fp8_mfma_entry<MT, NB, 1, MX, QX>();
    case 2: return fp8_mfma_entry<MT, NB, 2, MX, QX>();
    case 4: return fp8_mfma_entry<MT, NB, 4, MX, QX>();
    default: return nullptr;
    }
}

template <int MT, bool MX, bool QX>
Fp8MfmaLaunch fp8_mfma_nb(int NB, int D) {
    return NB == 1 ? fp8_mfma_d<MT, 1, MX, QX>(D) : NB == 2 ? fp8_mfma_d<MT, 2, MX, QX>(D)
                   : NB == 4 ? fp8_mfma_d<MT, 4, MX, QX>(D) : nullptr;
}

template <bool MX, bool QX>
Fp8MfmaLaunch fp8_mfma_mt(int MT, int NB, int D) {
    switch (MT) {
    case 1: return fp8_mfma_nb<1, MX, QX>(NB, D);
    case 2: return fp8_mfma_nb<2, MX, QX>(NB, D);
    case 3: return fp8_mfma_nb<3, MX, QX>(NB, D);
    case 4: return fp8_mfma_nb<4, MX, QX>(NB, D);
    case 5: return fp8_mfma_nb<5, MX, QX>(NB, D);
    case 6: return fp8_mfma_nb<6, MX, QX>(NB, D);
    case 7: return fp8_mfma_nb<7, MX, QX>(NB, D);
    case 8: return fp8_mfma_nb<8, MX, QX>(NB, D);
    default: return nullptr;
    }
}

}  // namespace

bool fp8_mfma_quant_ok(int MT, int NB, int D, int threads) {
    return threads <= 256 && fp8_mfma_mt<false, true>(MT, NB, D) != nullptr;
}

bool fp8_dot_quant_ok(int M, int C, int V, int threads) {
    if (M < 1 || M > kDotMaxM || fp8_dot_m<false, true>(M, C, V) == nullptr) return false;
    return threads <= fp8_dot_max_threads(M, C, V, false, true);
}

int launch_fp8(const SkgPlan &p, const Fp8Args &a, float *ws, unsigned *tickets, int M, int N,
               int K, hipStream_t stream) {
    const bool mx = a.mode == SKG_FP8_MX32;
    if (p.kind == SKG_KIND_DOT) {
        Fp8DotLaunch f = mx      ? fp8_dot_m<true, false>(M, p.cols, p.depth)
                         : a.qx ? fp8_dot_m<false, true>(M, p.cols, p.depth)
                                : fp8_dot_m<false, false>(M, p.cols, p.depth);
        if (!f) return (int)hipErrorInvalidConfiguration;
        return f(p, a, N, K, stream);
    }
    // fused quantisation: the dot and MFMA split-K kernels only (the caller
    // quantises x first for every other plan)
    if (a.qx && (mx || p.kind != SKG_KIND_SPLITK)) return (int)hipErrorInvalidConfiguration;
    if (p.kind == SKG_KIND_TILED) return launch_fp8_tiled(p, a, ws, tickets, M, N, K, stream);
    if (p.kind == SKG_KIND_ROWS) return launch_fp8_rows(p, a, M, N, K, stream);
    Fp8MfmaLaunch f = mx     ? fp8_mfma_mt<true, false>(p.m_tiles, p.cols, p.depth)
                      : a.qx ? fp8_mfma_mt<false, true>(p.m_tiles, p.cols, p.depth)
                             : fp8_mfma_mt<false, false>(p.m_tiles, p.cols, p.depth);
    if (!f) return (int)hipErrorInvalidConfiguration;
    int rc = f(p, a, ws, tickets, M, N, K, stream);
    if (rc != (int)hipSuccess || p.splits == 1 || p.reduce != SKG_REDUCE_KERNEL) return rc;
    return launch_splitk_reduce(ws, a.bias, a.out, a.out_f32, M, N, p.splits, stream,
                                mx ? nullptr : a.sx,
                                mx ? nullptr : a.sw);
}

}  // namespace skg
