// internal.h -- declarations shared by the library's translation units.
// Not installed; the public ABI is include/skinny_gemm.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "skinny_gemm.h"

namespace skg {

// FP8 plans, per-tensor or MX scales: the same kernels and limits; the two
// dtypes only key separate dispatch-table entries.
constexpr bool is_fp8(int dtype) { return dtype == SKG_DTYPE_FP8 || dtype == SKG_DTYPE_FP8_MX; }

// Limits of the kernels as built.
constexpr int kMaxThreads = 1024;
constexpr int kDotMaxM = 16;          // dot kernel is instantiated for M = 1..16
constexpr int kSplitKMaxLdsFloats = 16384;  // 64 KB of LDS for the wave reduction
constexpr int kMaxSplits = 256;
constexpr int kNumCusMI355X = 256;
constexpr long kMaxBufferBytes = 0x7FFFFFFFL;  // one buffer resource covers < 2 GiB

// DOT: vectors (16 B) per thread per column that the kernel is built for.
constexpr int kDotVecs[] = {1, 2, 3, 4, 6, 7, 8, 12, 14, 16};
// One-wave dot workgroups (64 threads) store without the LDS reduction for
// M up to this (larger M run 64 threads through the general kernel).
constexpr int kDotOneWaveMaxM = 8;
// Registers a DOT thread holds: C rows of W and M rows of x, V 16-byte
// vectors each, x counted twice (the compiler widens x to fp32 ahead of
// use), and C*M accumulators.  Only the 256 architectural VGPRs feed VALU
// work: a kernel is built only when this is <= 224 and may run 1024-thread
// workgroups (4 waves per SIMD, 128 VGPRs each) only when it is <= 96.
// (Checked against the compiler's resource report: no kernel spills.)
// With the dot2 instruction x stays packed (no widening): M + C rows.
constexpr int dot_regs(int M, int C, int V, bool dot2) {
    return ((dot2 ? M : 2 * M) + C) * V * 4 + C * M;
}
constexpr int kDotRegsMax = 224;
constexpr int dot_max_threads(int M, int C, int V, bool dot2) {
    return dot_regs(M, C, V, dot2) <= 96 ? 1024 : 512;
}

// DOT with x staged in LDS (SKG_FLAG_DOT_XLDS), K = 512 * V exactly: every
// wave owns CW output columns over the whole K (64 lanes x V 16-byte
// vectors per column), all
// M rows of x sit in LDS, loaded once per workgroup; a workgroup of nw
// waves covers CW * nw columns.  Registers: the CW * V W vectors in flight,
// one step's M x vectors, CW * M accumulators and some addressing; the
// same launch bounds as the plain dot kernel.  The whole x must fit the
// LDS a workgroup may use, and the W loads of a thread must fit vmcnt's
// 6 bits (the kernel waits for its x loads by counting them).
constexpr int kXldsVecs[] = {4, 6, 8, 12, 14, 16};
constexpr int xlds_regs(int M, int CW, int V) { return CW * V * 4 + 4 * M + CW * M + 16; }
constexpr int xlds_max_threads(int M, int CW, int V) { return xlds_regs(M, CW, V) <= 96 ? 1024 : 512; }
constexpr bool xlds_built(int M, int CW, int V) {
    return (CW == 1 || CW == 2 || CW == 4) && xlds_regs(M, CW, V) <= kDotRegsMax && CW * V < 64;
}
constexpr long kXldsMaxLds = 160 * 1024 - 256;
// LDS of one workgroup: the M x K8 16-byte chunks of x.
constexpr long xlds_lds_bytes(int M, int K8) { return (long)M * K8 * 16; }

// ROWS (MFMA, M <= 64): stages of KS = 512 (or 256 with SKG_FLAG_ROWS_HALF)
// K elements; R = 8 or 16 columns per workgroup (also 10 or 12 up to 16
// rows, to spread N over more CUs); each of the R W rows and MP x rows of a stage (MP = M up to
// 16 rows, else M rounded up to 24, 32, 48 or 64) is one LDS row of 2*KS
// bytes, plus 1 KB that takes the padding loads.  A load instruction fills
// 1 KB: one row (KS = 512) or two (KS = 256).  Wave w issues the W
// instructions w, w+NW, ... and the x instructions likewise.  Built when
// the ring fits the LDS a workgroup may use and the ring's vmcnt wait
// (loads of NS-2 stages) fits its 6-bit field.
constexpr int kRowsMaxM = 64;
constexpr int rows_mp(int M) { return M <= 16 ? M : M <= 24 ? 24 : M <= 32 ? 32 : M <= 48 ? 48 : 64; }
constexpr int rows_per_load(int KS) { return 1024 / (2 * KS); }
constexpr int rows_w_loads(int NW, int R, int KS) {
    return (R / rows_per_load(KS) + NW - 1) / NW;
}
constexpr int rows_x_loads(int MP, int NW, int KS) {
    return ((MP + rows_per_load(KS) - 1) / rows_per_load(KS) + NW - 1) / NW;
}
constexpr int rows_stage_bytes(int MP, int R, int KS) {
    return (R + (MP + rows_per_load(KS) - 1) / rows_per_load(KS) * rows_per_load(KS)) * 2 * KS +
           1024;
}
constexpr long rows_lds_bytes(int MP, int NS, int R, int KS) {
    return (long)NS * rows_stage_bytes(MP, R, KS);
}
constexpr bool rows_built(int MP, int NW, int NS, int R, int KS) {
    return MP >= 1 && MP <= kRowsMaxM && MP == rows_mp(MP) && (NW == 4 || NW == 8) &&
           (R == 8 || R == 16 || ((R == 10 || R == 12) && MP <= 16)) &&
           (KS == 512 || KS == 256) && NS >= 3 && NS <= 6 &&
           rows_lds_bytes(MP, NS, R, KS) <= 160 * 1024 - 256 &&
           (NS - 2) * (rows_w_loads(NW, R, KS) + rows_x_loads(MP, NW, KS)) < 64;
}

// FP8 ROWS (M <= 32): the bf16 ring's layout with SB = 1024 (or 512) K per
// stage, codes of R W rows and XR x rows (MP rounded to whole loads), the
// padding KB, and for MX one KB block of scale bytes per 32 (or 64) rows of
// each operand.  MP = the power of two at or above M.  MX needs K % 512 == 0.
constexpr int kFp8RowsMaxM = 32;
constexpr int kFp8RowsMxK = 512;
constexpr int fp8_rows_mp(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : M <= 16 ? 16 : 32; }
constexpr int fp8_rows_xr(int MP, int SB) { return (MP + 1024 / SB - 1) / (1024 / SB) * (1024 / SB); }
constexpr int fp8_rows_scale_loads(int rows, int SB) { return (rows + 32768 / SB - 1) / (32768 / SB); }
constexpr int fp8_rows_stage_bytes(int MP, int R, int SB, bool MX) {
    return (R + fp8_rows_xr(MP, SB)) * SB + 1024 +
           (MX ? (fp8_rows_scale_loads(R, SB) + fp8_rows_scale_loads(fp8_rows_xr(MP, SB), SB)) * 1024
               : 0);
}
constexpr long fp8_rows_lds_bytes(int MP, int NS, int R, int SB, bool MX) {
    return (long)NS * fp8_rows_stage_bytes(MP, R, SB, MX);
}
constexpr int fp8_rows_loads(int MP, int NW, int R, int SB, bool MX) {
    return (R / (1024 / SB) + NW - 1) / NW + (fp8_rows_xr(MP, SB) / (1024 / SB) + NW - 1) / NW +
           (MX ? 1 : 0);
}
constexpr bool fp8_rows_built(int MP, int NW, int NS, int R, int SB, bool MX) {
    return MP >= 1 && MP <= kFp8RowsMaxM && MP == fp8_rows_mp(MP) && (NW == 4 || NW == 8) &&
           (R == 8 || R == 16) && (SB == 1024 || SB == 512) && (SB / 128) % NW == 0 && NS >= 3 &&
           NS <= 6 && fp8_rows_lds_bytes(MP, NS, R, SB, MX) <= 160 * 1024 - 256 &&
           (NS - 2) * fp8_rows_loads(MP, NW, R, SB, MX) < 64 &&
           (!MX || fp8_rows_scale_loads(R, SB) + fp8_rows_scale_loads(fp8_rows_xr(MP, SB), SB) <= NW) &&
           NW * ((MP + 15) / 16) * 16 * 17 * 4 <= NS * fp8_rows_stage_bytes(MP, R, SB, MX);
}

// SPLITK per-lane registers: two stages of D steps of (NB + MT) vectors and
// NB*MT accumulators of 4 (those may live in AGPRs).  Above 224 the kernel
// is bounded to 256 threads (one wave per SIMD); up to 96 it may run 1024
// (16 waves: four per SIMD at 128 VGPRs), else 512.
constexpr int splitk_regs(int MT, int NB, int D) { return 2 * D * (NB + MT) * 4 + NB * MT * 4; }
constexpr int splitk_max_threads(int MT, int NB, int D) {
    return splitk_regs(MT, NB, D) > 224 ? 256 : splitk_regs(MT, NB, D) <= 96 ? 1024 : 512;
}
constexpr bool splitk_built(int MT, int NB, int D) { return NB * MT <= 32 && D * (NB + MT) <= 40; }

// SPLITK: K steps (32 wide) in flight per wave per stage.
constexpr int kSplitKDepths[] = {1, 2, 4, 8};

// TILED: 4 waves as WM x WN over MT m-tiles (a power of two covering M) and
// NB column blocks; a wave owns MT/WM x NB/WN tiles.  A ring of NS LDS
// stages of U (2 or 4) 32-wide K steps, (MT + NB) * U KB per stage, plus
// 1 KB of padding.  Built when the accumulators and one stage's fragments
// fit 200 of the 256 VGPRs (the accumulators live in VGPRs), the ring fits
// 144 KB and also holds the fp32 output tile of the epilogue, and the vmcnt
// wait of the ring (loads of NS-2 stages) fits its 6-bit field.
constexpr int kTiledThreads = 256;
constexpr int kTiledMaxRows = 128;  // rows per workgroup (MT <= 8); more M: row blocks
// Row blocks of MT*16 rows that cover M (1 unless M > 128).
constexpr int tiled_row_blocks(int M, int MT) { return (M + MT * 16 - 1) / (MT * 16); }
// gfx950 gives a workgroup up to 160 KB of LDS; the tiled kernels keep 256
// bytes of it for their static variables.
constexpr int kTiledMaxLds = 160 * 1024 - 256;
constexpr int kTiledStages[] = {2, 3, 4, 5, 6, 8};
constexpr size_t tiled_lds_bytes(int MT, int NB, int NS, int U) {
    return (size_t)NS * U * (MT + NB) * 1024 + 1024;
}
constexpr bool tiled_built(int MT, int NB, int WM, int NS, int U) {
    return (WM == 1 || WM == 2 || WM == 4) && MT % WM == 0 && NB % (4 / WM) == 0 &&
           4 * (MT / WM) * (NB / (4 / WM)) + 4 * U * (MT / WM + NB / (4 / WM)) <= 200 &&
           tiled_lds_bytes(MT, NB, NS, U) <= kTiledMaxLds &&
           tiled_lds_bytes(MT, NB, NS, U) >= (size_t)MT * 16 * (NB * 16 + 4) * 4 &&
           (NS - 2) * ((U * MT + 3) / 4 + (U * NB + 3) / 4) < 64;
}

// FP8 dot kernel: x counted packed plus its widened words (as for bf16
// without dot2) and, in MX mode, one scale byte per (row, vector); a plan is
// checked for the MX count, the larger.  With several columns the compiler
// keeps every x vector widened to fp32 (16 VGPRs) for reuse across the
// columns, so C > 1 is also bounded by that count (fitted to the compiler's
// resource report, conservatively: no kernel built under it spills).
constexpr int kFp8DotVecs[] = {1, 2, 4};
constexpr int fp8_dot_wide_regs(int M, int C, int V) {
    return C > 1 ? 16 * M * V + 8 * C * V + C * M + 16 : 0;
}
constexpr int fp8_dot_regs(int M, int C, int V, bool mx) {
    const int base = dot_regs(M, C, V, false) + (mx ? (M + C) * V : 0);
    return base > fp8_dot_wide_regs(M, C, V) ? base : fp8_dot_wide_regs(M, C, V);
}
// With x arriving as bf16 and quantised on load (static per-tensor FP8),
// each vector of a row is two 16-byte loads (8 VGPRs) until it is packed
// into 4 VGPRs of codes; counted as 12 per (row, vector) plus W.
constexpr int fp8q_dot_regs(int M, int C, int V) {
    const int base = M * V * 12 + 4 * C * V + C * M;
    return base > fp8_dot_wide_regs(M, C, V) ? base : fp8_dot_wide_regs(M, C, V);
}
constexpr int fp8_dot_max_threads(int M, int C, int V, bool mx, bool qx = false) {
    return (qx ? fp8q_dot_regs(M, C, V) : fp8_dot_regs(M, C, V, mx)) <= 96 ? 1024 : 512;
}

// FP8 MFMA split-K (v_mfma_scale_f32_16x16x128_f8f6f4, 128-wide K steps):
// per lane per step two 16-byte halves per operand block (8 VGPRs) and a
// scale byte; two stages of D steps plus NB*MT accumulators of 4.
constexpr int fp8_mfma_regs(int MT, int NB, int D) { return 2 * D * (NB + MT) * 9 + NB * MT * 4; }
// MX variants keep one scale byte per operand block and step alive beside
// the data and, measured on the compiler's resource report, need the full
// 512 registers of one wave per SIMD: they are bounded to 256 threads.
constexpr int fp8_mfma_max_threads(int MT, int NB, int D, bool mx) {
    return (mx || fp8_mfma_regs(MT, NB, D) > 224) ? 256 : 512;
}
constexpr bool fp8_mfma_built(int MT, int NB, int D) {
    return NB * MT <= 32 && D * (NB + MT) <= 14;  // MX spills beyond (resource report)
}
// With x arriving as bf16 (fused static quantisation, per-tensor only), a
// stage keeps 16 VGPRs of raw x per (step, m-tile) instead of 8; built for
// up to 32 rows (the small-M plans the fused path meets).  The conversion
// needs temporaries beside them: above 160 by this count the resource
// report showed spills, so the bound is 160.
constexpr int fp8q_mfma_regs(int MT, int NB, int D) { return 2 * D * (NB * 9 + MT * 16) + NB * MT * 4; }
constexpr bool fp8q_mfma_built(int MT, int NB, int D) {
    return MT <= 2 && fp8_mfma_built(MT, NB, D) && fp8q_mfma_regs(MT, NB, D) <= 160;
}

// FP8 TILED: the bf16 tiled kernel's ring with 128-wide K steps; a stage
// holds U (1 or 2) steps: (MT + NB) blocks of 16 rows x 128U bytes, plus in
// MX mode the stage's scale bytes (rows x 4U, rounded up to 256 bytes per
// operand).  The ring is sized for MX in both modes.  Built when the
// accumulators and one stage's fragments fit 200 VGPRs, the ring fits
// 144 KB and holds the epilogue tile, the vmcnt wait fits 6 bits, and each
// operand's scales take at most one load per wave.
constexpr size_t fp8_tiled_stage_bytes(int MT, int NB, int U) {
    return (size_t)(MT + NB) * 2048 * U;
}
constexpr size_t fp8_tiled_lds_bytes(int MT, int NB, int NS, int U) {
    return (size_t)NS * fp8_tiled_stage_bytes(MT, NB, U) + 1024;
}
// MX: the e8m0 bytes of a workgroup's K chunk (k_chunk / 32 per row) sit
// after the ring, rows SR bytes apart with SR = 16 mod 32 (the 16 rows of one
// fragment read then hit 16 different banks), x rows then W rows, each
// area a whole number of KB.
constexpr int fp8_tiled_scale_stride(int k_chunk) { return (k_chunk / 32 + 47) / 32 * 32 - 16; }
constexpr size_t fp8_tiled_scale_area(int rows, int k_chunk) {
    return ((size_t)rows * fp8_tiled_scale_stride(k_chunk) + 1023) / 1024 * 1024;
}
constexpr size_t fp8_tiled_mx_lds_bytes(int MT, int NB, int NS, int U, int k_chunk) {
    return fp8_tiled_lds_bytes(MT, NB, NS, U) + fp8_tiled_scale_area(MT * 16, k_chunk) +
           fp8_tiled_scale_area(NB * 16, k_chunk);
}
constexpr bool fp8_tiled_built(int MT, int NB, int WM, int NS, int U) {
    return (WM == 1 || WM == 2 || WM == 4) && MT % WM == 0 && NB % (4 / WM) == 0 &&
           (U == 1 || U == 2) && MT * U <= 16 && NB * U <= 16 &&
           4 * (MT / WM) * (NB / (4 / WM)) + 8 * U * (MT / WM + NB / (4 / WM)) <= 200 &&
           fp8_tiled_lds_bytes(MT, NB, NS, U) <= kTiledMaxLds &&
           fp8_tiled_lds_bytes(MT, NB, NS, U) >= (size_t)MT * 16 * (NB * 16 + 4) * 4 &&
           (NS - 2) * ((MT * 2 * U + 3) / 4 + (NB * 2 * U + 3) / 4 + 2) < 64;
}

// The arguments of one FP8 call, passed to the FP8 launchers.
struct Fp8Args {
    const void *x, *W, *bias;
    void *out;
    int mode;                 // SKG_FP8_PER_TENSOR or SKG_FP8_MX32
    const float *sx, *sw;     // per-tensor scales (device)
    const uint8_t *xe, *we;   // MX exponents (device)
    int out_f32;              // 1: fp32 output, 0: bf16
    bool qx;                  // x is bf16, quantised on load with sx (DOT only)
};

// Host-side validation and planning (plan.cpp).  No HIP calls.
int check_sizes(int M, int N, int K, int dtype);
int complete_plan(int M, int N, int K, int dtype, SkgPlan *p);
int default_plan(int M, int N, int K, int dtype, int num_cus, SkgPlan *p);
bool table_plan(int M, int N, int K, int dtype, SkgPlan *p);

// Workspace needed by a completed plan (api.hip): fp32 split partials, and
// room for M*K e4m3 codes where x is quantised before the GEMM (placed after
// the partials, which are then rounded up to 64 floats).
size_t workspace_floats(const SkgPlan &p, int M, int N);
size_t round_floats(size_t floats);
size_t quant_floats(int M, int K);
int tile_count(const SkgPlan &p, int N);

// Launchers (kernels_*.hip).  Return a hipError_t as int.
// out_f32: 1 writes fp32 outputs, 0 bf16.
int launch_dot(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
               int out_f32, int M, int N, int K, hipStream_t stream);
int launch_rows(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                int out_f32, int M, int N, int K, hipStream_t stream);
int launch_splitk(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                  int out_f32, float *ws, unsigned *tickets, int M, int N, int K,
                  hipStream_t stream);
int launch_tiled(const SkgPlan &p, const void *x, const void *W, const void *bias, void *out,
                 int out_f32, float *ws, unsigned *tickets, int M, int N, int K,
                 hipStream_t stream);
int launch_splitk_reduce(const float *ws, const void *bias, void *out, int out_f32, int M, int N,
                         int S, hipStream_t stream, const float *sx = nullptr,
                         const float *sw = nullptr);
// Static e4m3 quantisation of n bf16 values with the device scale s.
int launch_quant_e4m3(const void *x, const float *s, void *q, long n, hipStream_t stream);
int launch_fp8(const SkgPlan &p, const Fp8Args &a, float *ws, unsigned *tickets, int M, int N,
               int K, hipStream_t stream);
int launch_fp8_tiled(const SkgPlan &p, const Fp8Args &a, float *ws, unsigned *tickets, int M,
                     int N, int K, hipStream_t stream);
int launch_fp8_rows(const SkgPlan &p, const Fp8Args &a, int M, int N, int K, hipStream_t stream);
// Whether the FP8 dot kernel that quantises bf16 x on load exists for (M, V)
// and accepts workgroups of `threads` (its registers bound it lower than the
// plain FP8 dot kernel).
bool fp8_dot_quant_ok(int M, int C, int V, int threads);
bool fp8_mfma_quant_ok(int MT, int NB, int D, int threads);

}  // namespace skg
