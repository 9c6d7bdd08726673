// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skg {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- buffers
// A raw buffer resource (gfx9 descriptor word 3 = 0x00020000: 32-bit
// dwords, no swizzle).  A load whose byte offset is at or past num_records
// returns zeros and touches no memory; kOOB is such an offset for every
// buffer the planner admits (all are < 2^31 bytes, and offsets added to kOOB
// stay below 2^32).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr unsigned kOOB = 0x80000000u;

__device__ __forceinline__ Rsrc make_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// cache-policy bits of the buffer instruction: bit 1 = nt (streaming),
// bit 4 = sc1.  An sc1 access is what an agent-scope relaxed atomic load or
// store of a dword compiles to on gfx950 (global_load/store_dword ... sc1):
// a 16-byte sc1 access gives each of its dwords that same coherence.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;
constexpr int kCacheCoherent = 16;

template <int POLICY>
__device__ __forceinline__ u32x4 load16(Rsrc r, unsigned byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, POLICY);
}

// ---------------------------------------------------------------- LDS
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer straight into LDS at dst + 16 * lane
// (dst wave-uniform; LDS-DMA, no VGPR round trip).  Kept out of the kernel
// body: used there directly, the builtin made the host pass drop the
// kernels' launch stubs.
template <int POLICY>
__device__ __forceinline__ void lds_load16(Rsrc r, unsigned char *dst, unsigned off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, off, 0, 0, POLICY);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8 = 0).  Vector memory
// loads return in issue order, so vmcnt(N) means all but this wave's last
// N loads have landed (in registers or, for LDS-DMA, in LDS).  Waiting for
// lgkmcnt too means this wave's own LDS reads have returned, so a barrier
// after it also orders them before later LDS writes by any wave.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}

// s_barrier without a memory fence.  The asm statements keep the compiler
// from moving LDS accesses across it; the hardware ordering comes from the
// explicit vmcnt wait that precedes it.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(unsigned v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(unsigned v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((unsigned)b << 16); }

// fp32 -> bf16, round to nearest, ties to even.  NaN stays NaN (quiet bit
// set); overflow carries into the exponent and gives +-inf.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    unsigned u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- epilogue operands
// The bias does not depend on the main loop, so the kernels load it at the
// start (the second-pass reduction also its FP8 per-tensor scales) and its
// memory latency hides under the operand stream; loaded in the epilogue,
// each value was one more round trip after the last product (0.1-0.6 us a
// call, measured).  The loads go through buffer views: a null pointer gives
// a zero-size view whose loads return 0 and touch no memory, and a column
// n >= N, or live = false (kOOB), also returns 0 without touching memory.
// In a ring kernel they are issued in the prologue, before the ring loop:
// a load older than the ring's only makes the in-order vmcnt waits that
// count the ring's loads stricter.
// Callers keep testing the pointer before adding or multiplying: s + 0.0f
// is not s when s = -0.0f.
__device__ __forceinline__ Rsrc bias_rsrc(const uint16_t *bias, int N) {
    return make_rsrc(bias, bias ? (unsigned)N * 2u : 0u);
}
// The bits are returned zero-extended in a dword: kept as 16-bit values,
// the compiler packed pairs of them into one register right after the loads
// and so waited for the loads there.
__device__ __forceinline__ unsigned load_bias_bits(Rsrc br, int n, bool live = true) {
    return __builtin_amdgcn_raw_buffer_load_b16(br, live ? (unsigned)n * 2u : kOOB, 0,
                                                kCacheDefault);
}
__device__ __forceinline__ float load_scale(const float *p) {
    return __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p, p ? 4u : 0u), 0u, 0, kCacheDefault));
}

// The final store of one output element: bf16 (one RNE rounding of the fp32
// value) or, for fp32 outputs, the fp32 value itself.
__device__ __forceinline__ void store_out(void *out, size_t i, float v, int out_f32) {
    if (out_f32)
        static_cast<float *>(out)[i] = v;
    else
        static_cast<uint16_t *>(out)[i] = f32_to_bf16_rne(v);
}

// ---------------------------------------------------------------- FP8 quant
// Static per-tensor FP8 quantisation ("sglang PR #28333" page, the static
// FP8 quant kernel): q = e4m3(clamp(x * inv, -448, 448)) with inv = 1/s, in
// fp32.  The clamp is written with comparisons so that NaN passes through
// (min/max would replace it); v_cvt_pk_fp8_f32 rounds to the nearest e4m3
// value, ties to even (checked code by code against the reference).
__device__ __forceinline__ float quant_clamp(float v) {
    return v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v);
}

// Two bf16 values (low half first) -> two e4m3 codes in the low or high
// 16 bits of `old`.
template <bool HIGH>
__device__ __forceinline__ int quant_pair(unsigned w, float inv, int old) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(quant_clamp(bf16_lo(w) * inv),
                                           quant_clamp(bf16_hi(w) * inv), old, HIGH);
}

// 16 bf16 values (lo: elements 0-7, hi: 8-15) -> 16 e4m3 codes, byte k =
// element k.
__device__ __forceinline__ u32x4 quant16_e4m3(u32x4 lo, u32x4 hi, float inv) {
    u32x4 r;
    r.x = (unsigned)quant_pair<true>(lo.y, inv, quant_pair<false>(lo.x, inv, 0));
    r.y = (unsigned)quant_pair<true>(lo.w, inv, quant_pair<false>(lo.z, inv, 0));
    r.z = (unsigned)quant_pair<true>(hi.y, inv, quant_pair<false>(hi.x, inv, 0));
    r.w = (unsigned)quant_pair<true>(hi.w, inv, quant_pair<false>(hi.z, inv, 0));
    return r;
}

// acc + sum of the 8 products of two 16-byte bf16 vectors, k ascending,
// each product exact in fp32 and each addition rounded once (fused).
__device__ __forceinline__ float dot8_fma(u32x4 a, u32x4 b, float acc) {
    acc = __builtin_fmaf(bf16_lo(a.x), bf16_lo(b.x), acc);
    acc = __builtin_fmaf(bf16_hi(a.x), bf16_hi(b.x), acc);
    acc = __builtin_fmaf(bf16_lo(a.y), bf16_lo(b.y), acc);
    acc = __builtin_fmaf(bf16_hi(a.y), bf16_hi(b.y), acc);
    acc = __builtin_fmaf(bf16_lo(a.z), bf16_lo(b.z), acc);
    acc = __builtin_fmaf(bf16_hi(a.z), bf16_hi(b.z), acc);
    acc = __builtin_fmaf(bf16_lo(a.w), bf16_lo(b.w), acc);
    acc = __builtin_fmaf(bf16_hi(a.w), bf16_hi(b.w), acc);
    return acc;
}

// acc + the same 8 products with gfx950's bf16 dot instruction (two
// products and the accumulator per instruction, no widening).  Its
// internal sum is not rounded per IEEE step: an accumulator far below the
// two products can be lost (error bounded by ~2^-24 of the largest term).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8_dot2(u32x4 a, u32x4 b, float acc) {
    // Pairs are taken from the 8-element view with shufflevector: bit-casting
    // the 32-bit lanes a.y/a.z/a.w one by one is folded onto a.x by this
    // compiler (every product then uses the first pair).
    const bf16x8 a8 = __builtin_bit_cast(bf16x8, a);
    const bf16x8 b8 = __builtin_bit_cast(bf16x8, b);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a8, a8, 0, 1),
                                          __builtin_shufflevector(b8, b8, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a8, a8, 2, 3),
                                          __builtin_shufflevector(b8, b8, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a8, a8, 4, 5),
                                          __builtin_shufflevector(b8, b8, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a8, a8, 6, 7),
                                          __builtin_shufflevector(b8, b8, 6, 7), acc, false);
    return acc;
}

// Wait until every memory operation this wave issued has completed (for a
// store: acknowledged by the L2).  s_waitcnt with all counters zero.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// ---------------------------------------------------------------- reductions
// sum_{i < n} ld(i), added in ascending i starting from 0.0f.  The loads go
// out in groups of CH before any of them is added, so n partials cost about
// n / CH memory latencies instead of n; the additions keep their order, so
// the bits do not depend on CH.
template <int CH, class Load>
__device__ __forceinline__ float ordered_sum(int n, Load ld) {
    float v = 0.0f;
    for (int i0 = 0; i0 < n; i0 += CH) {
        float t[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) t[i] = (i0 + i < n) ? ld(i0 + i) : 0.0f;
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (i0 + i < n) v += t[i];
    }
    return v;
}

// DPP lane moves within a 16-lane row (gfx9 dpp_ctrl encodings).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane 7-i within 8
constexpr int kDppMirror = 0x140;     // row_mirror: lane 15-i within 16

// Sum over the 64 lanes of a wave, returned in every lane.  A fixed tree:
// pairs, quads, 8-lane halves and 16-lane rows by DPP, then the four rows
// by two butterfly shuffles.  Every lane ends with the same bits (each step
// adds the same two values in either order, and fp addition commutes).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_mov<kDppQuadSwap1>(v);
    v += dpp_mov<kDppQuadSwap2>(v);
    v += dpp_mov<kDppHalfMirror>(v);
    v += dpp_mov<kDppMirror>(v);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// ---------------------------------------------------------------- reduce-scatter
// The wave-wide sums of P = 2^L values that every lane holds (v[0..P-1]),
// each sum landing in its own group of lanes: afterwards v[0] of lane l is
// the sum over all 64 lanes of value index l >> (6 - L).  Six exchange
// levels, in a fixed order: lanes l and l^32, then l and l^16 (the two
// v_permlane*_swap instructions of gfx950), then l and 15-l within a
// 16-lane row (row_mirror), l and 7-l within 8 (row_half_mirror), l^2 and
// l^1 (quad_perm).  At each of the first L levels the lanes whose level bit
// is 1 keep the upper half of the values and the others the lower half, so
// each level halves the values a lane holds; the remaining levels add the
// single value and its partner.  A level pairs the same two lanes for every
// value index, and a pair's sum does not depend on which lane forms it (fp
// addition commutes), so every index is summed by the same tree: the bits
// do not depend on where a value sits in v.  Values of different indices
// are never added together, so padding v with zeros changes nothing.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The partner's x at exchange level LEV (2..5) within a 16-lane row.
template <int LEV>
__device__ __forceinline__ float rs_partner(float x) {
    if constexpr (LEV == 2) return dpp_f<kDppMirror>(x);
    else if constexpr (LEV == 3) return dpp_f<kDppHalfMirror>(x);
    else if constexpr (LEV == 4) return dpp_f<kDppQuadSwap2>(x);
    else return dpp_f<kDppQuadSwap1>(x);
}

// One exchange level: lanes l and its level-LEV partner (l^32, l^16, 15-l
// in a row, 7-l in 8, l^2, l^1).  While a lane still holds more than one
// value it keeps the upper half when its level bit (bit 5 - LEV) is set,
// else the lower half, each added to the partner's copy of the same index.
template <int L, int LEV>
__device__ __forceinline__ void rs_level(float (&v)[1 << L], unsigned lane) {
    constexpr int n = LEV < L ? (1 << (L - LEV)) : 1;  // values held before this level
    if constexpr (LEV < 2) {
        // one swap exchanges the two values of a pair between the halves
        // (rows); r[0] + r[1] is the sum of the index this lane keeps
        constexpr int h = n > 1 ? n / 2 : 1;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const unsigned a = __float_as_uint(v[i]);
            const unsigned b = n > 1 ? __float_as_uint(v[i + (n > 1 ? h : 0)]) : a;
            const auto r = LEV == 0 ? __builtin_amdgcn_permlane32_swap(a, b, false, false)
                                    : __builtin_amdgcn_permlane16_swap(a, b, false, false);
            v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    } else {
        const bool upper = (lane >> (5 - LEV)) & 1u;
        if constexpr (n > 1) {
            constexpr int h = n / 2;
#pragma unroll
            for (int i = 0; i < h; ++i) {
                const float keep = upper ? v[i + h] : v[i];
                const float send = upper ? v[i] : v[i + h];
                v[i] = keep + rs_partner<LEV>(send);
            }
        } else {
            v[0] = v[0] + rs_partner<LEV>(v[0]);
        }
    }
}

template <int L>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[1 << L]) {
    static_assert(L >= 0 && L <= 6, "at most 64 values per lane");
    const unsigned lane = threadIdx.x & 63u;
    rs_level<L, 0>(v, lane);
    rs_level<L, 1>(v, lane);
    rs_level<L, 2>(v, lane);
    rs_level<L, 3>(v, lane);
    rs_level<L, 4>(v, lane);
    rs_level<L, 5>(v, lane);
    return v[0];
}

}  // namespace skg
