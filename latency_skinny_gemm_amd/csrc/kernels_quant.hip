// kernels_quant.hip -- static per-tensor FP8 (e4m3) quantisation of bf16
// activations, the standalone form of the quantisation that the FP8 dot
// kernel fuses into its x loads.
//
// "sglang PR #28333" page, static FP8 quant kernel: with a given scale s,
// q = e4m3(clamp(x * (1/s), -448, 448)), evaluated in fp32 (one reciprocal,
// one product, round to nearest e4m3, ties to even).
#include "device_common.h"
#include "internal.h"

namespace skg {

// Thread t converts elements [16t, 16t+16): two 16-byte loads of bf16 and
// one 16-byte store of codes; the last partial group goes element by element.
__global__ void __launch_bounds__(256)
    quant_e4m3_kernel(const uint16_t *__restrict__ x, long n, const float *__restrict__ s,
                      uint8_t *__restrict__ q) {
    const float inv = 1.0f / s[0];  // correctly rounded (no fast-math)
    const long i0 = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 16;
    if (i0 >= n) return;
    if (i0 + 16 <= n) {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(x + i0);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(x + i0 + 8);
        *reinterpret_cast<u32x4 *>(q + i0) = quant16_e4m3(lo, hi, inv);
        return;
    }
    for (long i = i0; i < n; ++i) {
        const unsigned w = x[i];
        q[i] = (uint8_t)(quant_pair<false>(w, inv, 0) & 0xFF);
    }
}

int launch_quant_e4m3(const void *x, const float *s, void *q, long n, hipStream_t stream) {
    if (n <= 0) return (int)hipSuccess;
    const long groups = (n + 15) / 16;
    hipLaunchKernelGGL(quant_e4m3_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                       stream, (const uint16_t *)x, n, s, (uint8_t *)q);
    return (int)hipGetLastError();
}

}  // namespace skg
