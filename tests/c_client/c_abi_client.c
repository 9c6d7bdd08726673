/*
 * c_abi_client.c -- a client of the C ABI with no Python and no torch: it
 * allocates with the HIP runtime, calls skinny_gemm_bf16 (the automatic
 * plan) and skinny_gemm_bf16_planned (a split-K and a tiled plan) on its own
 * stream, and checks every output exactly against a closed form:
 *
 *   x[m, k] = (k % 7) - 3 + m        small integers, exact in bf16
 *   W[n, k] = 1 if k == (5 n) % K    one-hot rows
 *   bias[n] = (n % 3) / 2
 *   out[m, n] = x[m, (5 n) % K] + bias[n]   (a half-integer below 16: exact)
 *
 * Exit status 0 when every call returns SKG_OK and every output matches.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "skinny_gemm.h"

static uint16_t bf16_bits(float f) { /* exact for the small values used here */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static float bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

#define HIP_OK(call)                                                         \
    do {                                                                     \
        hipError_t e_ = (call);                                              \
        if (e_ != hipSuccess) {                                              \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); \
            return 2;                                                        \
        }                                                                    \
    } while (0)

static int check(const char *what, const uint16_t *out, int M, int N, int K) {
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            const float want = (float)(((5 * n) % K) % 7 - 3 + m) + (float)(n % 3) * 0.5f;
            const float got = bf16_value(out[(size_t)m * N + n]);
            if (got != want) {
                fprintf(stderr, "%s: out[%d][%d] = %g, want %g\n", what, m, n, got, want);
                return 1;
            }
        }
    return 0;
}

int main(void) {
    const int M = 5, N = 300, K = 2880;
    uint16_t *hx = malloc((size_t)M * K * 2), *hw = calloc((size_t)N * K, 2);
    uint16_t *hb = malloc((size_t)N * 2), *ho = malloc((size_t)M * N * 2);
    if (!hx || !hw || !hb || !ho) return 2;
    for (int m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) hx[(size_t)m * K + k] = bf16_bits((float)(k % 7 - 3 + m));
    for (int n = 0; n < N; ++n) {
        hw[(size_t)n * K + (5 * n) % K] = bf16_bits(1.0f);
        hb[n] = bf16_bits((float)(n % 3) * 0.5f);
    }
    void *dx, *dw, *db, *dout;
    HIP_OK(hipMalloc(&dx, (size_t)M * K * 2));
    HIP_OK(hipMalloc(&dw, (size_t)N * K * 2));
    HIP_OK(hipMalloc(&db, (size_t)N * 2));
    HIP_OK(hipMalloc(&dout, (size_t)M * N * 2));
    HIP_OK(hipMemcpy(dx, hx, (size_t)M * K * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dw, hw, (size_t)N * K * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(db, hb, (size_t)N * 2, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    int failed = 0;
    /* the automatic plan */
    int rc = skinny_gemm_bf16(dx, dw, db, NULL, dout, M, N, K, stream);
    if (rc != SKG_OK) {
        fprintf(stderr, "skinny_gemm_bf16: %s\n", skinny_gemm_status_string(rc));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(ho, dout, (size_t)M * N * 2, hipMemcpyDeviceToHost));
    failed |= check("automatic plan", ho, M, N, K);

    /* two caller-made plans: split-K (second-kernel reduction) and tiled */
    SkgPlan plans[2];
    memset(plans, 0, sizeof plans);
    plans[0].kind = SKG_KIND_SPLITK;
    plans[0].threads = 256;
    plans[0].cols = 1;
    plans[0].splits = 6;
    plans[0].depth = 2;
    plans[0].reduce = SKG_REDUCE_KERNEL;
    plans[1].kind = SKG_KIND_TILED;
    plans[1].threads = 256;
    plans[1].cols = 4;
    plans[1].splits = 3;
    plans[1].depth = 3;
    plans[1].reduce = SKG_REDUCE_KERNEL;
    const char *names[2] = {"split-K plan", "tiled plan"};
    rc = skinny_gemm_reserve(M, N, K, 8, stream);
    if (rc != SKG_OK) {
        fprintf(stderr, "skinny_gemm_reserve: %s\n", skinny_gemm_status_string(rc));
        return 1;
    }
    for (int i = 0; i < 2; ++i) {
        HIP_OK(hipMemset(dout, 0, (size_t)M * N * 2));
        rc = skinny_gemm_plan_complete(M, N, K, SKG_DTYPE_BF16, &plans[i]);
        if (rc == SKG_OK) rc = skinny_gemm_bf16_planned(dx, dw, db, dout, M, N, K, &plans[i], stream);
        if (rc != SKG_OK) {
            fprintf(stderr, "%s: %s\n", names[i], skinny_gemm_status_string(rc));
            return 1;
        }
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(ho, dout, (size_t)M * N * 2, hipMemcpyDeviceToHost));
        failed |= check(names[i], ho, M, N, K);
    }
    /* an out-of-domain call is refused before any HIP work */
    if (skinny_gemm_bf16(dx, dw, db, NULL, dout, M, N, 2884, stream) != SKG_ERR_UNSUPPORTED) {
        fprintf(stderr, "K %% 8 != 0 was not refused\n");
        failed = 1;
    }
    (void)skinny_gemm_release_all();
    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dw));
    HIP_OK(hipFree(db));
    HIP_OK(hipFree(dout));
    free(hx);
    free(hw);
    free(hb);
    free(ho);
    if (!failed) printf("c-abi client: ok\n");
    return failed;
}
