/*
 * skinny_gemm.h -- C ABI of the small-M ("skinny") GEMM library for AMD
 * MI355X (gfx950).
 *
 * The operation (every entry point):
 *
 *     out[m, n] = bf16( sum_k x[m, k] * W[n, k]  (+ bias[n]) )
 *
 * with fp32 accumulation and one rounding (round-to-nearest-even) of the
 * fp32 result to bf16, the bias added in fp32 before that rounding.
 * Defined on the "sglang PR #30117" page, key source snippet (kernel header
 * comment: x[M,K] times weight[N,K] transposed, optional bias[N], bf16
 * in/out, fp32 accumulation) and used as the MoE router GEMM on the
 * "vllm PR #42562" page (summary and impl. items 1-3).
 *
 * Layouts.  Every tensor is dense and row-major with no strides:
 *   x[M, K], W[N, K], bias[N], out[M, N].
 * W[N, K] row-major is the same memory as the column-major [K, N] weight of
 * the "sglang PR #28333" page's FP8 snippet.  Callers make tensors
 * contiguous; the library never reads strides (the "sglang PR #30117"
 * review found leading-dimension detection error-prone).
 *
 * Domain.  1 <= M <= 512, N >= 1, K >= 8 and K % 8 == 0 (bf16) so every row
 * starts 16-byte aligned (the "vllm PR #48774" page keeps only router shapes
 * with K a multiple of 8; the "vllm PR #42562" review settles on 16-byte
 * alignment for 128-bit loads).  Above M = 128 (the larger-M regime of the
 * "sglang PR #34042" page's M = 512 comparison) only the tiled kernels run,
 * in row blocks of 128, and K must also be a multiple of 32 (bf16) or 128
 * (FP8).  M * N < 2^31, and a plan must exist whose launch counts fewer
 * than 2^32 work-items (grid * threads; about N * 256 for the dot kernel
 * at large K).  M == 0 or N == 0 is a successful no-op.
 * Anything else out of domain returns SKG_ERR_UNSUPPORTED: there is no
 * silent fallback (the "sglang PR #34042" page: an explicit request errors
 * instead of falling back).
 *
 * Pointers.  All tensor pointers are DEVICE pointers on the current HIP
 * device.  x and W must be 16-byte aligned; bias and out 2-byte aligned.
 * out must not overlap x, W or bias.  The caller owns every tensor; the
 * library never frees or retains them past the call.
 *
 * Streams.  Work is enqueued on `stream` (0 = the null stream) and the call
 * returns without synchronising.  Completion follows stream order.  A call
 * allocates nothing once workspace is reserved (skinny_gemm_reserve), so it
 * may be captured into a HIP graph.
 *
 * Errors.  Every entry point returns SKG_OK (0) or a negative SKG_ERR_*.
 * Arguments are validated on the host before any HIP call, so a rejected
 * call touches no device state.  SKG_ERR_HIP reports a launch failure
 * (hipGetLastError after the launch).
 *
 * Threads.  The planner and its table are immutable; calls from several
 * host threads are safe.  Split-K calls use a workspace owned per (device,
 * stream), and for hipStreamPerThread (one handle, a different stream in
 * every host thread) per (device, calling thread): calls that overlap in
 * time on the same workspace race, calls on different streams do not.  A
 * graph captured on a stream keeps that stream's workspace: replay it on
 * its capture stream, or at least never while other calls that use that
 * workspace run.
 */
#ifndef SKINNY_GEMM_H
#define SKINNY_GEMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
#define SKG_OK 0
#define SKG_ERR_INVALID_ARG (-1) /* NULL pointer, negative size, overlap, bad plan */
#define SKG_ERR_ALIGNMENT (-2)   /* pointer not aligned as required above */
#define SKG_ERR_UNSUPPORTED (-3) /* outside the domain, or a mode not built */
#define SKG_ERR_WORKSPACE (-4)   /* split-K workspace too small during graph capture */
#define SKG_ERR_HIP (-5)         /* HIP reported an error */

/* ------------------------------------------------------------ enums */
#define SKG_DTYPE_BF16 0
#define SKG_DTYPE_FP8 1
#define SKG_DTYPE_F32 2 /* output dtype only: fp32 logits */
/* Planning dtype for FP8 with MX block scales (skinny_gemm_plan and
 * skinny_gemm_plan_complete only): the same kernels and limits as
 * SKG_DTYPE_FP8 with K % 32 == 0, but its own dispatch-table entries, since
 * the two scale modes are fastest with different plans.  The GEMM entry
 * points take the mode from skinny_fp8_scales. */
#define SKG_DTYPE_FP8_MX 3

#define SKG_FP8_PER_TENSOR 1
#define SKG_FP8_MX32 2

#define SKG_KIND_DOT 1    /* dot-product kernel: whole K per workgroup */
#define SKG_KIND_SPLITK 2 /* MFMA kernel, K split over workgroups */
#define SKG_KIND_TILED 3  /* MFMA kernel with x and W tiles streamed into an LDS ring
                             (K % 32 == 0), K split
                             over workgroups (wide column tiles, larger M) */
#define SKG_KIND_ROWS 4   /* bf16, M <= 64: MFMA kernel streaming whole row
                             segments (1 KB, or 512 bytes with SKG_FLAG_ROWS_HALF)
                             of x and W into an LDS ring; a workgroup owns 8 or 16
                             columns and the whole K, its waves split the K steps
                             (no cross-workgroup reduction) */

#define SKG_REDUCE_NONE 0  /* splits == 1: no cross-workgroup reduction */
#define SKG_REDUCE_LAST 1  /* the last workgroup to finish a tile reduces it */
#define SKG_REDUCE_KERNEL 2 /* a second kernel reduces every tile */

#define SKG_FLAG_DOT2 1 /* DOT: multiply-add with v_dot2c_f32_bf16 (bf16 pairs, fp32
                          accumulator; not rounded per IEEE step: an accumulator far
                          below both products can be lost, error ~2^-24 of the
                          largest term) */
#define SKG_FLAG_TILED_WIDE 2 /* TILED: LDS stages of four 32-wide K steps (256 bytes of
                                each row) instead of two (128 bytes) */
#define SKG_FLAG_DOT_XLDS 4 /* DOT (bf16, together with SKG_FLAG_DOT2): all M rows
                              of x staged in LDS once per workgroup; each wave
                              owns cols / (threads / 64) columns (1, 2 or 4) over
                              the whole K, so `cols` may be up to 64 and no
                              cross-wave reduction is needed.  Needs K = 512 * V
                              with V in {4, 6, 8, 12, 14, 16} and M * K * 2 bytes
                              of LDS (at most 160 KB - 256). */

#define SKG_FLAG_ROWS_HALF 8 /* ROWS: stages of 256 K elements (512 bytes of each row)
                               instead of 512; room in LDS for more rows of x */

#define SKG_FLAG_DOT_WFIRST 16 /* DOT (bf16, together with SKG_FLAG_DOT2, without
                                 SKG_FLAG_DOT_XLDS): every W load is issued before
                                 the first x load instead of in the compiler's
                                 interleaved order.  Same arithmetic, same bits;
                                 only the time differs, by shape. */

#define SKG_MAX_M 512 /* above 128 rows only tiled plans (K % 32, FP8 K % 128) */

/* FP8 scales (host struct; its pointers are DEVICE pointers).
 *  mode SKG_FP8_PER_TENSOR: sx, sw -> one fp32 each (the "sglang PR #28333"
 *    page's bmm_fp8 call: x_scale and weight_scale as one-element tensors);
 *    out = bf16(sx * sw * sum(xq * wq) + bias), the scale product applied once.
 *  mode SKG_FP8_MX32: x_e8m0[M, K/32], w_e8m0[N, K/32], row-major, one e8m0
 *    exponent per 32 consecutive K of a row (the MX block scaling of the
 *    "sglang PR #34042" page, stored plainly instead of swizzled). */
typedef struct skinny_fp8_scales {
    int mode;
    const float *sx;
    const float *sw;
    const uint8_t *x_e8m0;
    const uint8_t *w_e8m0;
} skinny_fp8_scales;

/* A launch plan: what the dispatcher chose for one (M, N, K, dtype).
 * The "vllm PR #42562" and "vllm PR #48774" pages key their compiled
 * kernels by (backend, M, K, block size, split_k, stages); this is the same
 * idea as a plain struct.  Fields marked (derived) are filled in by the
 * library from the others. */
typedef struct SkgPlan {
    int kind;     /* SKG_KIND_DOT, SKG_KIND_SPLITK, SKG_KIND_TILED or SKG_KIND_ROWS */
    int threads;  /* workgroup size, a multiple of 64, <= 1024 (TILED: 256;
                     ROWS: 256 or 512) */
    int cols;     /* DOT: output columns per workgroup (bf16: 1-4; FP8: 1, 2, 4;
                     with SKG_FLAG_DOT_XLDS: 1, 2 or 4 per wave);
                     SPLITK: 16-column blocks per workgroup (1, 2, 4);
                     TILED: 16-column blocks per workgroup (1, 2, 4, 8, 16);
                     ROWS: output columns per workgroup (8, 16; bf16 up to 16
                     rows also 10, 12) */
    int splits;   /* SPLITK, TILED: number of K chunks S (>= 1); DOT, ROWS: 1 */
    int depth;    /* SPLITK: 32-wide K steps a wave keeps in flight (1, 2, 4, 8);
                     TILED: stages of the LDS ring (2, 3, 4, 5, 6, 8);
                     ROWS: stages of the LDS ring (3, 4, 5, 6);
                     DOT: 16-byte vectors per thread per column (derived) */
    int waves_m;  /* TILED: waves along M (1, 2, 4; the other 4/waves_m waves
                     split the columns); 0 = chosen by the library */
    int reduce;   /* SKG_REDUCE_*; NONE iff splits == 1 */
    int flags;    /* SKG_FLAG_* */
    int k_chunk;  /* (derived) SPLITK, TILED: K elements per split, multiple of 32 */
    int m_tiles;  /* TILED: 16-row tiles per row block.  0 asks for the power of
                     two (1, 2, 4, 8) at or above ceil(M / 16), capped at 8 (more
                     rows: row blocks of 128); a smaller power of two splits the
                     rows into ceil(M / (16 * m_tiles)) row blocks (wider,
                     shorter tiles).  (derived) for the other kinds: SPLITK
                     ceil(M / 16), DOT and ROWS 1 */
    int grid;     /* (derived) workgroups in the main launch */
    int from_table; /* (derived) 1 when the tuned table supplied the plan */
} SkgPlan;

/* bf16 GEMM.  `scales` must be NULL (it exists so both entry points share one
 * argument order).  Picks a plan with skinny_gemm_plan and launches it. */
int skinny_gemm_bf16(const void *x, const void *W, const void *bias, const void *scales,
                     void *out, int M, int N, int K, hipStream_t stream);

/* skinny_gemm_bf16 for callers that cannot allocate device memory: code
 * under HIP graph capture with no workspace reserved, serving loops and
 * harnesses that forbid hipMalloc.  Same arguments, plans and results as
 * skinny_gemm_bf16 (bit for bit), and it never calls hipMalloc, hipFree or
 * an allocating routine.  Split-K and tiled plans keep their fp32 partials
 * in a fixed device array inside the library, 8 MiB (2^21 floats) per GPU,
 * held from the first call on that GPU until the process ends; a plan whose
 * partials (splits * M * N floats) exceed it returns SKG_ERR_WORKSPACE and
 * launches nothing.  Such plans reduce with the second kernel (a plan that
 * would use the last-arriver reduction is switched to it: same sums, same
 * order, same bits), so nothing in the array has to start at zero.  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (on any streams) race and give wrong results; calls ordered on
 * one stream do not.  A GPU's first call looks up the array's device
 * address (hipGetSymbolAddress, no allocation): make one call on each GPU
 * before capturing a graph there. */
int skinny_gemm_bf16_noalloc(const void *x, const void *W, const void *bias,
                             const void *scales, void *out, int M, int N, int K,
                             hipStream_t stream);

/* FP8 e4m3fn GEMM with bf16 bias and output; `scales` is a HOST pointer to
 * the struct above (its pointers are device pointers; sx, sw 4-byte
 * aligned).  x[M,K] and W[N,K] are e4m3fn bytes, row-major, 16-byte
 * aligned.  K % 16 == 0 (per-tensor) or K % 32 == 0 (MX).  Accumulation in
 * fp32; per-tensor mode multiplies by sx*sw once before the bias; MX mode
 * scales every 32-element block product by its two exponents.  An e8m0 byte
 * 0xFF (NaN) makes the outputs that use it NaN. */
int skinny_gemm_fp8(const void *x, const void *W, const void *bias,
                    const skinny_fp8_scales *scales, void *out, int M, int N, int K,
                    hipStream_t stream);

/* FP8 GEMM with a caller-made plan (any kind; completed as by
 * skinny_gemm_plan_complete with SKG_DTYPE_FP8). */
int skinny_gemm_fp8_planned(const void *x, const void *W, const void *bias,
                            const skinny_fp8_scales *scales, void *out, int M, int N, int K,
                            const SkgPlan *plan, hipStream_t stream);

/* The dispatcher's decision for (M, N, K, dtype), written to *plan; no HIP
 * call.  The "vllm PR #48774" page's rule: a tuned (K, N) -> {M: config}
 * table first (ours, from a sweep on MI355X), else a default rule.
 *   bf16: the dot product when M <= 4 or K < 2048 (the page's threshold),
 *         or up to 16 rows when N <= 512 and M * K <= 98304; else the
 *         tiled MFMA kernel; split-K where K is not a multiple of 32.
 *   FP8:  the dot product when M <= 4; from 5 to 16 rows split-K without
 *         a K split when N >= 2048, else the tiled kernel; above 16 rows
 *         the tiled kernel (K % 128 == 0), else split-K.
 * dtype: SKG_DTYPE_BF16,
 * SKG_DTYPE_FP8 (per-tensor scales) or SKG_DTYPE_FP8_MX (MX block scales;
 * skinny_gemm_fp8 plans with it when given SKG_FP8_MX32).  Returns SKG_OK, or
 * the error the GEMM call would return for these sizes. */
int skinny_gemm_plan(int M, int N, int K, int dtype, SkgPlan *plan);

/* Checks a caller-made plan for (M, N, K, dtype) and fills its derived
 * fields.  SKG_ERR_INVALID_ARG if the plan cannot cover the problem or
 * exceeds a kernel limit (among them: grid * threads below 2^32, the
 * launch's 32-bit work-item count).  No HIP call. */
int skinny_gemm_plan_complete(int M, int N, int K, int dtype, SkgPlan *plan);

/* bf16 GEMM with a caller-made plan (completed as above): for sweeps and
 * tests that must exercise a given kernel.  Same contract otherwise. */
int skinny_gemm_bf16_planned(const void *x, const void *W, const void *bias, void *out,
                             int M, int N, int K, const SkgPlan *plan, hipStream_t stream);

/* Reserves workspace for `stream` on the current device, large enough for
 * any call with M <= max_M, N <= max_N, K <= max_K and a plan of at most
 * max_S splits: the split partials (fp32 [S][M][N]) plus, for
 * skinny_gemm_fp8_quant plans that quantise x before the GEMM, room for its
 * M*K e4m3 codes.  max_K = 0 reserves no such room (enough for every other
 * entry point).  Allocates (hipMalloc) and zeroes the tile counters; call it
 * before graph capture.  Outside capture a call that needs more grows the
 * workspace itself; during capture it returns SKG_ERR_WORKSPACE instead.
 * SKG_ERR_INVALID_ARG if max_M, max_N or max_S is below 1, max_M exceeds
 * SKG_MAX_M, max_S exceeds 256, max_K is negative, or max_K * 1024 bytes
 * reaches 2 GiB. */
int skinny_gemm_reserve(int max_M, int max_N, int max_K, int max_S, hipStream_t stream);

/* bf16 GEMM with fp32 output (router logits): out[m, n] = fp32 value of the
 * fp32-accumulated sum plus bias, with no bf16 rounding.  The router split-K
 * kernel of the "vllm PR #42562" page writes its logits in fp32 (its output
 * dtype is fixed to float).  out: DEVICE fp32 [M, N], 4-byte aligned, not
 * overlapping x, W or bias; everything else as skinny_gemm_bf16, with the
 * same plans (the table's bf16 entries). */
int skinny_gemm_bf16_f32(const void *x, const void *W, const void *bias, float *out, int M,
                         int N, int K, hipStream_t stream);

/* The same with a caller-made plan (as skinny_gemm_bf16_planned). */
int skinny_gemm_bf16_f32_planned(const void *x, const void *W, const void *bias, float *out,
                                 int M, int N, int K, const SkgPlan *plan, hipStream_t stream);

/* Per-tensor FP8 GEMM on bf16 activations, quantised statically on the way:
 *     q[m, k] = e4m3( clamp( x[m, k] * (1 / sx), -448, 448 ) )   (in fp32)
 *     out     = sx * sw * sum_k q[m, k] * W[n, k]  (+ bias[n])
 * The quantisation is the static FP8 quant kernel of the "sglang PR #28333"
 * page (a given scale, one reciprocal, a product, a clamp, the cast to e4m3
 * with round-to-nearest-even), followed by that page's per-tensor GEMM.
 * The dot-product plan quantises x as it loads it, so the call is one
 * launch (the automatic dot plan then shares each x load over four or two
 * columns where it can).  A caller's MFMA split-K plan (up to 32 rows) does
 * too; the automatic plan, and every other plan, quantises x into the
 * workspace first (a second launch: faster than quantising in every
 * workgroup once the split-K kernel takes over from the dot kernel).  x: DEVICE bf16 [M, K], 16-byte aligned; W: DEVICE e4m3fn
 * [N, K], 16-byte aligned; sx, sw: DEVICE fp32 scalars, 4-byte aligned;
 * K % 16 == 0.  out_dtype: SKG_DTYPE_BF16 (bf16 out, 2-byte aligned) or
 * SKG_DTYPE_F32 (fp32 out, 4-byte aligned).  NaN in x gives NaN outputs. */
int skinny_gemm_fp8_quant(const void *x, const void *W, const void *bias, const float *sx,
                          const float *sw, void *out, int out_dtype, int M, int N, int K,
                          hipStream_t stream);

/* The same with a caller-made FP8 plan (as skinny_gemm_fp8_planned). */
int skinny_gemm_fp8_quant_planned(const void *x, const void *W, const void *bias,
                                  const float *sx, const float *sw, void *out, int out_dtype,
                                  int M, int N, int K, const SkgPlan *plan, hipStream_t stream);

/* The static quantisation alone: q[i] = e4m3(clamp(x[i] * (1/s), -448,
 * 448)) for i < n, as in skinny_gemm_fp8_quant.  x: DEVICE bf16 [n],
 * q: DEVICE bytes [n], both 16-byte aligned and disjoint; s: DEVICE fp32,
 * 4-byte aligned.  n == 0 is a no-op; n < 0 is SKG_ERR_INVALID_ARG. */
int skinny_quant_e4m3(const void *x, const float *s, void *q, long n, hipStream_t stream);

/* Frees every workspace the library holds, on each device it holds one on,
 * after synchronising those devices (and only those); the current device is
 * the same afterwards.  With nothing held it makes no HIP call.  No call may
 * be in flight. */
int skinny_gemm_release_all(void);

/* Human-readable name of a status code (static storage). */
const char *skinny_gemm_status_string(int status);

/* skinny_gemm_plan for a device with `num_cus` compute units, without
 * touching any device: the dispatch logic as a pure function, for tests
 * with a made-up device.  The tuned table applies only when num_cus is the
 * MI355X's 256; other counts take the default rule, sized to num_cus.
 * skinny_gemm_plan is this function at 256 CUs. */
int skinny_gemm_plan_on(int M, int N, int K, int dtype, int num_cus, SkgPlan *plan);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_GEMM_H */
