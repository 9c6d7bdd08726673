// api.hip -- the C ABI: argument checks, workspace, and launches.
//
// Checks run on the host before any HIP call, so a rejected call changes no
// device state (and the checks run on machines without a GPU).  The dtype
// guards follow the "vllm PR #42562" review (bf16 weights and activations
// only on the bf16 path); the "sglang PR #34042" page's rule that an
// explicit request errors rather than falling back is why every unsupported
// case returns a status instead of routing elsewhere.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "internal.h"

namespace skg {

namespace {

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void *a, size_t abytes, const void *b, size_t bbytes) {
    if (!a || !b) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// Pointer checks shared by the bf16 entry points (sizes already checked and
// M, N > 0).  out_f32: out holds fp32 (4-byte) elements instead of bf16.
int check_pointers_bf16(const void *x, const void *W, const void *bias, void *out, int M, int N,
                        int K, int out_f32 = 0) {
    if (!x || !W || !out) return SKG_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(W, 16)) return SKG_ERR_ALIGNMENT;
    if (!aligned(out, out_f32 ? 4 : 2) || (bias && !aligned(bias, 2))) return SKG_ERR_ALIGNMENT;
    const size_t ob = (size_t)M * N * (out_f32 ? 4 : 2);
    if (overlap(out, ob, x, (size_t)M * K * 2) || overlap(out, ob, W, (size_t)N * K * 2) ||
        overlap(out, ob, bias, (size_t)N * 2))
        return SKG_ERR_INVALID_ARG;
    return SKG_OK;
}

// ---------------------------------------------------------------- workspace
// Split-K partials (fp32 [S][M][N]) and one ticket counter per output tile,
// owned per (device, stream, owner).  Counters are zero at rest: the
// workgroup that reduces a tile sets its counter back to zero.  owner is 0
// except for hipStreamPerThread, one handle that names a different stream
// in every host thread: its workspaces belong to the calling thread.
struct Workspace {
    int device;
    hipStream_t stream;
    long owner;
    float *ws;
    size_t ws_floats;
    unsigned *tickets;
    size_t n_tickets;
};

std::mutex g_mu;
std::vector<Workspace> g_ws;
struct Retired {
    int device;
    void *p;
};
std::vector<Retired> g_retired;  // replaced buffers, freed by release_all

// Calls find their workspace without the lock through a per-thread copy of
// the last one they used, valid while no workspace has been replaced or
// freed since: every such change bumps the generation (under the lock).
std::atomic<unsigned> g_generation{1};
struct WorkspaceCache {
    unsigned generation;
    Workspace w;
};
thread_local WorkspaceCache t_cache{0, Workspace{-1, nullptr, 0, nullptr, 0, nullptr, 0}};

// The owner of a stream's workspace: the calling host thread for
// hipStreamPerThread, else 0 (any thread).
long stream_owner(hipStream_t stream) {
    if (stream != hipStreamPerThread) return 0;
    static std::atomic<long> next{1};
    thread_local const long tag = next.fetch_add(1, std::memory_order_relaxed);
    return tag;
}

// Grows w for `stream` (outside graph capture; the caller has synchronised
// the stream, so no kernel still uses a buffer that is retired here).  New
// tile counters are zeroed on `stream` itself: a plain hipMemset is queued
// on the null stream, which a non-blocking stream does not wait for, so the
// first kernel could read uninitialised counters and no workgroup of a tile
// would see itself arrive last.
int grow(Workspace &w, size_t floats, size_t tickets, hipStream_t stream) {
    if (floats > w.ws_floats) {
        float *p = nullptr;
        if (hipMalloc((void **)&p, floats * sizeof(float)) != hipSuccess) return SKG_ERR_HIP;
        if (w.ws) g_retired.push_back(Retired{w.device, w.ws});
        w.ws = p;
        w.ws_floats = floats;
        g_generation.fetch_add(1, std::memory_order_acq_rel);
    }
    if (tickets > w.n_tickets) {
        unsigned *t = nullptr;
        if (hipMalloc((void **)&t, tickets * sizeof(unsigned)) != hipSuccess) return SKG_ERR_HIP;
        if (hipMemsetAsync(t, 0, tickets * sizeof(unsigned), stream) != hipSuccess)
            return SKG_ERR_HIP;
        if (w.tickets) g_retired.push_back(Retired{w.device, w.tickets});
        w.tickets = t;
        w.n_tickets = tickets;
        g_generation.fetch_add(1, std::memory_order_acq_rel);
    }
    return SKG_OK;
}

Workspace *find(int device, hipStream_t stream, long owner) {
    for (auto &w : g_ws)
        if (w.device == device && w.stream == stream && w.owner == owner) return &w;
    return nullptr;
}

// Workspace for this (device, stream, owner) with room for the request.
// Grows it outside graph capture; during capture a short workspace is an
// error.
int acquire(hipStream_t stream, size_t floats, size_t tickets, float **ws, unsigned **tk) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SKG_ERR_HIP;
    const long owner = stream_owner(stream);
    const Workspace &c = t_cache.w;  // fast path: no lock
    if (t_cache.generation == g_generation.load(std::memory_order_acquire) && c.device == dev &&
        c.stream == stream && c.owner == owner && c.ws_floats >= floats &&
        c.n_tickets >= tickets) {
        *ws = c.ws;
        *tk = c.tickets;
        return SKG_OK;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace *w = find(dev, stream, owner);
    if (!w || w->ws_floats < floats || w->n_tickets < tickets) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return SKG_ERR_HIP;
        if (cs != hipStreamCaptureStatusNone) return SKG_ERR_WORKSPACE;
        if (!w) {
            g_ws.push_back(Workspace{dev, stream, owner, nullptr, 0, nullptr, 0});
            w = &g_ws.back();
        }
        // no kernel of this stream may still use a buffer we retire
        if (hipStreamSynchronize(stream) != hipSuccess) return SKG_ERR_HIP;
        int rc = grow(*w, floats, tickets, stream);
        if (rc != SKG_OK) return rc;
    }
    *ws = w->ws;
    *tk = w->tickets;
    t_cache = WorkspaceCache{g_generation.load(std::memory_order_acquire), *w};
    return SKG_OK;
}

int run_bf16(const void *x, const void *W, const void *bias, void *out, int out_f32, int M, int N,
             int K, const SkgPlan &p, hipStream_t stream) {
    if (p.kind == SKG_KIND_DOT || p.kind == SKG_KIND_ROWS) {
        int e = p.kind == SKG_KIND_DOT ? launch_dot(p, x, W, bias, out, out_f32, M, N, K, stream)
                                       : launch_rows(p, x, W, bias, out, out_f32, M, N, K, stream);
        return e == (int)hipSuccess ? SKG_OK : SKG_ERR_HIP;
    }
    float *ws = nullptr;
    unsigned *tk = nullptr;
    if (p.splits > 1) {
        int rc = acquire(stream, workspace_floats(p, M, N), (size_t)tile_count(p, N), &ws, &tk);
        if (rc != SKG_OK) return rc;
    }
    int e = p.kind == SKG_KIND_TILED
                ? launch_tiled(p, x, W, bias, out, out_f32, ws, tk, M, N, K, stream)
                : launch_splitk(p, x, W, bias, out, out_f32, ws, tk, M, N, K, stream);
    return e == (int)hipSuccess ? SKG_OK : SKG_ERR_HIP;
}

// quant_x: x is bf16 and is quantised statically with sc->sx (per-tensor
// mode).  The DOT kernel does it on load, and so does the MFMA split-K
// kernel when fuse_mfma is set; every other plan quantises x into the
// workspace first (one extra launch) and multiplies those codes.
int run_fp8(const void *x, const void *W, const void *bias, const skinny_fp8_scales *sc, void *out,
            int out_f32, bool quant_x, bool fuse_mfma, int M, int N, int K, const SkgPlan &p,
            hipStream_t stream) {
    Fp8Args a{x, W, bias, out, sc->mode, sc->sx, sc->sw, sc->x_e8m0, sc->w_e8m0, out_f32, false};
    const bool fused =
        quant_x && ((p.kind == SKG_KIND_DOT && fp8_dot_quant_ok(M, p.cols, p.depth, p.threads)) ||
                    (fuse_mfma && p.kind == SKG_KIND_SPLITK &&
                     fp8_mfma_quant_ok(p.m_tiles, p.cols, p.depth, p.threads)));
    a.qx = fused;
    // partials first, then the quantised x if needed (the partials then
    // rounded up to 256 bytes, so that x starts aligned)
    const size_t qfloats = (quant_x && !fused) ? quant_floats(M, K) : 0;
    size_t part = (p.kind != SKG_KIND_DOT && p.splits > 1) ? workspace_floats(p, M, N) : 0;
    if (qfloats) part = round_floats(part);
    float *ws = nullptr;
    unsigned *tk = nullptr;
    if (part + qfloats > 0) {
        int rc = acquire(stream, part + qfloats, (size_t)tile_count(p, N), &ws, &tk);
        if (rc != SKG_OK) return rc;
    }
    if (quant_x && !fused) {
        void *q = ws + part;
        if (launch_quant_e4m3(x, sc->sx, q, (long)M * K, stream) != (int)hipSuccess)
            return SKG_ERR_HIP;
        a.x = q;
    }
    int e = launch_fp8(p, a, ws, tk, M, N, K, stream);
    return e == (int)hipSuccess ? SKG_OK : SKG_ERR_HIP;
}

// Checks of the FP8 entry points (sizes already checked, M, N > 0).
// x_bytes: bytes per x element (1 for e4m3 codes, 2 for bf16 to quantise).
int check_fp8(const void *x, const void *W, const void *bias, const skinny_fp8_scales *scales,
              void *out, int out_f32, int x_bytes, int M, int N, int K) {
    if (!scales || !x || !W || !out) return SKG_ERR_INVALID_ARG;
    const int mode = scales->mode;
    if (mode != SKG_FP8_PER_TENSOR && mode != SKG_FP8_MX32) return SKG_ERR_INVALID_ARG;
    if (mode == SKG_FP8_PER_TENSOR && (!scales->sx || !scales->sw)) return SKG_ERR_INVALID_ARG;
    if (mode == SKG_FP8_MX32 && (!scales->x_e8m0 || !scales->w_e8m0)) return SKG_ERR_INVALID_ARG;
    if (mode == SKG_FP8_MX32 && K % 32 != 0) return SKG_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(out, out_f32 ? 4 : 2) ||
        (bias && !aligned(bias, 2)))
        return SKG_ERR_ALIGNMENT;
    if (mode == SKG_FP8_PER_TENSOR && (!aligned(scales->sx, 4) || !aligned(scales->sw, 4)))
        return SKG_ERR_ALIGNMENT;
    const size_t ob = (size_t)M * N * (out_f32 ? 4 : 2);
    if (overlap(out, ob, x, (size_t)M * K * x_bytes) || overlap(out, ob, W, (size_t)N * K) ||
        overlap(out, ob, bias, (size_t)N * 2))
        return SKG_ERR_INVALID_ARG;
    return SKG_OK;
}

// skinny_gemm_fp8_quant and its planned form.
int fp8_quant_common(const void *x, const void *W, const void *bias, const float *sx,
                     const float *sw, void *out, int out_dtype, int M, int N, int K,
                     const SkgPlan *plan, hipStream_t stream) {
    int rc = check_sizes(M, N, K, SKG_DTYPE_FP8);
    if (rc != SKG_OK) return rc;
    if (out_dtype != SKG_DTYPE_BF16 && out_dtype != SKG_DTYPE_F32) return SKG_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return SKG_OK;
    const int out_f32 = out_dtype == SKG_DTYPE_F32;
    skinny_fp8_scales sc{SKG_FP8_PER_TENSOR, sx, sw, nullptr, nullptr};
    rc = check_fp8(x, W, bias, &sc, out, out_f32, 2, M, N, K);
    if (rc != SKG_OK) return rc;
    SkgPlan p;
    if (plan) {
        p = *plan;
        rc = complete_plan(M, N, K, SKG_DTYPE_FP8, &p);
    } else {
        rc = skinny_gemm_plan(M, N, K, SKG_DTYPE_FP8, &p);
        // Where the FP8 table picks the dot kernel, the fused form reads x
        // as bf16 (twice the bytes of its codes) in every workgroup, so it
        // takes four (else two) columns per workgroup of 256 threads to cut
        // those L2 reads; failing both, the table's plan, else 512 threads
        // (the fused kernel holds bf16 x until it is quantised and may need
        // smaller workgroups).  At K = N = 4096 four columns took M = 1
        // from 6.9 to 5.5 us and M = 4 from 17.0 to 10.4 us.
        if (rc == SKG_OK && p.kind == SKG_KIND_DOT) {
            const int tries[4][2] = {{256, 4}, {256, 2}, {p.threads, p.cols}, {512, p.cols}};
            for (const auto &t : tries) {
                SkgPlan q = p;
                q.threads = t[0];
                q.cols = t[1];
                if (complete_plan(M, N, K, SKG_DTYPE_FP8, &q) == SKG_OK &&
                    fp8_dot_quant_ok(M, q.cols, q.depth, q.threads)) {
                    p = q;
                    break;
                }
            }
        }
    }
    if (rc != SKG_OK) return rc;
    // A caller's split-K plan quantises on load as asked.  The automatic
    // plan does not: every workgroup then reads x as bf16 and quantises it
    // again, and two launches measured faster at K = N = 4096 (8.75 against
    // 9.45 us at M = 8, 10.07 against 10.26 at M = 16).
    return run_fp8(x, W, bias, &sc, out, out_f32, true, plan != nullptr, M, N, K, p, stream);
}

// skinny_gemm_bf16_f32 and its planned form.
int bf16_f32_common(const void *x, const void *W, const void *bias, float *out, int M, int N,
                    int K, const SkgPlan *plan, hipStream_t stream) {
    int rc = check_sizes(M, N, K, SKG_DTYPE_BF16);
    if (rc != SKG_OK) return rc;
    if (M == 0 || N == 0) return SKG_OK;
    rc = check_pointers_bf16(x, W, bias, out, M, N, K, 1);
    if (rc != SKG_OK) return rc;
    SkgPlan p;
    if (plan) {
        p = *plan;
        rc = complete_plan(M, N, K, SKG_DTYPE_BF16, &p);
    } else {
        rc = skinny_gemm_plan(M, N, K, SKG_DTYPE_BF16, &p);
    }
    if (rc != SKG_OK) return rc;
    return run_bf16(x, W, bias, out, 1, M, N, K, p, stream);
}

}  // namespace

size_t round_floats(size_t floats) { return (floats + 63) / 64 * 64; }

size_t quant_floats(int M, int K) { return ((size_t)M * K + 3) / 4; }

size_t workspace_floats(const SkgPlan &p, int M, int N) {
    return p.splits > 1 ? (size_t)p.splits * M * N : 0;
}

int tile_count(const SkgPlan &p, int N) {
    return (p.kind == SKG_KIND_SPLITK || p.kind == SKG_KIND_TILED)
               ? (N + 16 * p.cols - 1) / (16 * p.cols)
               : 0;
}

}  // namespace skg

using namespace skg;

extern "C" int skinny_gemm_bf16(const void *x, const void *W, const void *bias,
                                const void *scales, void *out, int M, int N, int K,
                                hipStream_t stream) {
    int rc = check_sizes(M, N, K, SKG_DTYPE_BF16);
    if (rc != SKG_OK) return rc;
    if (M == 0 || N == 0) return SKG_OK;
    if (scales) return SKG_ERR_INVALID_ARG;
    rc = check_pointers_bf16(x, W, bias, out, M, N, K);
    if (rc != SKG_OK) return rc;
    SkgPlan p;
    rc = skinny_gemm_plan(M, N, K, SKG_DTYPE_BF16, &p);
    if (rc != SKG_OK) return rc;
    return run_bf16(x, W, bias, out, 0, M, N, K, p, stream);
}

extern "C" int skinny_gemm_bf16_planned(const void *x, const void *W, const void *bias, void *out,
                                        int M, int N, int K, const SkgPlan *plan,
                                        hipStream_t stream) {
    int rc = check_sizes(M, N, K, SKG_DTYPE_BF16);
    if (rc != SKG_OK) return rc;
    if (M == 0 || N == 0) return SKG_OK;
    if (!plan) return SKG_ERR_INVALID_ARG;
    rc = check_pointers_bf16(x, W, bias, out, M, N, K);
    if (rc != SKG_OK) return rc;
    SkgPlan p = *plan;
    rc = complete_plan(M, N, K, SKG_DTYPE_BF16, &p);
    if (rc != SKG_OK) return rc;
    return run_bf16(x, W, bias, out, 0, M, N, K, p, stream);
}

extern "C" int skinny_gemm_fp8(const void *x, const void *W, const void *bias,
                               const skinny_fp8_scales *scales, void *out, int M, int N, int K,
                               hipStream_t stream) {
    int rc = check_sizes(M, N, K, SKG_DTYPE_FP8);
    if (rc != SKG_OK) return rc;
    if (M == 0 || N == 0) return SKG_OK;
    rc = check_fp8(x, W, bias, scales, out, 0, 1, M, N, K);
    if (rc != SKG_OK) return rc;
    SkgPlan p;
    rc = skinny_gemm_plan(M, N, K, scales->mode == SKG_FP8_MX32 ? SKG_DTYPE_FP8_MX : SKG_DTYPE_FP8,
                          &p);
    if (rc != SKG_OK) return rc;
    return run_fp8(x, W, bias, scales, out, 0, false, false, M, N, K, p, stream);
}

extern "C" int skinny_gemm_fp8_planned(const void *x, const void *W, const void *bias,
                                       const skinny_fp8_scales *scales, void *out, int M, int N,
                                       int K, const SkgPlan *plan, hipStream_t stream) {
    int rc = check_sizes(M, N, K, SKG_DTYPE_FP8);
    if (rc != SKG_OK) return rc;
    if (M == 0 || N == 0) return SKG_OK;
    if (!plan) return SKG_ERR_INVALID_ARG;
    rc = check_fp8(x, W, bias, scales, out, 0, 1, M, N, K);
    if (rc != SKG_OK) return rc;
    SkgPlan p = *plan;
    // validated for the scale mode it runs in (MX plans have their own limits)
    rc = complete_plan(M, N, K, scales->mode == SKG_FP8_MX32 ? SKG_DTYPE_FP8_MX : SKG_DTYPE_FP8, &p);
    if (rc != SKG_OK) return rc;
    return run_fp8(x, W, bias, scales, out, 0, false, false, M, N, K, p, stream);
}

extern "C" int skinny_gemm_bf16_f32(const void *x, const void *W, const void *bias, float *out,
                                    int M, int N, int K, hipStream_t stream) {
    return bf16_f32_common(x, W, bias, out, M, N, K, nullptr, stream);
}

extern "C" int skinny_gemm_bf16_f32_planned(const void *x, const void *W, const void *bias,
                                            float *out, int M, int N, int K, const SkgPlan *plan,
                                            hipStream_t stream) {
    if (!plan) return SKG_ERR_INVALID_ARG;
    return bf16_f32_common(x, W, bias, out, M, N, K, plan, stream);
}

extern "C" int skinny_gemm_fp8_quant(const void *x, const void *W, const void *bias,
                                     const float *sx, const float *sw, void *out, int out_dtype,
                                     int M, int N, int K, hipStream_t stream) {
    return fp8_quant_common(x, W, bias, sx, sw, out, out_dtype, M, N, K, nullptr, stream);
}

extern "C" int skinny_gemm_fp8_quant_planned(const void *x, const void *W, const void *bias,
                                             const float *sx, const float *sw, void *out,
                                             int out_dtype, int M, int N, int K,
                                             const SkgPlan *plan, hipStream_t stream) {
    if (!plan) return SKG_ERR_INVALID_ARG;
    return fp8_quant_common(x, W, bias, sx, sw, out, out_dtype, M, N, K, plan, stream);
}

extern "C" int skinny_quant_e4m3(const void *x, const float *s, void *q, long n,
                                 hipStream_t stream) {
    if (n < 0) return SKG_ERR_INVALID_ARG;
    if (n == 0) return SKG_OK;
    if (!x || !s || !q) return SKG_ERR_INVALID_ARG;
    if (n > kMaxBufferBytes) return SKG_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return SKG_ERR_ALIGNMENT;
    if (overlap(q, (size_t)n, x, (size_t)n * 2) || overlap(q, (size_t)n, s, 4))
        return SKG_ERR_INVALID_ARG;
    return launch_quant_e4m3(x, s, q, n, stream) == (int)hipSuccess ? SKG_OK : SKG_ERR_HIP;
}

extern "C" int skinny_gemm_reserve(int max_M, int max_N, int max_K, int max_S,
                                   hipStream_t stream) {
    if (max_M < 1 || max_N < 1 || max_K < 0 || max_S < 1 || max_M > SKG_MAX_M ||
        max_S > kMaxSplits || (long)SKG_MAX_M * max_K * 2 > kMaxBufferBytes)
        return SKG_ERR_INVALID_ARG;
    float *ws = nullptr;
    unsigned *tk = nullptr;
    // the largest request any call can make: split partials, rounded, then
    // x quantised into the workspace (skinny_gemm_fp8_quant's two-launch
    // plans); the most tiles any plan can have: 16-column blocks of max_N
    const size_t floats =
        round_floats((size_t)max_S * max_M * max_N) + quant_floats(max_M, max_K);
    return acquire(stream, floats, (size_t)(max_N + 15) / 16, &ws, &tk);
}

extern "C" int skinny_gemm_release_all(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ws.empty() && g_retired.empty()) return SKG_OK;  // nothing held: no HIP call
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return SKG_ERR_HIP;
    // only the devices this library holds memory on: wait for their work,
    // then free it there
    std::vector<int> devs;
    auto note = [&](int d) {
        for (int e : devs)
            if (e == d) return;
        devs.push_back(d);
    };
    for (const auto &w : g_ws) note(w.device);
    for (const auto &r : g_retired) note(r.device);
    int rc = SKG_OK;
    for (int d : devs)
        if (hipSetDevice(d) != hipSuccess || hipDeviceSynchronize() != hipSuccess) rc = SKG_ERR_HIP;
    for (const auto &w : g_ws) {
        if (hipSetDevice(w.device) != hipSuccess) rc = SKG_ERR_HIP;
        if (w.ws && hipFree(w.ws) != hipSuccess) rc = SKG_ERR_HIP;
        if (w.tickets && hipFree(w.tickets) != hipSuccess) rc = SKG_ERR_HIP;
    }
    for (const auto &r : g_retired)
        if (hipSetDevice(r.device) != hipSuccess || hipFree(r.p) != hipSuccess) rc = SKG_ERR_HIP;
    if (hipSetDevice(cur) != hipSuccess) rc = SKG_ERR_HIP;
    g_ws.clear();
    g_retired.clear();
    g_generation.fetch_add(1, std::memory_order_acq_rel);  // every per-thread copy is stale
    return rc;
}

// ---------------------------------------------------------------- no allocation
// skinny_gemm_bf16_noalloc keeps its split partials in this file-scope
// device array instead of an allocated workspace: each device that loads
// the library holds one copy, at its own address, until the process ends.
// Host code never passes `scratch` itself (on the host it is only a stand-in
// symbol); it passes the address hipGetSymbolAddress returns on the device,
// looked up once per device with that device current.
constexpr size_t kScratchFloats = size_t(1) << 21;  // 8 MiB of fp32 partials
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
std::atomic<float *> g_scratch[kMaxScratchDevices];

// The current device's copy of `scratch`, found once per device.
int scratch_on_current_device(float **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SKG_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return SKG_ERR_UNSUPPORTED;
    float *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_acquire);
        if (!p) {
            void *q = nullptr;
            if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q)
                return SKG_ERR_HIP;
            p = static_cast<float *>(q);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SKG_OK;
}

}  // namespace

extern "C" int skinny_gemm_bf16_noalloc(const void *x, const void *W, const void *bias,
                                        const void *scales, void *out, int M, int N, int K,
                                        hipStream_t stream) {
    int rc = check_sizes(M, N, K, SKG_DTYPE_BF16);
    if (rc != SKG_OK) return rc;
    if (M == 0 || N == 0) return SKG_OK;
    if (scales) return SKG_ERR_INVALID_ARG;
    rc = check_pointers_bf16(x, W, bias, out, M, N, K);
    if (rc != SKG_OK) return rc;
    SkgPlan p;
    rc = skinny_gemm_plan(M, N, K, SKG_DTYPE_BF16, &p);
    if (rc != SKG_OK) return rc;
    if (p.kind == SKG_KIND_DOT || p.splits == 1)
        return run_bf16(x, W, bias, out, 0, M, N, K, p, stream);
    // The last-arriver reduction needs tile counters that are zero at rest;
    // the second-kernel reduction sums the same partials in the same order
    // (identical bits) and needs nothing but this call's partials, which it
    // reads after the main kernel has written all of them.
    if (p.reduce == SKG_REDUCE_LAST) {
        p.reduce = SKG_REDUCE_KERNEL;
        rc = complete_plan(M, N, K, SKG_DTYPE_BF16, &p);
        if (rc != SKG_OK) return rc;
    }
    if (workspace_floats(p, M, N) > kScratchFloats) return SKG_ERR_WORKSPACE;
    float *ws = nullptr;
    rc = scratch_on_current_device(&ws);
    if (rc != SKG_OK) return rc;
    const int e = p.kind == SKG_KIND_TILED
                      ? launch_tiled(p, x, W, bias, out, 0, ws, nullptr, M, N, K, stream)
                      : launch_splitk(p, x, W, bias, out, 0, ws, nullptr, M, N, K, stream);
    return e == (int)hipSuccess ? SKG_OK : SKG_ERR_HIP;
}

extern "C" const char *skinny_gemm_status_string(int status) {
    switch (status) {
    case SKG_OK: return "SKG_OK";
    case SKG_ERR_INVALID_ARG: return "SKG_ERR_INVALID_ARG";
    case SKG_ERR_ALIGNMENT: return "SKG_ERR_ALIGNMENT";
    case SKG_ERR_UNSUPPORTED: return "SKG_ERR_UNSUPPORTED";
    case SKG_ERR_WORKSPACE: return "SKG_ERR_WORKSPACE";
    case SKG_ERR_HIP: return "SKG_ERR_HIP";
    default: return "SKG_ERR_UNKNOWN";
    }
}
