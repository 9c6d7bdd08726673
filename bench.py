"""Benchmark of the small-M bf16 GEMM on one MI355X.

Workload (one "step"): the router GEMM out[M,256] = x[M,7168] @ W[256,7168]^T
for M = 1, 2, ..., 16, one call each, back to back on one stream.  bf16 in
and out, fp32 accumulation, no bias.  Inputs are seeded synthetic data
(x ~ N(0,1), W ~ N(0,1/K), drawn by torch's device generator) resident in
HBM before timing starts.

Cold weights: every call reads a different W from a pool of distinct
(x, W, out) sets whose W bytes total >= 1 GiB (> 4x the 256 MB Infinity
Cache), so no call finds its W in any cache.  The calls of a step are
captured in HIP graphs (one per step of the pool's rotation) and replayed;
HIP events on the launch stream bracket the timed replays.

value = algorithmic bytes of the step / time of the step, in GB/s, with
bytes per call = N*K*2 + M*K*2 + M*N*2 (W, x, out).

Also reported: per-M microseconds per call (graphs of one M over the whole
pool), the empty-kernel and read-stream floors at the same shape and each
M's operand-intake floor (the dot plan's loads with no arithmetic), the
roofline line of the dominant kernel, and the CPU oracle's time on a
bounded sample of the same workload (its outputs also checked against the
GPU's).  Then every other configuration, each with its own cold pool and
read-stream floor: the small router GEMM (K = 2048, N = 256, M = 1), the
router sweep at N = 384, the router shapes (4096, 256), (6144, 256) and
(2880, 128) with and without bias, the dense decode linears with and
without bias, FP8 K = N = 4096 in both scale modes, and the fp32-output and
fused-quantisation variants; sampled outputs of every configuration are
checked against the oracle.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu]
"""
import argparse
import ctypes
import json
import statistics
import os
import sys
import time
import zlib

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of peak), bf16 M=1–16, K=7168, N=256"
PEAK_GBS = 8000.0
K_DIM, N_DIM, M_VALUES = 7168, 256, list(range(1, 17))
POOL_BYTES = 1 << 30


def call_bytes(M, N=N_DIM, K=K_DIM):
    return N * K * 2 + M * K * 2 + M * N * 2


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dot_bf16_router_k7168_n256_traffic.md")
KERNEL_SOURCES = ("kernels_dot.hip", "kernels_splitk.hip", "splitk_common.h", "device_common.h")
ROUTER_TABLE_KEY = "SKG_DTYPE_BF16, 7168, 256,"  # the table rows of the router workload


def router_sources_sha256():
    """SHA-256 of what the router workload runs: the kernel sources and the
    dispatch-table rows of (bf16, K = 7168, N = 256)."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "latency_skinny_gemm_amd", "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(csrc, "dispatch_table.inc")) as fh:
        # the plans only: the timing comments change with every re-emission
        h.update("".join(l.split("//")[0] for l in fh if ROUTER_TABLE_KEY in l).encode())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 --pmc
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain copy), or None when
    there is none or the kernel sources changed since it was taken."""
    if kernel != "dot" or not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if " = " in line:
            k, v = line.strip().split(" = ", 1)
            fields[k] = v
    if fields.get("kernel_sources_sha256") != router_sources_sha256():
        return None
    return float(fields["traffic_bytes_per_launch_dot"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 section")
    ap.add_argument("--no-decode", action="store_true", help="skip the dense decode shapes")
    ap.add_argument("--no-router-configs", action="store_true",
                    help="skip the router shapes other than the headline one")
    ap.add_argument("--no-f3", action="store_true",
                    help="skip the fp32-output and fused-quantisation section")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="for rocprofv3 --pmc: the MFMA configurations (FP8 K = N = 4096 at "
                         "M >= 64, bf16 K = 7168, N = 4096 at M >= 128), a few cold calls each, "
                         "and exit")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for rocprofv3 --pmc: the decode (K = 7168, N = 4096, M = 8 and 128) "
                         "and FP8 (K = N = 4096, M = 16 and 128, both scale modes) calls, a few "
                         "cold calls each, then a 64 MiB reference copy, and exit")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for rocprofv3 --pmc: launch each headline call a few times on cold "
                         "weights, then a 64 MiB reference copy, and exit")
    return ap.parse_args()


COPY_BYTES = 64 << 20  # the reference copy's size (read and written once)


def pmc_probe(skg, torch, floors, stream, sptr, W, X, OUT, n_slots):
    """Eager launches for hardware-counter passes: 8 cold calls per M (each
    on its own pool slot), then one copy of COPY_BYTES, so a counter's value
    per GEMM dispatch can be scaled by what it reads for a known copy."""
    slot = 0
    with torch.cuda.stream(stream):
        for M in M_VALUES:
            for _ in range(8):
                rc = skg.lib().skinny_gemm_bf16(X[slot].data_ptr(), W[slot].data_ptr(), None, None,
                                                OUT[slot].data_ptr(), M, N_DIM, K_DIM, sptr)
                if rc != 0:
                    raise skg.SkinnyGemmError(rc, "pmc probe")
                slot = (slot + 1) % n_slots
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=W.device)
        dst = torch.empty_like(src)
        rc = floors.skinny_floor_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                      ctypes.c_size_t(COPY_BYTES), sptr)
        if rc != 0:
            raise RuntimeError(f"skinny_floor_copy failed: {rc}")
    stream.synchronize()
    print(json.dumps({"pmc_probe": "done", "calls_per_M": 8, "copy_bytes": COPY_BYTES}), flush=True)
    return 0


MFMA_PROBE_CALLS = 4
PER_M_REPLAYS = 11  # timed graph replays per M: median, p10, p90


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: the first processor's model
    name with its family, model and stepping numbers, and the logical CPU
    count the OS reports."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if fields:
                    break  # end of the first processor's block
                continue
            k, v = (t.strip() for t in line.split(":", 1))
            if k in ("model name", "cpu family", "model", "stepping", "vendor_id"):
                fields.setdefault(k, v)
    except OSError:
        return None
    return {"model_name": fields.get("model name"), "vendor": fields.get("vendor_id"),
            "family": fields.get("cpu family"), "model": fields.get("model"),
            "stepping": fields.get("stepping"), "logical_cpus": os.cpu_count()}


TRAFFIC_PROBE_CALLS = 4


def traffic_probe(skg, torch, floors, stream, sptr):
    """Eager launches for HBM byte counters of the tiled and FP8 plans:
    TRAFFIC_PROBE_CALLS cold calls (each on its own W) of every
    configuration below in the printed order, then one copy of COPY_BYTES
    to scale the counters.  Every input is made before the first GEMM, so
    the library's dispatches are exactly the printed calls."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(78)
    n = TRAFFIC_PROBE_CALLS
    KB, NB, K8, N8 = DECODE_K, 4096, 4096, 4096
    WB = (torch.randn((n, NB, KB), generator=g, device=dev) * KB ** -0.5).to(torch.bfloat16)
    W8 = torch.empty((2 * n, N8, K8), dtype=torch.float8_e4m3fn, device=dev)
    for i in range(2 * n):
        W8[i].copy_(torch.randn((N8, K8), generator=g, device=dev).to(torch.float8_e4m3fn))
    XB = {M: torch.randn((M, KB), generator=g, device=dev).to(torch.bfloat16) for M in (8, 128)}
    X8 = {M: torch.randn((M, K8), generator=g, device=dev).to(torch.float8_e4m3fn) for M in (16, 128)}
    XE = {M: torch.randint(126, 129, (M, K8 // 32), generator=g, device=dev).to(torch.uint8)
          for M in (16, 128)}
    WE = torch.randint(126, 129, (N8, K8 // 32), generator=g, device=dev).to(torch.uint8)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    out = torch.empty((128, 4096), dtype=torch.bfloat16, device=dev)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    order = []
    with torch.cuda.stream(stream):
        for M in (8, 128):
            p = skg.plan(M, NB, KB)
            for i in range(n):
                rc = skg.lib().skinny_gemm_bf16(XB[M].data_ptr(), WB[i].data_ptr(), None, None,
                                                out.data_ptr(), M, NB, KB, sptr)
                if rc != 0:
                    raise skg.SkinnyGemmError(rc, f"traffic probe bf16 M={M}")
            order.append({"config": f"bf16_M{M}_N{NB}_K{KB}", "calls": n, **plan_brief(p),
                          "algorithmic_bytes": 2 * NB * KB + 2 * M * KB + 2 * M * NB})
        slot = 0
        for M in (16, 128):
            for mode in ("tensor", "mx"):
                sc = skg.Fp8Scales()
                if mode == "tensor":
                    sc.mode, sc.sx, sc.sw = skg.FP8_PER_TENSOR, one.data_ptr(), one.data_ptr()
                else:
                    sc.mode, sc.x_e8m0, sc.w_e8m0 = skg.FP8_MX32, XE[M].data_ptr(), WE.data_ptr()
                p = skg.plan(M, N8, K8, skg.DTYPE_FP8 if mode == "tensor" else skg.DTYPE_FP8_MX)
                for _ in range(n):
                    rc = skg.lib().skinny_gemm_fp8(X8[M].data_ptr(), W8[slot].data_ptr(), None,
                                                   ctypes.byref(sc), out.data_ptr(), M, N8, K8, sptr)
                    if rc != 0:
                        raise skg.SkinnyGemmError(rc, f"traffic probe fp8 M={M} {mode}")
                    slot = (slot + 1) % (2 * n)
                extra = 8 if mode == "tensor" else (M + N8) * K8 // 32
                order.append({"config": f"fp8_{mode}_M{M}_N{N8}_K{K8}", "calls": n, **plan_brief(p),
                              "algorithmic_bytes": N8 * K8 + M * K8 + 2 * M * N8 + extra})
        rc = floors.skinny_floor_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                      ctypes.c_size_t(COPY_BYTES), sptr)
        if rc != 0:
            raise RuntimeError(f"skinny_floor_copy failed: {rc}")
    stream.synchronize()
    print(json.dumps({"traffic_probe": order, "copy_bytes": COPY_BYTES}), flush=True)
    return 0


def mfma_probe(skg, torch, stream, sptr):
    """Eager launches for MFMA counter passes: MFMA_PROBE_CALLS cold calls
    (each on its own W) of every configuration below, in the printed order;
    all inputs are made before the first GEMM, so the library's dispatches
    are exactly the printed calls (two each for plans with a reduction
    kernel)."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    n = MFMA_PROBE_CALLS
    K8 = N8 = 4096
    W8 = torch.empty((2 * n, N8, K8), dtype=torch.float8_e4m3fn, device=dev)
    for i in range(2 * n):
        W8[i].copy_(torch.randn((N8, K8), generator=g, device=dev).to(torch.float8_e4m3fn))
    one = torch.ones(1, dtype=torch.float32, device=dev)
    WE = torch.randint(126, 129, (N8, K8 // 32), generator=g, device=dev).to(torch.uint8)
    KB, NB = DECODE_K, 4096
    WB = (torch.randn((n, NB, KB), generator=g, device=dev) * KB ** -0.5).to(torch.bfloat16)
    fp8_m, bf16_m = (64, 128, 256, 512), (128, 256, 512)
    X8 = {M: torch.randn((M, K8), generator=g, device=dev).to(torch.float8_e4m3fn) for M in fp8_m}
    XE = {M: torch.randint(126, 129, (M, K8 // 32), generator=g, device=dev).to(torch.uint8)
          for M in fp8_m}
    XB = {M: torch.randn((M, KB), generator=g, device=dev).to(torch.bfloat16) for M in bf16_m}
    out = torch.empty((512, 4096), dtype=torch.float32, device=dev)  # room for either dtype
    torch.cuda.synchronize()
    order = []
    with torch.cuda.stream(stream):
        slot = 0
        for M in fp8_m:
            for mode in ("tensor", "mx"):
                sc = skg.Fp8Scales()
                if mode == "tensor":
                    sc.mode, sc.sx, sc.sw = skg.FP8_PER_TENSOR, one.data_ptr(), one.data_ptr()
                else:
                    sc.mode, sc.x_e8m0, sc.w_e8m0 = skg.FP8_MX32, XE[M].data_ptr(), WE.data_ptr()
                p = skg.plan(M, N8, K8, skg.DTYPE_FP8 if mode == "tensor" else skg.DTYPE_FP8_MX)
                for _ in range(n):
                    rc = skg.lib().skinny_gemm_fp8(X8[M].data_ptr(), W8[slot].data_ptr(), None,
                                                   ctypes.byref(sc), out.data_ptr(), M, N8, K8, sptr)
                    if rc != 0:
                        raise skg.SkinnyGemmError(rc, f"mfma probe fp8 M={M}")
                    slot = (slot + 1) % (2 * n)
                order.append({"config": f"fp8_{mode}_M{M}_N{N8}_K{K8}", "calls": n,
                              "dispatches_per_call": 2 if p.reduce == skg.REDUCE_KERNEL else 1,
                              "flops_per_call": 2 * M * N8 * K8})
        for M in bf16_m:
            p = skg.plan(M, NB, KB)
            for i in range(n):
                rc = skg.lib().skinny_gemm_bf16(XB[M].data_ptr(), WB[i].data_ptr(), None, None,
                                                out.data_ptr(), M, NB, KB, sptr)
                if rc != 0:
                    raise skg.SkinnyGemmError(rc, f"mfma probe bf16 M={M}")
            order.append({"config": f"bf16_M{M}_N{NB}_K{KB}", "calls": n,
                          "dispatches_per_call": 2 if p.reduce == skg.REDUCE_KERNEL else 1,
                          "flops_per_call": 2 * M * NB * KB})
    stream.synchronize()
    print(json.dumps({"mfma_probe": order}), flush=True)
    return 0


SECTION_REPLAYS = 11  # timed graph replays per configuration of a section


def graph_times(torch, stream, calls, n_calls, reps=SECTION_REPLAYS, passes=2):
    """Runs calls() once eagerly (growing any workspace outside capture),
    captures it in a graph and replays it, `passes` times over: returns the
    median, p10 and p90 microseconds per call over the last pass's `reps`
    timed replays (each pass starts with one untimed replay).  The first
    pass after a section allocates new inputs ran slower throughout, by up
    to 1 us a call (FP8 M = 16: 8.47 against 7.42 us on the next pass), so
    it is a warm-up."""
    for _ in range(passes):
        with torch.cuda.stream(stream):
            calls()
        stream.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            calls()
        ts = []
        with torch.cuda.stream(stream):
            gr.replay()
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                gr.replay()
                e1.record(stream)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / n_calls)
        del gr
    ts.sort()
    return ts[len(ts) // 2], ts[len(ts) // 10], ts[(9 * len(ts)) // 10]


def sample_outputs(M, N):
    """Rows and columns of an output sampled for the oracle check: the first
    and last row and 32 columns spread over N (the last one included)."""
    rows = sorted({0, M - 1})
    cols = sorted({(i * (N - 1)) // 31 for i in range(32)})
    return rows, cols


DECODE_K = 7168
DECODE_N = (576, 2112, 4096)
DECODE_M = (1, 8, 32, 64, 128)
LARGE_M = (256, 512)  # the larger-M regime, at N = 4096 only
SECTION_POOL = 512 << 20  # W bytes of a section's cold pool (> the 256 MB Infinity Cache)
KIND_NAMES = {1: "dot", 2: "splitk", 3: "tiled", 4: "rows"}

# The bf16 configurations other than the headline shape, by (K, N): the
# small router GEMM (K = 2048, N = 256, M = 1), the router sweep at N = 384
# (M = 1..16), the tuned router shapes (4096, 256), (6144, 256) and the
# non-tile-aligned (2880, 128) at M in {1, 3, 4, 5, 8, 9, 12, 16} with and
# without bias, and the dense decode linears (K = 7168, N in {576, 2112,
# 4096}, M in {1, 8, 32, 64, 128} with and without bias; M = 256 and 512 at
# N = 4096).
ROUTER_M = (1, 3, 4, 5, 8, 9, 12, 16)
BF16_SHAPES = (
    [("small_k2048_n256", 2048, 256, [(1, False)]),
     ("router_k7168_n384", 7168, 384, [(M, False) for M in range(1, 17)])]
    + [(f"router_k{K}_n{N}", K, N, [(M, b) for M in ROUTER_M for b in (False, True)])
       for (K, N) in ((4096, 256), (6144, 256), (2880, 128))]
    + [(f"decode_k{DECODE_K}_n{N}", DECODE_K, N,
        [(M, b) for M in DECODE_M for b in (False, True)]
        + ([(M, False) for M in LARGE_M] if N == 4096 else []))
       for N in DECODE_N])


def plan_brief(p):
    return {"kernel": KIND_NAMES[p.kind], "threads": p.threads, "cols": p.cols,
            "splits": p.splits, "depth": p.depth,
            "reduce": {0: "none", 1: "last", 2: "kernel"}[p.reduce]}


def read_floor_us(torch, floors, stream, sptr, W, row_bytes, sink):
    """The read-stream floor at one shape: a plain read of each pool slot's
    W, timed like the GEMM (the same graph replay over the same cold pool),
    two ways: one workgroup of 256 threads per row, and the same bytes read
    flat in 32 KB per workgroup; every load in flight at once in both.
    Returns (the faster, per-row, flat) microseconds per call."""
    slots, rows = W.shape[0], W.shape[1]
    nbytes = rows * row_bytes

    def per_row():
        for s in range(slots):
            rc = floors.skinny_floor_read(ctypes.c_void_p(W[s].data_ptr()), rows, row_bytes, 256,
                                          ctypes.c_void_p(sink.data_ptr()), sptr)
            if rc != 0:
                raise RuntimeError(f"skinny_floor_read failed: {rc}")

    def flat():
        for s in range(slots):
            rc = floors.skinny_floor_read_flat(ctypes.c_void_p(W[s].data_ptr()),
                                               ctypes.c_size_t(nbytes),
                                               ctypes.c_void_p(sink.data_ptr()), sptr)
            if rc != 0:
                raise RuntimeError(f"skinny_floor_read_flat failed: {rc}")
    t_rows = graph_times(torch, stream, per_row, slots)[0]
    t_flat = graph_times(torch, stream, flat, slots)[0]
    return min(t_rows, t_flat), t_rows, t_flat


def intake_floor_us(torch, floors, stream, sptr, X, W, M, N, K, p, sink):
    """The operand-intake floor of a dot-kernel plan: its W and x loads,
    exactly as the plan issues them, with no arithmetic (skinny_floor_intake),
    over the same cold pool; None when that plan's intake kernel is not
    built."""
    slots = W.shape[0]

    def calls():
        for s in range(slots):
            rc = floors.skinny_floor_intake(ctypes.c_void_p(X[s].data_ptr()),
                                            ctypes.c_void_p(W[s].data_ptr()), M, N, K, p.cols,
                                            p.threads, p.depth, ctypes.c_void_p(sink.data_ptr()),
                                            sptr)
            if rc != 0:
                raise RuntimeError(f"skinny_floor_intake failed: {rc}")
    try:
        return graph_times(torch, stream, calls, slots)[0]
    except RuntimeError:
        return None


def bf16_shape_section(skg, torch, floors, stream, sptr, samples, K, N, points, seed):
    """One bf16 shape (K, N) at the given (M, bias) points, each on the
    planner's plan: microseconds per call (median, p10, p90 of graph
    replays over a cold pool of >= 512 MB of distinct W, each slot with its
    own x and bias), the algorithmic GB/s and its fraction of 8 TB/s, and
    the fraction of the shape's read-stream floor; dot-kernel points also
    give their operand-intake floor.  Bias ~ N(0, 0.1) bf16 (variance 0.1)."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    slots = max(4, -(-SECTION_POOL // (N * K * 2)))
    Mmax = max(M for M, _ in points)
    W = torch.empty((slots, N, K), dtype=torch.bfloat16, device=dev)
    for i in range(slots):
        W[i].copy_((torch.randn((N, K), generator=g, device=dev) * K ** -0.5).to(torch.bfloat16))
    X = torch.randn((slots, Mmax, K), generator=g, device=dev).to(torch.bfloat16)
    B = (torch.randn((slots, N), generator=g, device=dev) * 0.1 ** 0.5).to(torch.bfloat16)
    O = torch.empty((slots, Mmax, N), dtype=torch.bfloat16, device=dev)
    sink = torch.zeros(max(N, 4096), dtype=torch.int32, device=dev)
    t_read, t_rows, t_flat = read_floor_us(torch, floors, stream, sptr, W, 2 * K, sink)
    res = {"read_stream_floor_us": round(t_read, 3), "read_per_row_us": round(t_rows, 3),
           "read_flat_us": round(t_flat, 3), "W_bytes": 2 * N * K, "pool_slots": slots}
    L = skg.lib()
    for M, bias in points:
        def calls(M=M, bias=bias):
            for s in range(slots):
                rc = L.skinny_gemm_bf16(X[s].data_ptr(), W[s].data_ptr(),
                                        B[s].data_ptr() if bias else None, None, O[s].data_ptr(),
                                        M, N, K, sptr)
                if rc != 0:
                    raise skg.SkinnyGemmError(rc, f"skinny_gemm_bf16 M={M} N={N} K={K}")
        us, p10, p90 = graph_times(torch, stream, calls, slots)
        torch.cuda.synchronize()
        key = f"M{M}" + ("_bias" if bias else "")
        rows, cols = sample_outputs(M, N)
        samples.append({"key": f"bf16_K{K}_N{N}_{key}", "kind": "bf16", "K": K,
                        "x": X[0][:M][rows].cpu(), "w": W[0][cols].cpu(),
                        "b": B[0][cols].cpu() if bias else None,
                        "out": O[0][:M][rows][:, cols].cpu()})
        byts = 2 * N * K + 2 * M * K + 2 * M * N + (2 * N if bias else 0)
        p = skg.plan(M, N, K)
        e = {"us_per_call": round(us, 3), "p10_us": round(p10, 3), "p90_us": round(p90, 3),
             "GBps": round(byts / (us * 1e-6) / 1e9, 1),
             "frac_of_8TBps": round(byts / (us * 1e-6) / (PEAK_GBS * 1e9), 4),
             "of_read_floor": round(t_read / us, 3),
             "TFLOPs": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 1), **plan_brief(p)}
        if p.kind == skg.KIND_DOT:
            t_in = intake_floor_us(torch, floors, stream, sptr, X, W, M, N, K, p, sink)
            if t_in is not None:
                e["intake_floor_us"] = round(t_in, 3)
                e["of_intake_floor"] = round(t_in / us, 3)
        res[key] = e
    del W, X, B, O
    torch.cuda.empty_cache()
    return res


def f3_section(skg, torch, stream, sptr):
    """The two output/quantisation variants, microseconds per call on cold W:
    fp32 logits beside bf16 at the router shape (K = 7168, N = 256), and the
    FP8 GEMM on bf16 activations at K = N = 4096 with the quantisation fused
    into the dot kernel beside quantise-then-GEMM (two launches)."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    res = {}

    def timed(calls, n):
        return round(graph_times(torch, stream, calls, n)[0], 3)

    L = skg.lib()
    K, N = 7168, 256
    slots = -(-(512 << 20) // (N * K * 2))
    W = (torch.randn((slots, N, K), generator=g, device=dev) * K ** -0.5).to(torch.bfloat16)
    for M in (1, 8, 16):
        X = torch.randn((slots, M, K), generator=g, device=dev).to(torch.bfloat16)
        O16 = torch.empty((slots, M, N), dtype=torch.bfloat16, device=dev)
        O32 = torch.empty((slots, M, N), dtype=torch.float32, device=dev)

        def c16():
            for s in range(slots):
                assert L.skinny_gemm_bf16(X[s].data_ptr(), W[s].data_ptr(), None, None,
                                          O16[s].data_ptr(), M, N, K, sptr) == 0

        def c32():
            for s in range(slots):
                assert L.skinny_gemm_bf16_f32(X[s].data_ptr(), W[s].data_ptr(), None,
                                              O32[s].data_ptr(), M, N, K, sptr) == 0
        res[f"router_M{M}"] = {"bf16_out_us": timed(c16, slots), "fp32_out_us": timed(c32, slots)}
    del W
    K = N = 4096
    slots = -(-(512 << 20) // (N * K))
    Wq = torch.empty((slots, N, K), dtype=torch.float8_e4m3fn, device=dev)
    for i in range(slots):
        Wq[i].copy_(torch.randn((N, K), generator=g, device=dev).to(torch.float8_e4m3fn))
    one = torch.ones(1, dtype=torch.float32, device=dev)
    sx = torch.full((1,), 0.01, dtype=torch.float32, device=dev)
    for M in (1, 8, 16):
        X = torch.randn((slots, M, K), generator=g, device=dev).to(torch.bfloat16)
        XQ = torch.empty((slots, M, K), dtype=torch.float8_e4m3fn, device=dev)
        O = torch.empty((slots, M, N), dtype=torch.bfloat16, device=dev)
        sc = skg.Fp8Scales()
        sc.mode, sc.sx, sc.sw = skg.FP8_PER_TENSOR, sx.data_ptr(), one.data_ptr()

        def quant_call():  # one launch where the dot kernel fuses it, else two
            for s in range(slots):
                assert L.skinny_gemm_fp8_quant(X[s].data_ptr(), Wq[s].data_ptr(), None,
                                               sx.data_ptr(), one.data_ptr(), O[s].data_ptr(),
                                               skg.DTYPE_BF16, M, N, K, sptr) == 0

        def two_step():
            for s in range(slots):
                assert L.skinny_quant_e4m3(X[s].data_ptr(), sx.data_ptr(), XQ[s].data_ptr(),
                                           M * K, sptr) == 0
                assert L.skinny_gemm_fp8(XQ[s].data_ptr(), Wq[s].data_ptr(), None,
                                         ctypes.byref(sc), O[s].data_ptr(), M, N, K, sptr) == 0
        res[f"fp8_quant_M{M}"] = {"fp8_quant_call_us": timed(quant_call, slots),
                                  "quant_then_gemm_us": timed(two_step, slots)}
    del Wq
    torch.cuda.empty_cache()
    return res


FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA


def fp8_section(skg, torch, floors, stream, sptr, samples):
    """FP8 e4m3, K = N = 4096, M in {1, 16, 64, 128, 256, 512}, per-tensor and MX
    scales: microseconds per call over a cold pool of >= 512 MB of distinct
    W, the achieved GB/s (W, x, out and scale bytes), its fraction of the
    read-stream floor of the same 16.8 MB, and the MFMA rate against the
    dense fp8 peak."""
    K = N = 4096
    dev = torch.device("cuda:0")
    slots = -(-(512 << 20) // (N * K))
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    W = torch.empty((slots, N, K), dtype=torch.float8_e4m3fn, device=dev)
    for i in range(slots):
        W[i].copy_(torch.randn((N, K), generator=g, device=dev).to(torch.float8_e4m3fn))
    sink = torch.zeros(N, dtype=torch.int32, device=dev)
    t_read, t_rows, t_flat = read_floor_us(torch, floors, stream, sptr, W, K, sink)
    res = {"read_stream_floor_us": round(t_read, 3), "read_per_row_us": round(t_rows, 3),
           "read_flat_us": round(t_flat, 3), "W_bytes": N * K, "pool_slots": slots}
    for M in (1, 16, 64, 128, 256, 512):
        X = torch.randn((slots, M, K), generator=g, device=dev).to(torch.float8_e4m3fn)
        O = torch.empty((slots, M, N), dtype=torch.bfloat16, device=dev)
        one = torch.ones(1, dtype=torch.float32, device=dev)
        # exponents 126..128, distinct per slot like W itself
        XE = torch.randint(126, 129, (slots, M, K // 32), generator=g, device=dev).to(torch.uint8)
        WE = torch.randint(126, 129, (slots, N, K // 32), generator=g, device=dev).to(torch.uint8)
        for mode in ("tensor", "mx"):
            scs = []
            for s in range(slots):
                sc = skg.Fp8Scales()
                if mode == "tensor":
                    sc.mode, sc.sx, sc.sw = skg.FP8_PER_TENSOR, one.data_ptr(), one.data_ptr()
                else:
                    sc.mode, sc.x_e8m0, sc.w_e8m0 = skg.FP8_MX32, XE[s].data_ptr(), WE[s].data_ptr()
                scs.append(sc)
            extra = 8 if mode == "tensor" else (M + N) * K // 32

            def calls():
                for s in range(slots):
                    rc = skg.lib().skinny_gemm_fp8(X[s].data_ptr(), W[s].data_ptr(), None,
                                                   ctypes.byref(scs[s]), O[s].data_ptr(), M, N, K, sptr)
                    if rc != 0:
                        raise skg.SkinnyGemmError(rc, f"skinny_gemm_fp8 M={M} {mode}")
            us, p10, p90 = graph_times(torch, stream, calls, slots)
            torch.cuda.synchronize()
            rows, cols = sample_outputs(M, N)
            samp = {"key": f"fp8_{mode}_M{M}", "kind": f"fp8_{mode}", "K": K,
                    "x": X[0][rows].cpu(), "w": W[0][cols].cpu(), "out": O[0][rows][:, cols].cpu()}
            if mode == "mx":
                samp["xe"], samp["we"] = XE[0][rows].cpu(), WE[0][cols].cpu()
            samples.append(samp)
            byts = N * K + M * K + M * N * 2 + extra
            tflops = 2.0 * M * N * K / (us * 1e-6) / 1e12
            res[f"M{M}_{mode}"] = {"us_per_call": round(us, 3), "p10_us": round(p10, 3),
                                   "p90_us": round(p90, 3),
                                   "GBps": round(byts / (us * 1e-6) / 1e9, 1),
                                   "frac_of_8TBps": round(byts / (us * 1e-6) / (PEAK_GBS * 1e9), 4),
                                   "of_read_floor": round(t_read / us, 3),
                                   "TFLOPs": round(tflops, 1),
                                   "mfma_util": round(tflops / FP8_PEAK_TFLOPS, 4),
                                   **plan_brief(skg.plan(M, N, K, skg.DTYPE_FP8 if mode == "tensor"
                                                         else skg.DTYPE_FP8_MX))}
        del X, O, XE, WE
    del W
    torch.cuda.empty_cache()
    return res


def check_samples(samples):
    """The sampled outputs of the timed sections against the oracle: "ok"
    when all are within the tolerance, else the first failure."""
    import torch

    import oracle
    from oracle import tolerance

    def bits16(t):
        return t.contiguous().view(torch.int16).numpy().view("uint16")

    def bits8(t):
        return t.contiguous().view(torch.uint8).numpy()

    for s in samples:
        if s["kind"] == "bf16":
            b = s.get("b")
            ref = oracle.gemm_bf16(bits16(s["x"]), bits16(s["w"]), None if b is None else bits16(b),
                                   threads=16)
        elif s["kind"] == "fp8_tensor":
            ref = oracle.gemm_fp8_tensor(bits8(s["x"]), bits8(s["w"]), 1.0, 1.0, threads=16)
        else:
            ref = oracle.gemm_fp8_mx(bits8(s["x"]), bits8(s["w"]), bits8(s["xe"]), bits8(s["we"]),
                                     threads=16)
        ok, msg = tolerance.check(s["out"], ref, s["K"])
        if not ok:
            return f"{s['key']}: {msg}"
    return f"ok ({len(samples)} configurations, 2 rows x 32 columns each)"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(each GPU runs the GEMM on its own shard of W with no collective, so one GPU's "
              "throughput is the figure)",
              file=sys.stderr)
        return 2
    import torch

    import latency_skinny_gemm_amd as skg

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.mfma_probe:
        st = torch.cuda.Stream()
        return mfma_probe(skg, torch, st, ctypes.c_void_p(st.cuda_stream))
    floors = ctypes.CDLL(os.path.join(ROOT, "latency_skinny_gemm_amd", "libskinny_floors.so"))
    floors.skinny_floor_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    floors.skinny_floor_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    floors.skinny_floor_intake.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 6 + \
        [ctypes.c_void_p, ctypes.c_void_p]
    floors.skinny_floor_read_flat.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                              ctypes.c_void_p]
    floors.skinny_floor_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]
    stream = torch.cuda.Stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    if args.traffic_probe:
        return traffic_probe(skg, torch, floors, stream, sptr)

    # ---------------------------------------------------------------- pool
    w_bytes = N_DIM * K_DIM * 2
    calls = len(M_VALUES)
    n_slots = -(-POOL_BYTES // w_bytes)
    n_slots = -(-n_slots // calls) * calls  # whole steps
    g = torch.Generator(device=dev)
    g.manual_seed(20261202)
    Ms = max(M_VALUES)
    W = torch.empty((n_slots, N_DIM, K_DIM), dtype=torch.bfloat16, device=dev)
    X = torch.empty((n_slots, Ms, K_DIM), dtype=torch.bfloat16, device=dev)
    OUT = torch.zeros((n_slots, Ms, N_DIM), dtype=torch.bfloat16, device=dev)
    for i in range(n_slots):
        W[i].copy_(torch.randn((N_DIM, K_DIM), generator=g, device=dev) * (K_DIM ** -0.5))
        X[i].copy_(torch.randn((Ms, K_DIM), generator=g, device=dev))
    torch.cuda.synchronize()

    if args.pmc_probe:
        return pmc_probe(skg, torch, floors, stream, sptr, W, X, OUT, n_slots)

    plans = {M: skg.plan(M, N_DIM, K_DIM) for M in M_VALUES}

    def launch(slot, M):
        rc = skg.lib().skinny_gemm_bf16(X[slot].data_ptr(), W[slot].data_ptr(), None, None,
                                        OUT[slot].data_ptr(), M, N_DIM, K_DIM, sptr)
        if rc != 0:
            raise skg.SkinnyGemmError(rc, f"skinny_gemm_bf16 M={M}")

    def capture(fn):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            fn()
        return gr

    with torch.cuda.stream(stream):
        skg.reserve(Ms, N_DIM, K_DIM, 256)
        # eager warm-up of every plan (and a first correctness sample below)
        for M in M_VALUES:
            launch(0, M)
    stream.synchronize()

    # ---------------------------------------------------------------- headline
    # One graph holds a whole cycle of the pool (every W once, n_cycle steps)
    # so that graph submission is amortised over 304 calls, as in the per-M
    # graphs below; one-step graphs make up a remainder, so exactly K steps
    # run in the timed region, each step on the next W sets of the rotation.
    n_cycle = n_slots // calls
    step_graphs = [capture(lambda gi=gi: [launch(gi * calls + j, M) for j, M in enumerate(M_VALUES)])
                   for gi in range(n_cycle)]
    cycle_graph = capture(lambda: [launch(gi * calls + j, M) for gi in range(n_cycle)
                                   for j, M in enumerate(M_VALUES)])

    def run_steps(k):
        full, rem = divmod(k, n_cycle)
        for _ in range(full):
            cycle_graph.replay()
        for gi in range(rem):
            step_graphs[gi].replay()

    with torch.cuda.stream(stream):
        # every graph the timed region replays has been replayed once before
        # it, whatever --warmup is: a graph's first replay uploads it and runs
        # slower (0.3 us a call on the 304-call cycle graph)
        full, rem = divmod(args.steps, n_cycle)
        if full:
            cycle_graph.replay()
        for gi in range(rem):
            step_graphs[gi].replay()
        run_steps(args.warmup)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        run_steps(args.steps)
        e1.record(stream)
    torch.cuda.synchronize()
    t_steps = e0.elapsed_time(e1) / 1e3  # seconds
    del cycle_graph, step_graphs
    ms_per_step = t_steps / args.steps * 1e3
    step_bytes = sum(call_bytes(M) for M in M_VALUES)
    value = step_bytes / (t_steps / args.steps) / 1e9

    # ---------------------------------------------------------------- per M
    def replay_times(gr, reps):
        """Seconds of each of `reps` timed replays (one warm-up replay first)."""
        out = []
        with torch.cuda.stream(stream):
            gr.replay()
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                gr.replay()
                e1.record(stream)
                e1.synchronize()
                out.append(e0.elapsed_time(e1) / 1e3)
        return sorted(out)

    per_m = {}
    for M in M_VALUES:
        gr = capture(lambda M=M: [launch(s, M) for s in range(n_slots)])
        ts = [t / n_slots * 1e6 for t in replay_times(gr, PER_M_REPLAYS)]
        us = statistics.median(ts)
        per_m[M] = {"us_per_call": round(us, 3), "p10_us": round(ts[len(ts) // 10], 3),
                    "p90_us": round(ts[(9 * len(ts)) // 10], 3),
                    "GBps": round(call_bytes(M) / (us * 1e-6) / 1e9, 1),
                    "frac_of_8TBps": round(call_bytes(M) / (us * 1e-6) / (PEAK_GBS * 1e9), 4),
                    **plan_brief(plans[M])}
        del gr

    # ---------------------------------------------------------------- floors
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)

    def floor_empty():
        for _ in range(n_slots):
            floors.skinny_floor_empty(256, 256, sptr)

    def floor_read():
        for s in range(n_slots):
            floors.skinny_floor_read(ctypes.c_void_p(W[s].data_ptr()), N_DIM, K_DIM * 2, 256,
                                     ctypes.c_void_p(sink.data_ptr()), sptr)

    def floor_read_flat():
        for s in range(n_slots):
            floors.skinny_floor_read_flat(ctypes.c_void_p(W[s].data_ptr()), ctypes.c_size_t(w_bytes),
                                          ctypes.c_void_p(sink.data_ptr()), sptr)

    t_empty = statistics.median(replay_times(capture(floor_empty), PER_M_REPLAYS)) / n_slots * 1e6
    t_read_rows = statistics.median(replay_times(capture(floor_read), PER_M_REPLAYS)) / n_slots * 1e6
    t_read_flat = statistics.median(replay_times(capture(floor_read_flat), PER_M_REPLAYS)) / n_slots * 1e6
    t_read = min(t_read_rows, t_read_flat)
    for M in M_VALUES:  # context: the same bytes read by a plain stream at this size
        per_m[M]["of_read_floor"] = round(t_read / per_m[M]["us_per_call"], 3)
    # the operand-intake floor of each M's dot plan: its loads alone
    for M in M_VALUES:
        if plans[M].kind != skg.KIND_DOT:
            continue
        t_in = intake_floor_us(torch, floors, stream, sptr, X, W, M, N_DIM, K_DIM, plans[M], sink)
        if t_in is not None:
            per_m[M]["intake_floor_us"] = round(t_in, 3)
            per_m[M]["of_intake_floor"] = round(t_in / per_m[M]["us_per_call"], 3)

    # ---------------------------------------------------------------- determinism
    # every plan twice on the same inputs: the outputs must agree bit for bit
    det = torch.empty((2, Ms, N_DIM), dtype=torch.bfloat16, device=dev)
    deterministic = True
    for M in M_VALUES:
        for r in range(2):
            with torch.cuda.stream(stream):
                launch(1, M)
                det[r, :M].copy_(OUT[1, :M])
            stream.synchronize()
        deterministic &= bool(torch.equal(det[0, :M].view(torch.int16), det[1, :M].view(torch.int16)))

    # ---------------------------------------------------------------- roofline
    by_kind = {}
    for M in M_VALUES:
        k = per_m[M]["kernel"]
        b, t, n = by_kind.get(k, (0, 0.0, 0))
        by_kind[k] = (b + call_bytes(M), t + per_m[M]["us_per_call"], n + 1)
    dom = max(by_kind, key=lambda k: by_kind[k][1])
    b, t, n = by_kind[dom]
    achieved = b / (t * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4), "traffic": measured_traffic(dom),
                "kernel": dom, "launches_per_step": n,
                "avg_launch_us": round(t / n, 3),
                "algorithmic_bytes_per_launch": round(b / n)}

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle
        from oracle import tolerance

        # every CPU this process may run on, unless the host's OpenMP setting
        # (the CPU share given to one GPU's jobs) is lower
        affinity = len(os.sched_getaffinity(0))
        share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
        threads = min(affinity, share) if share > 0 else affinity
        x0 = X[0].cpu()
        w0 = W[0].cpu()
        with torch.cuda.stream(stream):
            for M in M_VALUES:
                launch(0, M)  # leaves out[0] = the M = 16 result for slot 0
        stream.synchronize()
        xb = x0.view(torch.int16).numpy().view("uint16")
        wb = w0.view(torch.int16).numpy().view("uint16")
        worst = "ok"
        reps, t_cpu, done_bytes = 0, 0.0, 0
        while t_cpu < args.cpu_seconds or reps == 0:
            for M in M_VALUES:
                t0 = time.perf_counter()
                ref = oracle.gemm_bf16(xb[:M], wb, threads=threads)
                t_cpu += time.perf_counter() - t0
                done_bytes += call_bytes(M)
                if reps == 0:
                    with torch.cuda.stream(stream):
                        launch(0, M)
                    stream.synchronize()
                    ok, msg = tolerance.check(OUT[0, :M].cpu(), ref, K_DIM)
                    if not ok:
                        worst = f"M={M}: {msg}"
            reps += 1
        parity = worst
        # one host thread: the median of 3 passes over M = 1..16
        one = []
        for _ in range(3):
            t0 = time.perf_counter()
            for M in M_VALUES:
                oracle.gemm_bf16(xb[:M], wb, threads=1)
            one.append(time.perf_counter() - t0)
        step = sum(call_bytes(M) for M in M_VALUES)
        cpu = {"value": round(done_bytes / t_cpu / 1e9, 4), "unit": "GB/s",
               "cores": oracle.threads_used(threads), "kind": "oracle",
               "sample": f"{reps} pass(es) over M=1..16 at K=7168, N=256 (pool slot 0); "
                         f"{t_cpu:.1f} s of oracle time; us/call: "
                         f"{t_cpu / reps / len(M_VALUES) * 1e6:.0f} (mean over M)",
               "single_thread_value": round(step / statistics.median(one) / 1e9, 4),
               "single_thread_sample": "median of 3 passes over M=1..16, one thread",
               "affinity_cpus": affinity, "omp_num_threads": share or None,
               "cpu": cpu_model()}

    samples = []  # sampled outputs of the other sections, checked below
    fp8 = None if args.no_fp8 else fp8_section(skg, torch, floors, stream, sptr, samples)
    configs = {}
    for name, K, N, points in BF16_SHAPES:
        if args.no_decode if name.startswith("decode") else args.no_router_configs:
            continue
        configs[name] = bf16_shape_section(skg, torch, floors, stream, sptr, samples, K, N, points,
                                           seed=zlib.crc32(name.encode()))
        # the launch floor does not depend on the shape (1 and 256 workgroups
        # measure the same): the headline's empty kernel, beside each shape
        configs[name]["empty_kernel_floor_us"] = round(t_empty, 3)
    f3 = None if args.no_f3 else f3_section(skg, torch, stream, sptr)
    # CPU-baseline leg, continued: the sections' sampled outputs against the oracle
    parity_sections = None
    if not args.no_cpu and samples:
        parity_sections = check_samples(samples)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 router GEMM out[M,256]=x[M,7168]@W[256,7168]^T, "
                               "M=1..16 one call each per step, cold W (pool >= 1 GiB)",
                   "K": K_DIM, "N": N_DIM, "M": "1-16", "calls_per_step": calls,
                   "pool_slots": n_slots, "pool_W_bytes": n_slots * w_bytes},
        "us_per_call_mean": round(ms_per_step * 1e3 / calls, 3),
        "frac_of_peak": round(value / PEAK_GBS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "floors": {"empty_kernel_us": round(t_empty, 3), "read_stream_us": round(t_read, 3),
                   "read_per_row_us": round(t_read_rows, 3), "read_flat_us": round(t_read_flat, 3),
                   "read_stream_GBps": round(w_bytes / (t_read * 1e-6) / 1e9, 1),
                   "shape": "empty: 256 workgroups x 256 threads; read: 256 rows x 14336 B, "
                            "or flat in 32 KB per workgroup (the faster is the floor)"},
        "per_m": per_m,
        "fp8_k4096_n4096": fp8,
        "bf16_configs": configs,
        "fp32_out_and_fused_quant": f3,
        "parity": parity,
        "parity_sections": parity_sections,
        "deterministic": deterministic,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
