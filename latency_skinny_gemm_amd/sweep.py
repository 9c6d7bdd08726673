"""Offline sweep of launch plans on MI355X -> the dispatch table.

The "sglang PR #30117" page (related PR) and the "vllm PR #48774" page
(impl. items 3-4) freeze measured autotuning results into a static table
keyed by shape; this is the same method for this library's two kernels.

For each (M, N, K) point, every admissible plan is timed the way bench.py
times the GEMM: a HIP graph of back-to-back calls, each call on a different
W from a pool larger than the 256 MB Infinity Cache (cold weights),
replayed several times; the median replay time / calls is the plan's
microseconds per call.  Results are JSON lines.  --emit-table turns result
files into csrc/dispatch_table.inc (exact (K, N, M) keys).

    python -m latency_skinny_gemm_amd.sweep --points headline --out sweep.jsonl
    python -m latency_skinny_gemm_amd.sweep --emit-table sweep.jsonl [...]
"""
import argparse
import ctypes
import datetime
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TABLE = os.path.join(HERE, "csrc", "dispatch_table.inc")

KIND_NAMES = {"dot": 1, "splitk": 2, "tiled": 3, "rows": 4}
DOT_THREADS = (64, 128, 192, 256, 320, 384, 448, 512, 640, 768, 896, 1024)
SPLITS = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64)


def point_sets():
    sys.path.insert(0, ROOT)
    from workloads import configs

    bf16 = [p for p in configs.all_points() if p.dtype == "bf16"]
    uniq = lambda ps: sorted({(p.M, p.N, p.K) for p in ps}, key=lambda t: (t[2], t[1], t[0]))
    fp8 = [p for p in configs.all_points() if p.dtype != "bf16"]
    return {
        "headline": uniq(configs.HEADLINE),
        "router": uniq([p for p in bf16 if p.group in ("small_bf16", "router_k7168", "router_shapes")]),
        "decode": uniq([p for p in bf16 if p.group == "decode_linear"]),
        "all": uniq(bf16),
        "fp8": uniq([p for p in fp8 if p.group.startswith("fp8_")]),
        "large_bf16": uniq([p for p in configs.larger_m_full() if p.dtype == "bf16"]),
        "large_fp8": uniq([p for p in configs.larger_m_full() if p.dtype != "bf16"]),
    }


def _natural_mt(M):
    mt = -(-M // 16)
    return next((v for v in (1, 2, 4, 8) if v >= mt), 8)


def _mt_requests(M):
    """m_tiles a tiled plan may ask for at M rows: 0 (the rows' own power of
    two, 8 above 128 rows) and each smaller power of two (more row blocks)."""
    nat = _natural_mt(M)
    return (0,) + tuple(v for v in (1, 2, 4) if v < nat)


def _tiled_reductions(skg, S):
    """Reductions tried for a tiled plan with S splits: the last arriver reads
    S partial tiles in one workgroup, worth it only up to 16 splits."""
    if S == 1:
        return (skg.REDUCE_NONE,)
    return (skg.REDUCE_KERNEL, skg.REDUCE_LAST) if S <= 16 else (skg.REDUCE_KERNEL,)


def fp8_candidates(skg, M, N, K):
    """Admissible FP8 plans (dot kernel for M <= 16, MFMA split-K)."""
    out, seen = [], set()

    def add(p):
        try:
            q = skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
        except skg.SkinnyGemmError:
            return
        key = (q.kind, q.threads, q.cols, q.splits, q.depth, q.waves_m, q.reduce, q.flags,
               q.k_chunk, q.m_tiles)
        if key not in seen:
            seen.add(key)
            out.append(q)

    if M <= 16:
        for T in DOT_THREADS:
            for C in (1, 2, 4):
                add(skg.make_plan(skg.KIND_DOT, T, C))
    if M <= 32:
        # whole-row ring: 8 or 16 columns, 4 or 8 waves, stages of 1024 or 512 K
        for R in (8, 16):
            for T in (256, 512):
                for ns in (3, 4, 5, 6):
                    for fl in (0, skg.FLAG_ROWS_HALF):
                        add(skg.make_plan(skg.KIND_ROWS, T, R, depth=ns, flags=fl))
    # LDS-ring tiles (K % 128 == 0), also in row blocks of fewer m-tiles
    if K % 128 == 0 and (M > 4 or N >= 1024):
        for mtr in _mt_requests(M):
            MB = -(-M // (16 * (mtr or _natural_mt(M))))
            for NB in (1, 2, 4, 8, 16):
                groups = MB * -(-N // (16 * NB))
                for S in SPLITS:
                    if S > K // 128 or not (64 <= groups * S <= 2048):
                        continue
                    for wm in (1, 2, 4):
                        for ns, flags in ((2, 0), (3, 0), (4, 0), (5, 0), (6, 0), (8, 0),
                                          (2, skg.FLAG_TILED_WIDE), (3, skg.FLAG_TILED_WIDE),
                                          (4, skg.FLAG_TILED_WIDE), (5, skg.FLAG_TILED_WIDE)):
                            for red in _tiled_reductions(skg, S):
                                add(skg.make_plan(skg.KIND_TILED, 256, NB, S, ns, red,
                                                  flags=flags, waves_m=wm, m_tiles=mtr))
    ksteps = -(-K // 128)
    for NB in (1, 2, 4):
        groups = -(-N // (16 * NB))
        for S in SPLITS:
            if S > ksteps or groups * S > 8192:
                continue
            for nw in (1, 2, 4, 8):
                for d in (1, 2, 4):
                    for red in ((skg.REDUCE_NONE,) if S == 1 else (skg.REDUCE_LAST, skg.REDUCE_KERNEL)):
                        add(skg.make_plan(skg.KIND_SPLITK, nw * 64, NB, S, d, red))
    return out


def sweep_point_fp8(skg, torch, M, N, K, pool_bytes, reps, stream, log):
    """Times every FP8 plan in both scale modes; ranks by the sum."""
    dev = torch.device("cuda:0")
    slots = max(4, -(-pool_bytes // (N * K)))
    g = torch.Generator(device=dev)
    g.manual_seed(M * 1000003 + N * 1009 + K + 7)
    W = torch.randn((slots, N, K), generator=g, device=dev).clamp(-448, 448).to(torch.float8_e4m3fn)
    X = torch.randn((slots, M, K), generator=g, device=dev).to(torch.float8_e4m3fn)
    O = torch.empty((slots, M, N), dtype=torch.bfloat16, device=dev)
    sx = torch.ones(1, dtype=torch.float32, device=dev)
    # MX exponents per slot like W itself, so the scale bytes are cold too
    XE = torch.randint(126, 129, (slots, M, K // 32), generator=g, device=dev).to(torch.uint8)
    WE = torch.randint(126, 129, (slots, N, K // 32), generator=g, device=dev).to(torch.uint8)
    tensor = skg.Fp8Scales()
    tensor.mode, tensor.sx, tensor.sw = skg.FP8_PER_TENSOR, sx.data_ptr(), sx.data_ptr()
    mx = []
    for sl in range(slots):
        sc = skg.Fp8Scales()
        sc.mode, sc.x_e8m0, sc.w_e8m0 = skg.FP8_MX32, XE[sl].data_ptr(), WE[sl].data_ptr()
        mx.append(sc)
    modes = {"tensor": [tensor] * slots, "mx": mx}
    sptr = ctypes.c_void_p(stream.cuda_stream)
    L = skg.lib()
    results = []
    for p in fp8_candidates(skg, M, N, K):
        per_mode = {}
        for mname, sc in modes.items():
            if mname == "mx":
                # MX plans must also fit the scale bytes (tiled plans hold a
                # K chunk's worth in LDS): the others time per-tensor only
                try:
                    skg.plan_complete(M, N, K, p, skg.DTYPE_FP8_MX)
                except skg.SkinnyGemmError:
                    per_mode[mname] = None
                    continue
            def calls(p=p, sc=sc):
                for s in range(slots):
                    rc = L.skinny_gemm_fp8_planned(X[s].data_ptr(), W[s].data_ptr(), None,
                                                   ctypes.byref(sc[s]), O[s].data_ptr(), M, N, K,
                                                   ctypes.byref(p), sptr)
                    if rc != 0:
                        raise skg.SkinnyGemmError(rc, f"fp8 planned {p}")
            # the point's first timing is taken twice (the first pass after
            # new inputs runs slower), as in the bf16 sweep
            for _ in range(1 if (results or per_mode) else 2):
                with torch.cuda.stream(stream):
                    calls()
                stream.synchronize()
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=stream):
                    calls()
                times = []
                with torch.cuda.stream(stream):
                    gr.replay()
                    for _ in range(reps):
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        gr.replay()
                        e1.record(stream)
                        e1.synchronize()
                        times.append(e0.elapsed_time(e1) * 1e3 / slots)
                del gr
            times.sort()
            per_mode[mname] = times[len(times) // 2]
        results.append((per_mode["tensor"] + (per_mode["mx"] if per_mode["mx"] is not None
                                               else float("inf")), per_mode, p))
    results.sort(key=lambda r: r[0])
    _, best_modes, best = results[0]
    rec = {"dtype": "fp8", "M": M, "N": N, "K": K, "slots": slots, "tiled": "ring2",
           "mx_scales": "per_slot", "mx_tiled": "chunk_scales", "dot_wave1": "direct",
           "dot_reduce": "scatter",
           "best_us": round(max(best_modes.values()), 3),
           "best_us_tensor": round(best_modes["tensor"], 3), "best_us_mx": round(best_modes["mx"], 3),
           "best": plan_dict(best),
           "candidates": [[round(t, 3) if t != float("inf") else None,
                           {k: (round(v, 3) if v is not None else None) for k, v in pm.items()},
                           plan_dict(p)] for t, pm, p in results]}
    log.write(json.dumps(rec) + "\n")
    log.flush()
    kind = {1: "dot", 2: "splitk", 3: "tiled", 4: "rows"}[best.kind]
    print(f"FP8 M={M:3d} N={N:5d} K={K:5d}: best per-tensor {best_modes['tensor']:7.3f} us, "
          f"MX {best_modes['mx']:7.3f} us  {kind} {plan_dict(best)} ({len(results)} plans)", flush=True)
    return rec


def candidates(skg, M, N, K):
    """Every admissible plan of both kernels for (M, N, K), deduplicated on
    the completed plan."""
    out, seen = [], set()

    def add(p):
        try:
            q = skg.plan_complete(M, N, K, p)
        except skg.SkinnyGemmError:
            return
        key = (q.kind, q.threads, q.cols, q.splits, q.depth, q.waves_m, q.reduce, q.flags, q.k_chunk,
               q.m_tiles)
        if key not in seen:
            seen.add(key)
            out.append(q)

    if M <= 16:
        for flags in (0, skg.FLAG_DOT2, skg.FLAG_DOT2 | skg.FLAG_DOT_WFIRST):
            for cols in (1, 2, 3, 4):
                for T in DOT_THREADS:
                    add(skg.make_plan(skg.KIND_DOT, T, cols, flags=flags))
        # x in LDS: waves of 1, 2 or 4 columns
        for T in DOT_THREADS:
            for cw in (1, 2, 4):
                add(skg.make_plan(skg.KIND_DOT, T, cw * T // 64,
                                  flags=skg.FLAG_DOT_XLDS | skg.FLAG_DOT2))
    if M <= 64:
        # whole-row MFMA ring: 8, 10, 12 or 16 columns, 4 or 8 waves, 3-6
        # stages of 512 or 256 K (fewer columns make stages too small to keep
        # enough bytes in flight: 5.2 against 2.8 us for one column at the
        # router's M = 1)
        for R in (8, 10, 12, 16):
            for T in (256, 512):
                for ns in (3, 4, 5, 6):
                    for fl in (0, skg.FLAG_ROWS_HALF):
                        add(skg.make_plan(skg.KIND_ROWS, T, R, depth=ns, flags=fl))
    ksteps = -(-K // 32)
    MT = -(-M // 16)
    for NB in (1, 2, 4):
        if NB * MT > 32:
            continue
        groups = -(-N // (16 * NB))
        for S in SPLITS:
            if S > ksteps or groups * S > 8192:
                continue
            sps = -(-ksteps // S)
            for nw in (1, 2, 4, 8, 16):
                spw = -(-sps // nw)
                D = next((d for d in (1, 2, 4, 8) if d >= spw), 8)
                for d in sorted({D, max(1, D // 2)}):
                    for red in ((skg.REDUCE_NONE,) if S == 1 else (skg.REDUCE_LAST, skg.REDUCE_KERNEL)):
                        add(skg.make_plan(skg.KIND_SPLITK, nw * 64, NB, S, d, red))
    # LDS-ring tiles (K % 32 == 0): worth it once a workgroup covers many
    # columns; stages and steps per stage cover 2-16 steps in flight
    if (M > 4 or N >= 1024) and K % 32 == 0:
        for mtr in _mt_requests(M):
            MB = -(-M // (16 * (mtr or _natural_mt(M))))
            for NB in (1, 2, 4, 8, 16):
                groups = MB * -(-N // (16 * NB))
                for S in SPLITS:
                    if S > ksteps or not (64 <= groups * S <= 2048):
                        continue
                    for wm in (1, 2, 4):
                        for ns, flags in ((2, 0), (3, 0), (4, 0), (5, 0), (6, 0), (8, 0),
                                          (2, skg.FLAG_TILED_WIDE), (3, skg.FLAG_TILED_WIDE),
                                          (4, skg.FLAG_TILED_WIDE), (5, skg.FLAG_TILED_WIDE),
                                          (6, skg.FLAG_TILED_WIDE)):
                            for red in _tiled_reductions(skg, S):
                                add(skg.make_plan(skg.KIND_TILED, 256, NB, S, ns, red,
                                                  flags=flags, waves_m=wm, m_tiles=mtr))
    return out


def plan_dict(p):
    return {k: getattr(p, k) for k in ("kind", "threads", "cols", "splits", "depth", "waves_m",
                                       "reduce", "flags", "k_chunk", "m_tiles", "grid")}


def sweep_point(skg, torch, M, N, K, pool_bytes, reps, stream, log, kinds=None):
    dev = torch.device("cuda:0")
    slots = max(4, -(-pool_bytes // (N * K * 2)))
    g = torch.Generator(device=dev)
    g.manual_seed(M * 1000003 + N * 1009 + K)
    W = (torch.randn((slots, N, K), generator=g, device=dev) * K ** -0.5).to(torch.bfloat16)
    X = torch.randn((slots, M, K), generator=g, device=dev).to(torch.bfloat16)
    O = torch.empty((slots, M, N), dtype=torch.bfloat16, device=dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    L = skg.lib()
    results = []
    for p in candidates(skg, M, N, K):
        if kinds and p.kind not in kinds:
            continue

        def calls(p=p):
            for s in range(slots):
                rc = L.skinny_gemm_bf16_planned(X[s].data_ptr(), W[s].data_ptr(), None,
                                                O[s].data_ptr(), M, N, K, ctypes.byref(p), sptr)
                if rc != 0:
                    raise skg.SkinnyGemmError(rc, f"planned {p}")
        # the first pass after the point's inputs are allocated runs slower
        # throughout (measured up to 1 us a call): the first candidate is
        # timed twice and keeps the second
        for _ in range(1 if results else 2):
            with torch.cuda.stream(stream):
                calls()  # eager once: grows the workspace outside capture
            stream.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                calls()
            times = []
            with torch.cuda.stream(stream):
                gr.replay()
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    gr.replay()
                    e1.record(stream)
                    e1.synchronize()
                    times.append(e0.elapsed_time(e1) * 1e3 / slots)
            del gr
        times.sort()
        results.append((times[len(times) // 2], p))
    if not results:
        return None
    results.sort(key=lambda r: r[0])
    best_us, best = results[0]
    rec = {"M": M, "N": N, "K": K, "slots": slots, "tiled": "ring2", "dot_wave1": "direct",
           "dot_reduce": "scatter",
           "best_us": round(best_us, 3),
           "best": plan_dict(best),
           "candidates": [[round(us, 3), plan_dict(p)] for us, p in results]}
    log.write(json.dumps(rec) + "\n")
    log.flush()
    kind = {1: "dot", 2: "splitk", 3: "tiled", 4: "rows"}[best.kind]
    print(f"M={M:3d} N={N:5d} K={K:5d}: best {best_us:7.3f} us  {kind} {plan_dict(best)} "
          f"({len(results)} plans, slots={slots})", flush=True)
    return rec


def run(args):
    import torch

    import latency_skinny_gemm_amd as skg

    assert torch.cuda.is_available(), "the sweep runs on the GPU"
    pts = point_sets()[args.points]
    if args.M:
        pts = [p for p in pts if p[0] in args.M]
    if args.N:
        pts = [p for p in pts if p[1] in args.N]
    if args.K:
        pts = [p for p in pts if p[2] in args.K]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        skg.reserve(128, 4096, 0, 64)
    t0 = time.time()
    with open(args.out, "a") as log:
        for (M, N, K) in pts:
            if args.points in ("fp8", "large_fp8"):
                sweep_point_fp8(skg, torch, M, N, K, args.pool_mb << 20, args.reps, stream, log)
            else:
                sweep_point(skg, torch, M, N, K, args.pool_mb << 20, args.reps, stream, log,
                            kinds={KIND_NAMES[k] for k in args.kinds} if args.kinds else None)
            torch.cuda.empty_cache()
    print(f"swept {len(pts)} points in {time.time() - t0:.0f} s", flush=True)


def _mt_request_of(plan, M):
    """The m_tiles a recorded tiled plan asked for: 0 when it used the rows'
    own power of two (records from before row blocks below 129 rows carry
    none), else its m_tiles."""
    mt = plan.get("m_tiles", 0)
    return 0 if plan["kind"] != 3 or mt in (0, _natural_mt(M)) else mt


def _still_valid(skg, dt, M, N, K, b):
    """True when the current planner accepts the swept plan unchanged."""
    p = skg.make_plan(b["kind"], b["threads"], b["cols"], b["splits"], b["depth"], b["reduce"],
                      flags=b["flags"], waves_m=b.get("waves_m", 0),
                      m_tiles=_mt_request_of(b, M))
    try:
        q = skg.plan_complete(M, N, K, p, {"fp8": skg.DTYPE_FP8, "fp8_mx": skg.DTYPE_FP8_MX}.get(
            dt, skg.DTYPE_BF16))
    except skg.SkinnyGemmError:
        return False
    return (q.splits, q.depth, q.cols) == (b["splits"], b["depth"], b["cols"]) and \
        (b["kind"] != 3 or q.m_tiles == (b.get("m_tiles") or q.m_tiles))


def emit_table(files, out_path=TABLE):
    """Per (dtype, K, N, M), the fastest swept plan that the current planner
    still accepts, over every record of the given sweep logs.  A plan timed
    in several logs is ranked by the median of its timings, so one lucky
    run does not pick it."""
    import statistics

    import latency_skinny_gemm_amd as skg

    timings = {}
    for f in files:
        for line in open(f):
            r = json.loads(line)
            key = (r.get("dtype", "bf16"), r["K"], r["N"], r["M"])
            for c in r["candidates"]:
                us, plan = (c[0], c[-1])
                # TILED timings of earlier tiled kernels mean other plans
                if plan["kind"] == 3 and r.get("tiled") != "ring2":
                    continue
                # so do one-wave dot timings from before its direct-store path
                if plan["kind"] == 1 and plan["threads"] == 64 and r.get("dot_wave1") != "direct":
                    continue
                # and dot timings from before its reduce-scatter
                if plan["kind"] == 1 and r.get("dot_reduce") != "scatter":
                    continue
                ident = tuple(plan.get(f, 0) for f in ("kind", "threads", "cols", "splits", "depth",
                                                          "waves_m", "reduce", "flags"))
                ident += (_mt_request_of(plan, key[3]),)
                # FP8: one entry per scale mode, each from that mode's timing;
                # MX timings count only where the scale bytes were cold too
                per_key = [(key, us)] if key[0] != "fp8" else [(key, c[1]["tensor"])]
                # (MX timings of tiled plans only since their scale bytes load
                # once per K chunk)
                if key[0] == "fp8" and r.get("mx_scales") == "per_slot" and \
                        c[1].get("mx") is not None and \
                        (plan["kind"] != 3 or r.get("mx_tiled") == "chunk_scales"):
                    per_key.append((("fp8_mx",) + key[1:], c[1]["mx"]))
                for k, t in per_key:
                    timings.setdefault(k, {}).setdefault(ident, (plan, []))[1].append(t)
    best = {}
    for key, plans in timings.items():
        dt, K, N, M = key
        ranked = sorted(plans.values(), key=lambda v: statistics.median(v[1]))
        for plan, ts in ranked:
            if _still_valid(skg, dt, M, N, K, plan):
                best[key] = {"best_us": statistics.median(ts), "best": plan}
                break
    names = {0: "SKG_REDUCE_NONE", 1: "SKG_REDUCE_LAST", 2: "SKG_REDUCE_KERNEL"}
    kinds = {1: "SKG_KIND_DOT", 2: "SKG_KIND_SPLITK", 3: "SKG_KIND_TILED", 4: "SKG_KIND_ROWS"}
    lines = [
        "// dispatch_table.inc -- generated by latency_skinny_gemm_amd/sweep.py --emit-table",
        f"// from cold-weight graph-replay timings on one MI355X ({datetime.date.today()}).",
        "// {dtype, K, N, M, {kind, threads, cols, splits, depth, waves_m, reduce, flags",
        "//                   [, 0, m_tiles when a tiled plan asks for row blocks]}},  // us/call",
    ]
    dtypes = {"bf16": "SKG_DTYPE_BF16", "fp8": "SKG_DTYPE_FP8", "fp8_mx": "SKG_DTYPE_FP8_MX"}
    for key in sorted(best):
        dt, K, N, M = key
        b = best[key]["best"]
        mtr = _mt_request_of(b, M)
        lines.append(
            f"{{{dtypes[dt]}, {K}, {N}, {M}, {{{kinds[b['kind']]}, {b['threads']}, {b['cols']}, "
            f"{b['splits']}, {b['depth']}, {b.get('waves_m', 0)}, {names[b['reduce']]}, {b['flags']}"
            + (f", 0, {mtr}" if mtr else "") + f"}}}},  // {best[key]['best_us']:.3f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {len(best)} entries to {out_path}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--points", default="headline",
                    choices=("headline", "router", "decode", "all", "fp8", "large_bf16", "large_fp8"))
    ap.add_argument("--M", type=int, nargs="*", help="restrict to these M")
    ap.add_argument("--N", type=int, nargs="*", help="restrict to these N")
    ap.add_argument("--K", type=int, nargs="*", help="restrict to these K")
    ap.add_argument("--out", default="sweep.jsonl", help="JSON-lines log the sweep appends to")
    ap.add_argument("--pool-mb", type=int, default=512)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--emit-table", nargs="+", metavar="JSONL")
    ap.add_argument("--kinds", nargs="*", choices=sorted(KIND_NAMES),
                    help="bf16 points: time only these kernel kinds (the table ranks each plan "
                         "over every log, so a partial sweep adds to earlier ones)")
    args = ap.parse_args()
    if args.emit_table:
        emit_table(args.emit_table)
        return 0
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    run(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
