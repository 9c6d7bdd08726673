"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Every configured workload point runs on the plan the library picks, and on
each kernel explicitly (dot product where M <= 16, split-K with both
reductions).  Random inputs must meet the elementwise bound
|gpu - ref| <= 2^-7 |ref| + 1e-3 sqrt(K) rms(ref); inputs whose every fp32
partial sum is exact (small integers, one-hot, all-ones) must match the
oracle bit for bit.
"""
import ctypes
import functools

import numpy as np
import pytest
import torch

import oracle
from oracle import tolerance
from workloads import configs
from workloads import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def skg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import latency_skinny_gemm_amd as m
    m.lib()
    return m


@functools.lru_cache(maxsize=None)
def _ref_point(p):
    x, w, b = gen.point_inputs(p)
    ref = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), None if b is None else gen.bits16(b),
                           threads=16)
    return x, w, b, ref


def _dev(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _kernel_plans(skg, M, N, K):
    """The library's plan plus one explicit plan per kernel / reduction."""
    plans = [("default", None)]
    if M <= 16:
        for flags in (0, skg.FLAG_DOT2, skg.FLAG_DOT2 | skg.FLAG_DOT_WFIRST):
            for cols in (1, 2, 3, 4):
                for threads in range(256, 1025, 64):  # the smallest workgroup that fits
                    p = skg.make_plan(skg.KIND_DOT, threads, cols=cols, flags=flags)
                    try:
                        skg.plan_complete(M, N, K, p)
                    except skg.SkinnyGemmError:
                        continue
                    plans.append((f"dot_c{cols}_t{threads}_f{flags}", p))
                    break
                p = skg.make_plan(skg.KIND_DOT, 64, cols=cols, flags=flags)  # one wave: no LDS
                try:
                    skg.plan_complete(M, N, K, p)
                    plans.append((f"dot_c{cols}_t64_f{flags}", p))
                except skg.SkinnyGemmError:
                    pass
    if M <= 16:
        # x in LDS: the first multi-wave shape that fits, and one wave
        xl = skg.FLAG_DOT_XLDS | skg.FLAG_DOT2
        for group in (((512, 2), (256, 4), (512, 1), (256, 1)), ((64, 4), (64, 2), (64, 1))):
            for threads, cw in group:
                p = skg.make_plan(skg.KIND_DOT, threads, cols=cw * threads // 64, flags=xl)
                try:
                    skg.plan_complete(M, N, K, p)
                except skg.SkinnyGemmError:
                    continue
                plans.append((f"dotx_cw{cw}_t{threads}", p))
                break
    if M <= 64:
        # whole-row MFMA ring: the first of each pair that fits (16 or 8
        # columns, 4 or 8 waves, stages of 512 or 256 K)
        half = skg.FLAG_ROWS_HALF
        for pair in (((256, 16, 4, 0), (256, 16, 3, half)), ((512, 8, 3, 0), (512, 8, 4, half)),
                     ((512, 16, 6, half), (512, 16, 3, half)), ((256, 8, 5, half), (256, 8, 3, 0)),
                     ((256, 10, 5, half), (512, 12, 3, 0))):
            for threads, cols, ns, fl in pair:
                p = skg.make_plan(skg.KIND_ROWS, threads, cols=cols, depth=ns, flags=fl)
                try:
                    skg.plan_complete(M, N, K, p)
                except skg.SkinnyGemmError:
                    continue
                plans.append((f"rows_t{threads}_c{cols}_ns{ns}_f{fl}", p))
                break
    mt = (M + 15) // 16
    nb = 4 if mt >= 4 else (2 if mt >= 2 else 1)
    threads = 128 if nb * mt > 16 else 256
    plans.append(("splitk_last", skg.make_plan(skg.KIND_SPLITK, threads, cols=nb, splits=8,
                                               depth=2, reduce=skg.REDUCE_LAST)))
    plans.append(("splitk_kernel", skg.make_plan(skg.KIND_SPLITK, threads, cols=nb, splits=5,
                                                 depth=1, reduce=skg.REDUCE_KERNEL)))
    plans.append(("splitk_s1", skg.make_plan(skg.KIND_SPLITK, threads, cols=nb, splits=1,
                                             depth=4 if nb * mt <= 8 else 2)))
    for (S, D, red) in ((1, 4, skg.REDUCE_NONE), (3, 2, skg.REDUCE_KERNEL)):  # 16 waves
        p = skg.make_plan(skg.KIND_SPLITK, 1024, cols=1, splits=S, depth=D, reduce=red)
        try:
            skg.plan_complete(M, N, K, p)
        except skg.SkinnyGemmError:
            continue
        plans.append((f"splitk_t1024_s{S}", p))
    wide = skg.FLAG_TILED_WIDE
    for (nbt, S, ns, fl, red, wm) in ((16, 4, 3, 0, skg.REDUCE_LAST, 0),
                                      (8, 3, 2, wide, skg.REDUCE_KERNEL, 0),
                                      (4, 1, 4, 0, skg.REDUCE_NONE, 4),
                                      (2, 7, 2, wide, skg.REDUCE_LAST, 0),
                                      (8, 8, 4, 0, skg.REDUCE_KERNEL, 1),
                                      (16, 16, 4, 0, skg.REDUCE_KERNEL, 0),
                                      (4, 3, 5, wide, skg.REDUCE_KERNEL, 0),
                                      (2, 2, 6, wide, skg.REDUCE_KERNEL, 2)):
        p = skg.make_plan(skg.KIND_TILED, 256, cols=nbt, splits=S, depth=ns, reduce=red,
                          flags=fl, waves_m=wm)
        try:
            skg.plan_complete(M, N, K, p)
        except skg.SkinnyGemmError:
            continue
        plans.append((f"tiled_nb{nbt}_s{S}_ns{ns}_f{fl}_r{red}_wm{wm}", p))
    # row blocks of fewer m-tiles than the rows need (wider, shorter tiles)
    nat = 1 if M <= 16 else 2 if M <= 32 else 4 if M <= 64 else 8
    for (mt, nbt, S, ns, fl, red) in ((nat // 2, 4, 1, 3, 0, skg.REDUCE_NONE),
                                      (1, 4, 3, 2, wide, skg.REDUCE_KERNEL)):
        if mt < 1 or mt >= nat:
            continue
        p = skg.make_plan(skg.KIND_TILED, 256, cols=nbt, splits=S, depth=ns, reduce=red,
                          flags=fl, m_tiles=mt)
        try:
            skg.plan_complete(M, N, K, p)
        except skg.SkinnyGemmError:
            continue
        plans.append((f"tiled_rows_mt{mt}_nb{nbt}_s{S}", p))
    return plans


def _run(skg, x, w, b, p):
    out = skg.gemm_bf16(x, w, b) if p is None else skg.gemm_bf16_planned(x, w, p, b)
    torch.cuda.synchronize()
    return out.cpu()


BF16_POINTS = [p for p in configs.all_points() if p.dtype == "bf16"]


@pytest.mark.parametrize("p", BF16_POINTS, ids=lambda p: p.key())
def test_point_within_tolerance(skg, p):
    x, w, b, ref = _ref_point(p)
    xd, wd, bd = _dev(x, w, b)
    for name, plan in _kernel_plans(skg, p.M, p.N, p.K):
        if plan is not None:
            try:
                skg.plan_complete(p.M, p.N, p.K, plan)
            except skg.SkinnyGemmError:
                continue  # this explicit shape does not fit the problem
        out = _run(skg, xd, wd, bd, plan)
        ok, msg = tolerance.check(out, ref, p.K)
        assert ok, f"{p.key()} [{name}]: {msg}"


EXACT_SHAPES = [(1, 256, 2048), (3, 100, 2880), (4, 128, 2880), (5, 384, 7168), (9, 256, 4096),
                (16, 256, 6144), (16, 37, 8), (33, 72, 264), (64, 576, 7168), (128, 200, 2056),
                # ragged and degenerate: one column, one row, the shortest K, a K
                # of one 32-wide step, M just past a tile and past one row block
                (1, 1, 8), (2, 1, 4096), (17, 17, 1056), (7, 300, 32), (129, 33, 96),
                (130, 1, 64), (300, 20, 1024)]


@pytest.mark.parametrize("M,N,K", EXACT_SHAPES)
def test_small_integers_bitwise(skg, M, N, K):
    x, w, b = gen.small_integers(M, N, K, True, seed=M * 7919 + N * 31 + K)
    ref = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b), threads=16)
    xd, wd, bd = _dev(x, w, b)
    for name, plan in _kernel_plans(skg, M, N, K):
        if plan is not None:
            try:
                skg.plan_complete(M, N, K, plan)
            except skg.SkinnyGemmError:
                continue
        out = _run(skg, xd, wd, bd, plan)
        got = gen.bits16(out)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"[{name}] {len(bad)} mismatches, first {tuple(bad[0])}"


@pytest.mark.parametrize("M,N,K", [(2, 128, 2880), (16, 256, 7168), (40, 96, 4096)])
def test_one_hot_selects_x_bitwise(skg, M, N, K):
    x, w, pi = gen.one_hot(M, N, K, seed=N + K)
    want = gen.bits16(x)[:, pi.numpy()]
    xd, wd = _dev(x, w)
    for name, plan in _kernel_plans(skg, M, N, K):
        if plan is not None:
            try:
                skg.plan_complete(M, N, K, plan)
            except skg.SkinnyGemmError:
                continue
        got = gen.bits16(_run(skg, xd, wd, None, plan))
        assert np.array_equal(got, want), f"[{name}]"


@pytest.mark.parametrize("K", (2048, 2880, 4096, 6144, 7168))
def test_all_ones_gives_K(skg, K):
    x, w = gen.ones(16, 256, K)
    xd, wd = _dev(x, w)
    for name, plan in _kernel_plans(skg, 16, 256, K):
        out = _run(skg, xd, wd, None, plan)
        assert torch.all(out.float() == K), f"[{name}]"


@pytest.mark.parametrize("M,N,K,T,CW", [(3, 300, 2048, 256, 2), (8, 77, 2048, 512, 1),
                                        (1, 1000, 3072, 64, 4), (5, 130, 4096, 128, 2)])
@pytest.mark.parametrize("bias", (False, True))
def test_xlds_matches_one_wave_dot_bitwise(skg, M, N, K, T, CW, bias):
    # equal V: each lane sums the same vectors in the same order and the
    # wave's reduction tree is the same, so the bits must be the same; N
    # ragged against the workgroup's columns
    x, w, b = gen.bf16_inputs(M, N, K, bias, seed=1000 + M * 31 + N)
    xd, wd, bd = _dev(x, w, b)
    one = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_DOT, 64, 1, flags=skg.FLAG_DOT2))
    xl = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_DOT, T, CW * T // 64,
                                                  flags=skg.FLAG_DOT_XLDS | skg.FLAG_DOT2))
    assert one.depth == xl.depth == K // 512
    a = gen.bits16(_run(skg, xd, wd, bd, one))
    c = gen.bits16(_run(skg, xd, wd, bd, xl))
    assert np.array_equal(a, c), f"{np.count_nonzero(a != c)} of {a.size} differ"


@pytest.mark.parametrize("M,N,K,T,C", [(8, 256, 7168, 448, 1), (16, 384, 7168, 448, 2),
                                       (3, 130, 2880, 192, 1), (12, 1000, 4096, 256, 3),
                                       (1, 77, 2048, 64, 2), (5, 256, 6144, 1024, 4)])
@pytest.mark.parametrize("bias", (False, True))
def test_wfirst_matches_dot_bitwise(skg, M, N, K, T, C, bias):
    # the W-first load order changes no arithmetic: the same plan with and
    # without it gives the same bits (N ragged against the columns)
    x, w, b = gen.bf16_inputs(M, N, K, bias, seed=2000 + M * 37 + N)
    xd, wd, bd = _dev(x, w, b)
    outs = []
    for fl in (skg.FLAG_DOT2, skg.FLAG_DOT2 | skg.FLAG_DOT_WFIRST):
        plan = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_DOT, T, C, flags=fl))
        outs.append(gen.bits16(_run(skg, xd, wd, bd, plan)))
    assert np.array_equal(outs[0], outs[1]), f"{np.count_nonzero(outs[0] != outs[1])} differ"


def test_runs_are_bitwise_deterministic(skg):
    p = configs.Point("det", "bf16", 12, 384, 7168, True)
    x, w, b, _ = _ref_point(p)
    xd, wd, bd = _dev(x, w, b)
    for name, plan in _kernel_plans(skg, p.M, p.N, p.K):
        a = _run(skg, xd, wd, bd, plan)
        c = _run(skg, xd, wd, bd, plan)
        assert torch.equal(a.view(torch.int16), c.view(torch.int16)), f"[{name}]"


def test_reductions_agree_bitwise(skg):
    # the in-kernel last-arriver sum and the second-kernel sum add the same
    # partials in the same order, on the split-K and the tiled kernels; N % 4
    # == 0 takes the 16-byte coherent partials, N = 130 the per-float ones
    for (M, N, K) in ((8, 256, 7168), (64, 576, 7168), (5, 100, 2880), (7, 130, 2880),
                      (128, 1024, 2048), (33, 4096, 1024)):
        x, w, b = gen.bf16_inputs(M, N, K, True, seed=K + M)
        xd, wd, bd = _dev(x, w, b)
        for kind, T, cols, S, D, fl in ((skg.KIND_SPLITK, 128, 1, 7, 2, 0),
                                        (skg.KIND_TILED, 256, 4, 4, 3, 0),
                                        (skg.KIND_TILED, 256, 2, 3, 3, skg.FLAG_TILED_WIDE)):
            outs = []
            for red in (skg.REDUCE_LAST, skg.REDUCE_KERNEL):
                plan = skg.make_plan(kind, T, cols=cols, splits=S, depth=D, reduce=red, flags=fl)
                try:
                    plan = skg.plan_complete(M, N, K, plan)
                except skg.SkinnyGemmError:
                    break
                outs.append(_run(skg, xd, wd, bd, plan))
            if len(outs) == 2:
                assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), \
                    (M, N, K, kind, S)


def test_output_guard_bands_untouched(skg):
    M, N, K = 7, 130, 2880
    G = 4096
    x, w, b = gen.bf16_inputs(M, N, K, True, seed=5)
    ref = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b), threads=16)
    xd, wd, bd = _dev(x, w, b)
    for name, plan in _kernel_plans(skg, M, N, K):
        buf = torch.full((G + M * N + G,), -7.0, dtype=torch.bfloat16, device=DEV)
        out = buf[G:G + M * N].view(M, N)
        if plan is None:
            skg.gemm_bf16(xd, wd, bd, out=out)
        else:
            skg.gemm_bf16_planned(xd, wd, plan, bd, out=out)
        torch.cuda.synchronize()
        host = buf.cpu()
        assert torch.all(host[:G] == -7.0) and torch.all(host[G + M * N:] == -7.0), f"[{name}]"
        ok, msg = tolerance.check(host[G:G + M * N].view(M, N), ref, K)
        assert ok, f"[{name}] {msg}"


def test_graph_replays_match_eager(skg):
    shapes = [(1, 256, 7168), (8, 256, 7168), (16, 384, 7168), (64, 576, 7168)]
    stream = torch.cuda.Stream()
    data = []
    for (M, N, K) in shapes:
        x, w, b = gen.bf16_inputs(M, N, K, False, seed=M * N)
        data.append(_dev(x, w, b))
    with torch.cuda.stream(stream):
        skg.reserve(128, 4096, 0, 64)
        eager = [skg.gemm_bf16(x, w, b) for (x, w, b) in data]
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for (x, w, b), o in zip(data, outs):
            skg.gemm_bf16(x, w, b, out=o)
    for _ in range(3):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert torch.equal(e.view(torch.int16), o.view(torch.int16))


def test_capture_needs_reserved_workspace(skg):
    # a split plan captured on a stream with no workspace is refused (no
    # allocation or synchronisation inside a capture); once reserved, the
    # same capture replays equal to the eager result
    M, N, K = 16, 256, 7168
    x, w, b = _dev(*gen.bf16_inputs(M, N, K, True, seed=123))
    plan = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_SPLITK, 256, 1, 16, 4,
                                                    skg.REDUCE_KERNEL))
    skg.release_all()
    stream = torch.cuda.Stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    out = torch.zeros(M, N, dtype=torch.bfloat16, device=DEV)
    lib = skg.lib()

    def call():
        return lib.skinny_gemm_bf16_planned(x.data_ptr(), w.data_ptr(), b.data_ptr(),
                                            out.data_ptr(), M, N, K, ctypes.byref(plan), sptr)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        rc = call()
    assert rc == skg.ERR_WORKSPACE
    del g
    with torch.cuda.stream(stream):
        skg.reserve(M, N, K, 16)
        assert call() == skg.OK
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        rc = call()
    assert rc == skg.OK
    for _ in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
    del g
    # after a release the next eager call on the stream allocates afresh
    skg.release_all()
    out.fill_(0)
    with torch.cuda.stream(stream):
        assert call() == skg.OK
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


def test_threads_on_their_own_streams(skg):
    # host threads calling at once on their own streams: each stream gets
    # its own workspace (grown while the others run), and every result equals
    # the single-threaded one bit for bit
    import threading

    lib = skg.lib()
    cases = []
    for i, (M, N, K, S) in enumerate(((16, 256, 7168, 16), (32, 576, 7168, 8), (8, 384, 4096, 4),
                                      (64, 1024, 2048, 2))):
        x, w, b = _dev(*gen.bf16_inputs(M, N, K, True, seed=700 + i))
        plan = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_SPLITK, 256, 1, S, 2,
                                                        skg.REDUCE_KERNEL))
        ref = skg.gemm_bf16_planned(x, w, plan, b)
        cases.append((M, N, K, x, w, b, plan, ref))
    torch.cuda.synchronize()
    skg.release_all()
    errors = []

    def worker(case):
        M, N, K, x, w, b, plan, ref = case
        stream = torch.cuda.Stream()
        sptr = ctypes.c_void_p(stream.cuda_stream)
        outs = [torch.zeros(M, N, dtype=torch.bfloat16, device=DEV) for _ in range(20)]
        torch.cuda.synchronize()
        for o in outs:
            rc = lib.skinny_gemm_bf16_planned(x.data_ptr(), w.data_ptr(), b.data_ptr(), o.data_ptr(),
                                              M, N, K, ctypes.byref(plan), sptr)
            if rc != skg.OK:
                errors.append(f"M={M}: status {rc}")
                return
        stream.synchronize()
        for o in outs:
            if not torch.equal(o.view(torch.int16), ref.view(torch.int16)):
                errors.append(f"M={M} N={N}: differs from the single-threaded result")
                return

    threads = [threading.Thread(target=worker, args=(c,)) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors


def test_first_call_on_a_fresh_non_blocking_stream(skg):
    # A new workspace's tile counters are zeroed on the call's own stream.
    # torch's side streams do not wait for the null stream, so counters
    # zeroed there could still hold old bytes when the first kernel reads
    # them and whole tiles would go unwritten.  Old bytes are planted first:
    # memory filled with 0xFF and handed back to HIP, which the library's
    # next allocations are likely to reuse.
    M, N, K = 20, 700, 2056
    x, w, b = _dev(*gen.bf16_inputs(M, N, K, True, seed=901))
    plan = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_SPLITK, 256, 2, 11, 2, skg.REDUCE_LAST))
    ref = oracle.gemm_bf16(gen.bits16(x.cpu()), gen.bits16(w.cpu()), gen.bits16(b.cpu()), threads=16)
    for trial in range(3):
        torch.cuda.synchronize()
        skg.release_all()
        junk = torch.full((64 << 20,), -1, dtype=torch.int32, device=DEV)
        torch.cuda.synchronize()
        del junk
        torch.cuda.empty_cache()
        stream = torch.cuda.Stream()
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        torch.cuda.synchronize()
        got = skg.gemm_bf16_planned(x, w, plan, b, out=out, stream=stream)
        stream.synchronize()
        ok, msg = tolerance.check(got.cpu(), ref, K)
        assert ok, f"trial {trial}: {msg}"


def test_per_thread_stream_workspaces_belong_to_threads(skg):
    # hipStreamPerThread is one handle for a different stream in every host
    # thread; the library keys its workspaces by the calling thread there, so
    # threads running split-K calls with different split counts at once do
    # not share partials or tile counters
    import threading

    lib = skg.lib()
    per_thread = ctypes.c_void_p(2)  # hipStreamPerThread
    cases = []
    for i, (M, N, K, S, red) in enumerate(((16, 256, 7168, 16, skg.REDUCE_LAST),
                                           (16, 256, 7168, 7, skg.REDUCE_LAST),
                                           (8, 384, 4096, 4, skg.REDUCE_KERNEL),
                                           (8, 384, 4096, 9, skg.REDUCE_LAST))):
        x, w, b = _dev(*gen.bf16_inputs(M, N, K, True, seed=800 + i))
        plan = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_SPLITK, 256, 1, S, 2, red))
        ref = skg.gemm_bf16_planned(x, w, plan, b)
        cases.append((M, N, K, x, w, b, plan, ref))
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(len(cases))

    def worker(case):
        M, N, K, x, w, b, plan, ref = case
        torch.cuda.set_device(0)
        outs = [torch.zeros(M, N, dtype=torch.bfloat16, device=DEV) for _ in range(30)]
        torch.cuda.synchronize()
        # one eager call grows this thread's workspace, then all run at once
        if lib.skinny_gemm_bf16_planned(x.data_ptr(), w.data_ptr(), b.data_ptr(), outs[0].data_ptr(),
                                        M, N, K, ctypes.byref(plan), per_thread) != skg.OK:
            errors.append(f"M={M} S={plan.splits}: first call failed")
        start.wait()
        for o in outs:
            rc = lib.skinny_gemm_bf16_planned(x.data_ptr(), w.data_ptr(), b.data_ptr(), o.data_ptr(),
                                              M, N, K, ctypes.byref(plan), per_thread)
            if rc != skg.OK:
                errors.append(f"M={M}: status {rc}")
                return
        torch.cuda.synchronize()
        for o in outs:
            if not torch.equal(o.view(torch.int16), ref.view(torch.int16)):
                errors.append(f"M={M} S={plan.splits}: differs from the single-threaded result")
                return

    threads = [threading.Thread(target=worker, args=(c,)) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors


def test_release_all_keeps_the_current_device(skg):
    M, N, K = 16, 256, 7168
    x, w, b = _dev(*gen.bf16_inputs(M, N, K, False, seed=5))
    skg.gemm_bf16_planned(x, w, skg.make_plan(skg.KIND_SPLITK, 256, 1, 8, 2, skg.REDUCE_KERNEL))
    torch.cuda.synchronize()
    before = torch.cuda.current_device()
    skg.release_all()
    assert torch.cuda.current_device() == before
    skg.release_all()  # nothing held: a no-op
    assert torch.cuda.current_device() == before


def test_error_statuses_on_device(skg):
    x = torch.zeros(2, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(8, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        skg.gemm_bf16(x, torch.zeros(8, 56, dtype=torch.bfloat16, device=DEV))  # K mismatch
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.gemm_bf16(torch.zeros(2, 60, dtype=torch.bfloat16, device=DEV),
                      torch.zeros(8, 60, dtype=torch.bfloat16, device=DEV))
    assert e.value.status == skg.ERR_UNSUPPORTED  # K % 8 != 0
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.gemm_bf16(torch.zeros(513, 64, dtype=torch.bfloat16, device=DEV), w)
    assert e.value.status == skg.ERR_UNSUPPORTED  # M > 512
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.gemm_bf16(torch.zeros(129, 72, dtype=torch.bfloat16, device=DEV),
                      torch.zeros(8, 72, dtype=torch.bfloat16, device=DEV))
    assert e.value.status == skg.ERR_UNSUPPORTED  # M > 128 needs K % 32 == 0
    lib = skg.lib()
    flat = torch.zeros(2 * 64 + 8, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(2, 8, dtype=torch.bfloat16, device=DEV)
    rc = lib.skinny_gemm_bf16(flat.data_ptr() + 2, w.data_ptr(), None, None, out.data_ptr(),
                              2, 8, 64, None)
    assert rc == skg.ERR_ALIGNMENT
    rc = lib.skinny_gemm_bf16(x.data_ptr(), w.data_ptr(), None, None, x.data_ptr(), 2, 8, 64, None)
    assert rc == skg.ERR_INVALID_ARG  # out overlaps x
    torch.cuda.synchronize()


# ------------------------------------------------ larger M at full size
# M = 512 on the dense decode shape (N = 4096, K = 7168): the oracle computes
# sampled outputs one by one (an output depends only on its row of x and its
# row of W), in every row block and column group corner.
@pytest.mark.parametrize("bias", (False, True))
def test_large_M_full_size_sampled(skg, bias):
    M, N, K = 512, 4096, 7168
    x, w, b = gen.bf16_inputs(M, N, K, bias, seed=512 + bias)
    xd, wd = x.to(DEV), w.to(DEV)
    bd = None if b is None else b.to(DEV)
    out = skg.gemm_bf16(xd, wd, bd)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 255, 300, 384, 511])
    cols = np.concatenate([np.arange(0, 16), np.arange(4080, 4096),
                           np.random.default_rng(1).integers(0, N, 32)])
    ref = oracle.gemm_bf16(gen.bits16(x[rows]), gen.bits16(w[cols]),
                           None if b is None else gen.bits16(b[cols]), threads=16)
    got = out.cpu()[rows][:, cols]
    ok, msg = tolerance.check(got, ref, K)
    assert ok, msg


def test_binding_side_stream_matches_current_stream(skg):
    # the binding runs a call on the stream it is given (its new output is
    # allocated for that stream): the same bits as on the current stream
    M, N, K = 12, 384, 7168
    x, w, b = _dev(*gen.bf16_inputs(M, N, K, True, seed=321))
    ref = skg.gemm_bf16(x, w, b)
    ref32 = skg.gemm_bf16_f32(x, w, b)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = skg.gemm_bf16(x, w, b, stream=side)
    got32 = skg.gemm_bf16_f32(x, w, b, stream=side)
    side.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(got32.view(torch.int32), ref32.view(torch.int32))


# shapes off the dispatch table, one or more per branch of the default rule
# at 256 CUs: the dot kernel with 4 and with 1 column(s), the small-N dot
# kernel above 4 rows, the dot kernel with 3-4 columns between N = 512 and
# the ring, the whole-row ring (5 to 32 rows, 8-column groups
# filling half the CUs, M * K <= 114688; ragged K, 12 columns, half-width
# stages above 16 rows), the tiled kernel (too few groups, x past the bound,
# past 32 rows), and split-K for K not a multiple of 32
DEFAULT_RULE_SHAPES = [((2, 2048, 1024), "dot"), ((3, 300, 2048), "dot"), ((12, 256, 3072), "dot"),
                       ((6, 1536, 2048), "rows"), ((16, 2048, 2056), "rows"),
                       ((12, 3072, 2048), "rows"), ((32, 1024, 2048), "rows"),
                       ((8, 768, 4096), "dot"), ((10, 704, 6144), "dot"),
                       ((24, 640, 2048), "tiled"), ((18, 1024, 7168), "tiled"),
                       ((40, 2048, 2048), "tiled"), ((8, 700, 2056), "dot"),
                       ((24, 640, 2056), "splitk")]


@pytest.mark.parametrize("shape,kind", DEFAULT_RULE_SHAPES, ids=str)
def test_default_rule_plans_within_tolerance(skg, shape, kind):
    M, N, K = shape
    q = skg.plan(M, N, K)
    assert q.from_table == 0
    want = {"dot": skg.KIND_DOT, "rows": skg.KIND_ROWS, "tiled": skg.KIND_TILED,
            "splitk": skg.KIND_SPLITK}[kind]
    assert q.kind == want, q
    x, w, b = gen.bf16_inputs(M, N, K, True, seed=M + N + K)
    ref = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b), threads=16)
    out = _run(skg, *_dev(x, w, b), None)
    ok, msg = tolerance.check(out, ref, K)
    assert ok, f"{shape} plan {q}: {msg}"
