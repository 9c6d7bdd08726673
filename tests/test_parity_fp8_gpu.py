"""GPU parity of the FP8 e4m3 paths (per-tensor and MX scales) against the
CPU oracle, through the C ABI.

Random points must meet |gpu - ref| <= 2^-7 |ref| + 1e-3 sqrt(K) rms(ref);
inputs whose every fp32 partial sum is exact (small e4m3 integers, unit or
near-unit power-of-two scales) must match bit for bit.
"""
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


def _plans(skg, M, N, K):
    plans = [("default", None)]
    if M <= 16:
        for C in (1, 2, 4):
            for T in range(256, 1025, 64):
                p = skg.make_plan(skg.KIND_DOT, T, C)
                try:
                    skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
                except skg.SkinnyGemmError:
                    continue
                plans.append((f"dot_t{T}_c{C}", p))
                break
            p = skg.make_plan(skg.KIND_DOT, 64, C)  # one wave: no LDS
            try:
                skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
                plans.append((f"dot_t64_c{C}", p))
            except skg.SkinnyGemmError:
                pass
    mt = (M + 15) // 16
    nb = 2 if mt <= 3 else 1
    for (T, S, D, red) in ((256, 4, 1, skg.REDUCE_LAST), (128, 3, 2, skg.REDUCE_KERNEL),
                           (256, 1, 1, skg.REDUCE_NONE)):
        p = skg.make_plan(skg.KIND_SPLITK, T, nb, S, D, red)
        try:
            skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
        except skg.SkinnyGemmError:
            continue
        plans.append((f"mfma_t{T}_s{S}_d{D}_r{red}", p))
    wide = skg.FLAG_TILED_WIDE
    for (NBt, S, NS, fl, red, wm) in ((8, 4, 3, 0, skg.REDUCE_KERNEL, 0),
                                      (4, 2, 2, wide, skg.REDUCE_LAST, 0),
                                      (2, 1, 4, 0, skg.REDUCE_NONE, 4),
                                      (16, 8, 2, 0, skg.REDUCE_KERNEL, 1),
                                      (2, 3, 5, 0, skg.REDUCE_KERNEL, 0),
                                      (4, 2, 5, wide, skg.REDUCE_KERNEL, 2)):
        p = skg.make_plan(skg.KIND_TILED, 256, NBt, S, NS, red, flags=fl, waves_m=wm)
        try:
            skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
        except skg.SkinnyGemmError:
            continue
        plans.append((f"tiled_nb{NBt}_s{S}_ns{NS}_f{fl}_r{red}_wm{wm}", p))
    if M <= 32:
        # whole-row ring: the first of each pair that fits
        half = skg.FLAG_ROWS_HALF
        for pair in (((256, 16, 4, 0), (256, 16, 3, half)), ((512, 8, 3, 0), (256, 8, 5, half))):
            for T, R, NS, fl in pair:
                p = skg.make_plan(skg.KIND_ROWS, T, R, depth=NS, flags=fl)
                try:
                    skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
                except skg.SkinnyGemmError:
                    continue
                plans.append((f"rows_t{T}_c{R}_ns{NS}_f{fl}", p))
                break
    # row blocks of fewer m-tiles than the rows need (wider, shorter tiles)
    nat = 1 if M <= 16 else 2 if M <= 32 else 4 if M <= 64 else 8
    for (mt, NBt, S, NS, fl, red) in ((nat // 2, 4, 1, 3, 0, skg.REDUCE_NONE),
                                      (1, 4, 2, 2, wide, skg.REDUCE_KERNEL)):
        if mt < 1 or mt >= nat:
            continue
        p = skg.make_plan(skg.KIND_TILED, 256, NBt, S, NS, red, flags=fl, m_tiles=mt)
        try:
            skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
        except skg.SkinnyGemmError:
            continue
        plans.append((f"tiled_rows_mt{mt}_nb{NBt}_s{S}", p))
    return plans


def _run(skg, plan, xq, wq, bias, **sc):
    out = skg.gemm_fp8(xq, wq, bias=bias, **sc) if plan is None else \
        skg.gemm_fp8_planned(xq, wq, plan, bias=bias, **sc)
    torch.cuda.synchronize()
    return out.cpu()


def _oracle(mode, xq, wq, s1, s2, bias):
    b = None if bias is None else gen.bits16(bias)
    if mode == "fp8_tensor":
        return oracle.gemm_fp8_tensor(gen.bits8(xq), gen.bits8(wq), float(s1), float(s2), b,
                                      threads=16)
    return oracle.gemm_fp8_mx(gen.bits8(xq), gen.bits8(wq), gen.bits8(s1), gen.bits8(s2), b,
                              threads=16)


def _scales(mode, s1, s2):
    if mode == "fp8_tensor":
        return dict(sx=s1.to(DEV), sw=s2.to(DEV))
    return dict(xe=s1.to(DEV), we=s2.to(DEV))


FP8_POINTS = [p for p in configs.all_points() if p.dtype != "bf16"]


@pytest.mark.parametrize("p", FP8_POINTS, ids=lambda p: p.key())
@pytest.mark.parametrize("with_bias", (False, True))
def test_fp8_point_within_tolerance(skg, p, with_bias):
    xq, wq, s1, s2 = gen.point_inputs(p)
    bias = None
    if with_bias:
        bias = (torch.randn(p.N, generator=torch.Generator().manual_seed(p.M)) * 0.3).to(torch.bfloat16)
    ref = _oracle(p.dtype, xq, wq, s1, s2, bias)
    xd, wd = xq.to(DEV), wq.to(DEV)
    bd = None if bias is None else bias.to(DEV)
    for name, plan in _plans(skg, p.M, p.N, p.K):
        out = _run(skg, plan, xd, wd, bd, **_scales(p.dtype, s1, s2))
        ok, msg = tolerance.check(out, ref, p.K)
        assert ok, f"{p.key()} bias={with_bias} [{name}]: {msg}"


def _small_int_e4m3(rows, K, seed, lo=-2, hi=2):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (rows, K), generator=g).to(torch.float32).to(torch.float8_e4m3fn)


@pytest.mark.parametrize("M,N,K", [(1, 64, 4096), (5, 48, 4112), (16, 200, 2048), (37, 96, 1024),
                                   (128, 64, 4096), (2, 7, 4096), (4, 1, 1024)])
def test_fp8_per_tensor_integers_bitwise(skg, M, N, K):
    xq = _small_int_e4m3(M, K, M + K)
    wq = _small_int_e4m3(N, K, N + K + 1)
    one = torch.ones(1, dtype=torch.float32)
    bias = torch.randint(-3, 4, (N,), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    ref = _oracle("fp8_tensor", xq, wq, 1.0, 1.0, bias)
    for name, plan in _plans(skg, M, N, K):
        out = _run(skg, plan, xq.to(DEV), wq.to(DEV), bias.to(DEV), sx=one.to(DEV), sw=one.to(DEV))
        bad = np.argwhere(gen.bits16(out) != ref)
        assert bad.size == 0, f"[{name}] {len(bad)} mismatches, first {tuple(bad[0])}"


@pytest.mark.parametrize("M,N,K", [(1, 64, 4096), (9, 80, 2048), (64, 48, 1024), (128, 32, 4096),
                                   (3, 5, 2048)])
def test_fp8_mx_exact_scales_bitwise(skg, M, N, K):
    # exponents 126..128 on both sides: every scaled block sum and every
    # fp32 partial sum stays exact, so the result is unique
    xq = _small_int_e4m3(M, K, 3 * M + K)
    wq = _small_int_e4m3(N, K, 5 * N + K)
    g = torch.Generator().manual_seed(M * N)
    xe = torch.randint(126, 129, (M, K // 32), generator=g).to(torch.uint8)
    we = torch.randint(126, 129, (N, K // 32), generator=g).to(torch.uint8)
    ref = _oracle("fp8_mx", xq, wq, xe, we, None)
    for name, plan in _plans(skg, M, N, K):
        out = _run(skg, plan, xq.to(DEV), wq.to(DEV), None, xe=xe.to(DEV), we=we.to(DEV))
        bad = np.argwhere(gen.bits16(out) != ref)
        assert bad.size == 0, f"[{name}] {len(bad)} mismatches, first {tuple(bad[0])}"


# The bias with non-unit scales.  Per-tensor: out = bf16(sx * sw * sum + bias),
# the scale product applied once to the sum and the bias added after it
# ("sglang PR #28333" page: the key source snippet adds the bias to the
# GEMM's output; the motivation section: the scales are applied once).
# With e4m3 integers, sx = 2^-3, sw = 2^-2 and an integer bias every value
# is exact in fp32, so the output is unique; a bias added before the scale
# product (shrunk 32x) or dropped gives other bits in most elements, which
# each test checks on the oracle before it compares a plan.
POW2_SX, POW2_SW = 2.0 ** -3, 2.0 ** -2


def _int_bias(N, seed):
    return torch.randint(-3, 4, (N,), generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)


def _sees_bias(ref, wrong):
    return (ref != wrong).mean() > 0.5


@pytest.mark.parametrize("M,N,K", [(1, 64, 4096), (5, 48, 4112), (16, 200, 2048), (37, 96, 1024),
                                   (128, 64, 4096), (2, 7, 4096), (4, 1, 1024)])
def test_fp8_per_tensor_pow2_scales_bias_bitwise(skg, M, N, K):
    xq = _small_int_e4m3(M, K, 11 * M + K)
    wq = _small_int_e4m3(N, K, 13 * N + K)
    bias = _int_bias(N, M + N)
    ref = _oracle("fp8_tensor", xq, wq, POW2_SX, POW2_SW, bias)
    assert _sees_bias(ref, _oracle("fp8_tensor", xq, wq, POW2_SX, POW2_SW, None))
    shrunk = (bias.float() * (POW2_SX * POW2_SW)).to(torch.bfloat16)  # bias before the scales
    assert _sees_bias(ref, _oracle("fp8_tensor", xq, wq, POW2_SX, POW2_SW, shrunk))
    sx = torch.tensor([POW2_SX], dtype=torch.float32, device=DEV)
    sw = torch.tensor([POW2_SW], dtype=torch.float32, device=DEV)
    for name, plan in _plans(skg, M, N, K):
        out = _run(skg, plan, xq.to(DEV), wq.to(DEV), bias.to(DEV), sx=sx, sw=sw)
        bad = np.argwhere(gen.bits16(out) != ref)
        assert bad.size == 0, f"[{name}] {len(bad)} mismatches, first {tuple(bad[0])}"


@pytest.mark.parametrize("M,N,K", [(1, 64, 4096), (8, 80, 2048), (16, 48, 4096), (100, 40, 1024)])
def test_fp8_quant_pow2_scales_bias_bitwise(skg, M, N, K):
    # bf16 x = q * sx with small integers q: the static quantisation returns
    # exactly q, so the fused call must equal the integer reference bit for bit
    q = _small_int_e4m3(M, K, 17 * M + K)
    x = (q.float() * POW2_SX).to(torch.bfloat16)
    wq = _small_int_e4m3(N, K, 19 * N + K)
    bias = _int_bias(N, 2 * M + N)
    ref = _oracle("fp8_tensor", q, wq, POW2_SX, POW2_SW, bias)
    assert _sees_bias(ref, _oracle("fp8_tensor", q, wq, POW2_SX, POW2_SW, None))
    sx = torch.tensor([POW2_SX], dtype=torch.float32, device=DEV)
    sw = torch.tensor([POW2_SW], dtype=torch.float32, device=DEV)
    out = skg.gemm_fp8_quant(x.to(DEV), wq.to(DEV), sx, sw, bias=bias.to(DEV))
    torch.cuda.synchronize()
    bad = np.argwhere(gen.bits16(out.cpu()) != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first {tuple(bad[0])}"


@pytest.mark.parametrize("M,N,K", [(1, 64, 4096), (9, 80, 2048), (64, 48, 1024), (128, 32, 4096),
                                   (3, 5, 2048)])
def test_fp8_mx_exact_scales_bias_bitwise(skg, M, N, K):
    # MX: the bias is added once, after every block's scaled partial ("sglang
    # PR #34042" page: block scales inside the sum, the bias outside it)
    xq = _small_int_e4m3(M, K, 7 * M + K)
    wq = _small_int_e4m3(N, K, 3 * N + K)
    g = torch.Generator().manual_seed(M * N + 1)
    xe = torch.randint(126, 129, (M, K // 32), generator=g).to(torch.uint8)
    we = torch.randint(126, 129, (N, K // 32), generator=g).to(torch.uint8)
    bias = _int_bias(N, M * N + 2)
    ref = _oracle("fp8_mx", xq, wq, xe, we, bias)
    assert _sees_bias(ref, _oracle("fp8_mx", xq, wq, xe, we, None))
    for name, plan in _plans(skg, M, N, K):
        out = _run(skg, plan, xq.to(DEV), wq.to(DEV), bias.to(DEV), xe=xe.to(DEV), we=we.to(DEV))
        bad = np.argwhere(gen.bits16(out) != ref)
        assert bad.size == 0, f"[{name}] {len(bad)} mismatches, first {tuple(bad[0])}"


def test_fp8_mx_nan_exponent_propagates(skg):
    M, N, K = 4, 40, 1024
    xq, wq, xe, we = gen.fp8_inputs(M, N, K, "fp8_mx", seed=99)
    xe = xe.clone()
    xe[2, 5] = 0xFF          # row 2 of x, block 5: NaN scale
    we = we.clone()
    we[31, 0] = 0xFF         # column 31: NaN scale
    ref = tolerance.widen(_oracle("fp8_mx", xq, wq, xe, we, None))
    assert np.isnan(ref[2]).all() and np.isnan(ref[:, 31]).all()
    for name, plan in _plans(skg, M, N, K):
        out = tolerance.widen(_run(skg, plan, xq.to(DEV), wq.to(DEV), None, xe=xe.to(DEV), we=we.to(DEV)))
        assert np.array_equal(np.isnan(out), np.isnan(ref)), f"[{name}]"


def test_fp8_runs_bitwise_deterministic(skg):
    for mode in ("fp8_tensor", "fp8_mx"):
        xq, wq, s1, s2 = gen.fp8_inputs(16, 4096, 4096, mode, seed=5)
        xd, wd = xq.to(DEV), wq.to(DEV)
        for name, plan in _plans(skg, 16, 4096, 4096):
            a = _run(skg, plan, xd, wd, None, **_scales(mode, s1, s2))
            b = _run(skg, plan, xd, wd, None, **_scales(mode, s1, s2))
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{mode} [{name}]"


# FP8 shapes off the dispatch table, one or more per branch of the default
# rule at 256 CUs: the dot kernel (up to 2 rows, and 3-4 rows below a full
# grid of 8-column groups), the whole-row ring (3 to 32 rows from N = 512:
# 8 or 16 columns, full or half-width stages, 3 or 4 stages, any K per
# tensor, MX with K % 512 == 0), split-K without a K split (up to 16 rows,
# N >= 2048, ring refused), the tiled kernel and split-K for K % 128 != 0
# below N = 512
FP8_DEFAULT_RULE_SHAPES = [
    ((2, 1024, 1024, "fp8_tensor"), "dot"), ((4, 1024, 1024, "fp8_tensor"), "dot"),
    ((8, 512, 1024, "fp8_tensor"), "rows"), ((24, 4096, 1040, "fp8_tensor"), "rows"),
    ((4, 7168, 1024, "fp8_mx"), "rows"), ((6, 5120, 1024, "fp8_tensor"), "rows"),
    ((32, 4096, 1024, "fp8_mx"), "rows"), ((16, 2048, 1056, "fp8_mx"), "splitk"),
    ((12, 256, 2048, "fp8_tensor"), "tiled"), ((24, 256, 1024, "fp8_tensor"), "tiled"),
    ((24, 256, 1040, "fp8_tensor"), "splitk")]


@pytest.mark.parametrize("shape,kind", FP8_DEFAULT_RULE_SHAPES, ids=str)
def test_fp8_default_rule_plans_within_tolerance(skg, shape, kind):
    M, N, K, mode = shape
    dt = skg.DTYPE_FP8 if mode == "fp8_tensor" else skg.DTYPE_FP8_MX
    q = skg.plan(M, N, K, dt)
    assert q.from_table == 0
    want = {"dot": skg.KIND_DOT, "rows": skg.KIND_ROWS, "splitk": skg.KIND_SPLITK,
            "tiled": skg.KIND_TILED}[kind]
    assert q.kind == want, q
    if want == skg.KIND_SPLITK and M <= 16:
        assert q.splits == 1
    xq, wq, s1, s2 = gen.fp8_inputs(M, N, K, mode, seed=M + N + K)
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(K)) * 0.5).to(torch.bfloat16)
    ref = _oracle(mode, xq, wq, s1, s2, bias)
    out = _run(skg, None, xq.to(DEV), wq.to(DEV), bias.to(DEV), **_scales(mode, s1, s2))
    ok, msg = tolerance.check(out, ref, K)
    assert ok, f"{shape} plan {q}: {msg}"


@pytest.mark.parametrize("mode", ("fp8_tensor", "fp8_mx"))
def test_fp8_reductions_agree_bitwise(skg, mode):
    # last-arriver and second-kernel sums of the FP8 split-K and tiled
    # kernels add the same partials in the same order (and apply the
    # per-tensor scale product once, after the sum); N % 4 == 0 takes the
    # 16-byte coherent partials, N = 130 the per-float ones
    for (M, N, K) in ((16, 4096, 4096), (64, 1024, 2048), (7, 130, 2048), (128, 512, 4096)):
        xq, wq, s1, s2 = gen.fp8_inputs(M, N, K, mode, seed=M + N)
        xd, wd = xq.to(DEV), wq.to(DEV)
        bias = (torch.randn(N, generator=torch.Generator().manual_seed(N)) * 0.5).to(torch.bfloat16).to(DEV)
        dt = skg.DTYPE_FP8 if mode == "fp8_tensor" else skg.DTYPE_FP8_MX
        for kind, T, cols, S, D, fl in ((skg.KIND_SPLITK, 256, 1, 4, 2, 0),
                                        (skg.KIND_TILED, 256, 2, 4, 3, 0),
                                        (skg.KIND_TILED, 256, 4, 2, 3, skg.FLAG_TILED_WIDE)):
            outs = []
            for red in (skg.REDUCE_LAST, skg.REDUCE_KERNEL):
                try:
                    plan = skg.plan_complete(M, N, K, skg.make_plan(kind, T, cols, S, D, red, flags=fl), dt)
                except skg.SkinnyGemmError:
                    break
                outs.append(_run(skg, plan, xd, wd, bias, **_scales(mode, s1, s2)))
            if len(outs) == 2:
                assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), \
                    (mode, M, N, K, kind, S)
