"""GPU parity of the fp32-output GEMM and of the FP8 GEMM that quantises bf16
activations statically (q = e4m3(clamp(x * (1/sx), -448, 448))), through the
C ABI, against the CPU oracle.

- The quantiser must give the oracle's codes bit for bit (every bf16 code,
  several scales): the codes are integers decided in fp32 on both sides.
- fp32 outputs must lie within the rigorous bound of an fp32 summation in
  any order, (K + 3) * 2^-24 * sum_k |x_k w_k| (+ |bias|), plus half an fp32
  ulp for the oracle's own rounding; small-integer inputs must match exactly.
- A bf16 output must be the bf16 rounding of the fp32 output of the same
  plan (the two differ only in the final store).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import tolerance
from workloads import inputs as gen

from tests.test_parity_gpu import _kernel_plans

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -24


@pytest.fixture(scope="module")
def skg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import latency_skinny_gemm_amd as m
    m.lib()
    return m


def _f32(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def _decode_bf16(codes):
    with np.errstate(invalid="ignore"):
        return (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _decode_e4m3(codes):
    table = np.array([oracle.decode_e4m3(c) for c in range(256)])
    return table[codes]


# ------------------------------------------------------------- quantiser

@pytest.mark.parametrize("s", [1.0, 0.037, 3.5, 2.0 ** -4, 1e-3, 448.0 / 7.25, 0.9926469922065735])
def test_quant_every_bf16_code_bitwise(skg, s):
    codes = np.arange(65536, dtype=np.uint16)
    x = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(DEV)
    q = skg.quant_e4m3(x, _f32(s))
    torch.cuda.synchronize()
    got = gen.bits8(q.cpu())
    ref = oracle.quant_e4m3(codes, s)
    nan = np.isnan(_decode_bf16(codes))
    bad = np.nonzero((got != ref) & ~nan)[0]
    assert bad.size == 0, f"s={s}: {bad.size} codes differ, first bf16 0x{codes[bad[0]]:04x}: " \
                          f"gpu 0x{got[bad[0]]:02x} oracle 0x{ref[bad[0]]:02x}"
    assert np.all((got[nan] & 0x7F) == 0x7F)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 111, 4096 + 9])
def test_quant_lengths_and_tail(skg, n):
    g = torch.Generator().manual_seed(n)
    x = (torch.randn(n, generator=g) * 3).to(torch.bfloat16)
    q = skg.quant_e4m3(x.to(DEV), _f32(0.02))
    torch.cuda.synchronize()
    assert np.array_equal(gen.bits8(q.cpu()), oracle.quant_e4m3(gen.bits16(x), 0.02))


# ------------------------------------------------------------- fp32 output

def _fp32_bound(x16, w16, b16, K):
    ax = np.abs(_decode_bf16(x16))
    aw = np.abs(_decode_bf16(w16))
    mag = ax @ aw.T
    if b16 is not None:
        mag = mag + np.abs(_decode_bf16(b16))[None, :]
    return (K + 3) * U * mag


F32_POINTS = [(1, 256, 7168, False), (5, 256, 7168, True), (16, 384, 7168, False),
              (9, 256, 2880, True), (64, 576, 7168, True), (128, 2112, 7168, False),
              (37, 100, 1024, True)]


@pytest.mark.parametrize("M,N,K,bias", F32_POINTS)
def test_f32_output_within_fp32_bound(skg, M, N, K, bias):
    x, w, b = gen.bf16_inputs(M, N, K, bias, seed=M * 7 + N + K)
    x16, w16 = gen.bits16(x), gen.bits16(w)
    b16 = None if b is None else gen.bits16(b)
    ref = oracle.gemm_bf16(x16, w16, b16, out_f32=True, threads=16).astype(np.float64)
    bound = _fp32_bound(x16, w16, b16, K) + U * np.abs(ref)
    xd, wd = x.to(DEV), w.to(DEV)
    bd = None if b is None else b.to(DEV)
    for name, plan in _kernel_plans(skg, M, N, K):
        if plan is not None:
            try:
                skg.plan_complete(M, N, K, plan)
            except skg.SkinnyGemmError:
                continue
        out = skg.gemm_bf16_f32(xd, wd, bd, plan=plan)
        o16 = skg.gemm_bf16(xd, wd, bd) if plan is None else skg.gemm_bf16_planned(xd, wd, plan, bd)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), f"[{name}] {worst}: |{got[worst]} - {ref[worst]}| > {bound[worst]}"
        # the bf16 output of the same plan is the RNE of this fp32 output
        assert torch.equal(out.cpu().to(torch.bfloat16).view(torch.int16),
                           o16.cpu().view(torch.int16)), f"[{name}] bf16 != bf16(fp32)"


@pytest.mark.parametrize("M,N,K", [(1, 64, 7168), (7, 200, 2880), (16, 256, 7168), (100, 96, 1024)])
def test_f32_output_small_integers_exact(skg, M, N, K):
    x, w, b = gen.small_integers(M, N, K, True, seed=M + N)
    ref = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b), out_f32=True, threads=16)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    for name, plan in _kernel_plans(skg, M, N, K):
        if plan is not None:
            try:
                skg.plan_complete(M, N, K, plan)
            except skg.SkinnyGemmError:
                continue
        out = skg.gemm_bf16_f32(xd, wd, bd, plan=plan)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref), f"[{name}]"


# ------------------------------------------------------------- fused quant

def _quant_plans(skg, M, N, K):
    plans = [("default", None)]
    if M <= 16:
        for T, C in ((64, 1), (256, 1), (512, 1), (1024, 1), (256, 2), (256, 4)):
            p = skg.make_plan(skg.KIND_DOT, T, C)
            try:
                skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
            except skg.SkinnyGemmError:
                continue
            plans.append((f"dot_t{T}_c{C}", p))
    mt = (M + 15) // 16
    for (T, NB, S, D, red) in ((256, 1, 4, 1, skg.REDUCE_KERNEL), (256, 2 if mt <= 3 else 1, 1, 1,
                                                                   skg.REDUCE_NONE),
                               (256, 1, 3, 2, skg.REDUCE_LAST), (128, 4, 2, 1, skg.REDUCE_KERNEL)):
        p = skg.make_plan(skg.KIND_SPLITK, T, NB, S, D, red)
        try:
            skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
        except skg.SkinnyGemmError:
            continue
        plans.append((f"mfma_t{T}_nb{NB}_s{S}_d{D}_r{red}", p))
    p = skg.make_plan(skg.KIND_TILED, 256, 4, 2, 3, skg.REDUCE_KERNEL)
    try:
        skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
        plans.append(("tiled_s2", p))
    except skg.SkinnyGemmError:
        pass
    # whole-row ring, quantising x from LDS (where its bf16 stages fit)
    for (T, R, NS, fl) in ((256, 16, 4, skg.FLAG_ROWS_HALF), (256, 8, 4, 0), (512, 16, 3, 0)):
        p = skg.make_plan(skg.KIND_ROWS, T, R, depth=NS, flags=fl)
        try:
            skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
        except skg.SkinnyGemmError:
            continue
        plans.append((f"rows_t{T}_c{R}_ns{NS}_f{fl}", p))
    return plans


def _x_wide_range(M, K, seed):
    """bf16 x whose quantised values cover e4m3 subnormals, normals and the
    clamp at 448 with sx = 0.01."""
    g = torch.Generator().manual_seed(seed)
    mag = torch.exp2(torch.randint(-22, 4, (M, K), generator=g).float())
    return (torch.randn(M, K, generator=g) * mag).to(torch.bfloat16)


@pytest.mark.parametrize("M", [1, 3, 8, 16, 24, 64])
def test_fused_quant_codes_through_one_hot_W(skg, M):
    # W[n, k] = 1.0 exactly when k = perm(n): out[m, n] = sx * q[m, perm(n)]
    # in fp32, one product of exact values: equal to the oracle bit for bit
    N, K, sx = 512, 1024, 0.01
    x = _x_wide_range(M, K, seed=M)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(3))[:N]
    w = torch.zeros(N, K)
    w[torch.arange(N), perm] = 1.0
    wq = w.to(torch.float8_e4m3fn)
    ref = oracle.gemm_fp8_quant(gen.bits16(x), gen.bits8(wq), sx, 1.0, out_f32=True, threads=16)
    xd, wd = x.to(DEV), wq.to(DEV)
    for name, plan in _quant_plans(skg, M, N, K):
        out = skg.gemm_fp8_quant(xd, wd, _f32(sx), _f32(1.0), out_dtype=torch.float32, plan=plan)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        bad = np.argwhere(got.view(np.uint32) != ref.view(np.uint32))
        assert bad.size == 0, f"[{name}] {len(bad)} differ, first {tuple(bad[0])}: " \
                              f"{got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"


@pytest.mark.parametrize("M", [1, 5, 16, 64])
def test_fused_quant_equals_quant_then_gemm(skg, M):
    N, K = 1024, 4096
    x = (torch.randn(M, K, generator=torch.Generator().manual_seed(M)) * 2).to(torch.bfloat16)
    _, wq, _, sw = gen.fp8_inputs(M, N, K, "fp8_tensor", seed=11)
    xd, wd = x.to(DEV), wq.to(DEV)
    sxd, swd = _f32(0.013), sw.to(DEV)
    for name, plan in _quant_plans(skg, M, N, K):
        fused = skg.gemm_fp8_quant(xd, wd, sxd, swd, plan=plan)
        xq = skg.quant_e4m3(xd, sxd)
        two = skg.gemm_fp8(xq, wd, sx=sxd, sw=swd) if plan is None else \
            skg.gemm_fp8_planned(xq, wd, plan, sx=sxd, sw=swd)
        torch.cuda.synchronize()
        assert torch.equal(fused.cpu().view(torch.int16), two.cpu().view(torch.int16)), f"[{name}]"


@pytest.mark.parametrize("M,N", [(1, 1021), (3, 6), (5, 1)])
def test_fused_quant_ragged_columns(skg, M, N):
    # several columns per workgroup with N not a multiple of them: the last
    # workgroup's missing columns read zeros and store nothing
    K = 2048
    x = (torch.randn(M, K, generator=torch.Generator().manual_seed(N)) * 3).to(torch.bfloat16)
    _, wq, _, sw = gen.fp8_inputs(M, N, K, "fp8_tensor", seed=N + 1)
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(2)) * 0.3).to(torch.bfloat16)
    xd, wd, bd = x.to(DEV), wq.to(DEV), bias.to(DEV)
    sxd, swd = _f32(0.02), sw.to(DEV)
    for C in (2, 4):
        plan = skg.make_plan(skg.KIND_DOT, 256, C)
        out = torch.full((M + 2, N), -5.0, dtype=torch.bfloat16, device=DEV)
        fused = skg.gemm_fp8_quant(xd, wd, sxd, swd, bias=bd, plan=plan, out=out[1:M + 1])
        xq = skg.quant_e4m3(xd, sxd)
        two = skg.gemm_fp8_planned(xq, wd, skg.make_plan(skg.KIND_DOT, 256, 1), sx=sxd, sw=swd, bias=bd)
        torch.cuda.synchronize()
        host = out.cpu()
        assert torch.all(host[0] == -5.0) and torch.all(host[M + 1] == -5.0), f"C={C}: guard rows"
        assert torch.equal(fused.cpu().view(torch.int16), two.cpu().view(torch.int16)), f"C={C}"


@pytest.mark.parametrize("M,bias", [(1, False), (16, True), (64, False), (128, True)])
def test_fused_quant_points_within_tolerance(skg, M, bias):
    N = K = 4096
    x = (torch.randn(M, K, generator=torch.Generator().manual_seed(100 + M))).to(torch.bfloat16)
    _, wq, _, sw = gen.fp8_inputs(M, N, K, "fp8_tensor", seed=12)
    sx = float(x.float().abs().max()) / 448.0
    b = (torch.randn(N, generator=torch.Generator().manual_seed(7)) * 0.3).to(torch.bfloat16) \
        if bias else None
    ref = oracle.gemm_fp8_quant(gen.bits16(x), gen.bits8(wq), sx, float(sw), None if b is None
                                else gen.bits16(b), threads=16)
    bd = None if b is None else b.to(DEV)
    out = skg.gemm_fp8_quant(x.to(DEV), wq.to(DEV), _f32(sx), sw.to(DEV), bias=bd)
    torch.cuda.synchronize()
    ok, msg = tolerance.check(out.cpu(), ref, K)
    assert ok, msg


def test_fused_quant_nan_row(skg):
    M, N, K = 4, 64, 1024
    x = torch.randn(M, K, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    x[2, 17] = float("nan")
    _, wq, _, sw = gen.fp8_inputs(M, N, K, "fp8_tensor", seed=2)
    ref = tolerance.widen(oracle.gemm_fp8_quant(gen.bits16(x), gen.bits8(wq), 0.01, float(sw)))
    for name, plan in _quant_plans(skg, M, N, K):
        out = skg.gemm_fp8_quant(x.to(DEV), wq.to(DEV), _f32(0.01), sw.to(DEV), plan=plan)
        torch.cuda.synchronize()
        got = tolerance.widen(out.cpu())
        assert np.array_equal(np.isnan(got), np.isnan(ref)), f"[{name}]"


def test_capture_after_reserve_with_quantised_x_in_workspace(skg):
    # A tiled plan quantises x into the workspace before the GEMM, after the
    # split partials (rounded up to 64 floats); with S*M*N = 3000 the
    # rounding matters.  reserve(M, N, K, S) must cover both requests, and
    # the plain FP8 call with the same plan (partials only, unrounded), so
    # that both can be captured with no eager call first.
    import ctypes

    M, N, K, S = 5, 300, 4096, 2
    x = (torch.randn(M, K, generator=torch.Generator().manual_seed(5)) * 2).to(torch.bfloat16)
    _, wq, _, sw = gen.fp8_inputs(M, N, K, "fp8_tensor", seed=6)
    xd, wd = x.to(DEV), wq.to(DEV)
    sxd, swd = _f32(0.013), sw.to(DEV)
    xq = skg.quant_e4m3(xd, sxd)
    plan = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_TILED, 256, 4, S, 3,
                                                    skg.REDUCE_KERNEL), skg.DTYPE_FP8)
    sc = skg.Fp8Scales()
    sc.mode, sc.sx, sc.sw = skg.FP8_PER_TENSOR, sxd.data_ptr(), swd.data_ptr()
    lib = skg.lib()
    torch.cuda.synchronize()
    skg.release_all()
    stream = torch.cuda.Stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    out_q = torch.zeros(M, N, dtype=torch.bfloat16, device=DEV)
    out_p = torch.zeros(M, N, dtype=torch.bfloat16, device=DEV)

    def calls():
        rq = lib.skinny_gemm_fp8_quant_planned(xd.data_ptr(), wd.data_ptr(), None, sxd.data_ptr(),
                                               swd.data_ptr(), out_q.data_ptr(), skg.DTYPE_BF16,
                                               M, N, K, ctypes.byref(plan), sptr)
        rp = lib.skinny_gemm_fp8_planned(xq.data_ptr(), wd.data_ptr(), None, ctypes.byref(sc),
                                         out_p.data_ptr(), M, N, K, ctypes.byref(plan), sptr)
        return rq, rp
    with torch.cuda.stream(stream):
        skg.reserve(M, N, K, S)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        rcs = calls()
    assert rcs == (skg.OK, skg.OK), rcs
    with torch.cuda.stream(stream):
        assert calls() == (skg.OK, skg.OK)
    torch.cuda.synchronize()
    eager_q, eager_p = out_q.clone(), out_p.clone()
    # the fused quantisation and the quantise-then-GEMM path agree bit for bit
    assert torch.equal(eager_q.view(torch.int16), eager_p.view(torch.int16))
    for _ in range(3):
        out_q.fill_(0)
        out_p.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_q.view(torch.int16), eager_q.view(torch.int16))
        assert torch.equal(out_p.view(torch.int16), eager_p.view(torch.int16))
    del g
    skg.release_all()
