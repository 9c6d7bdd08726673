"""skinny_gemm_bf16_noalloc: the allocation-free form of skinny_gemm_bf16.

Called through the C ABI and compared bit for bit with skinny_gemm_bf16 on
the same inputs (the same plans and kernels, with the partials in the
library's fixed per-GPU array), two calls in a row with the second smaller,
plus the oracle's tolerance, the over-size rejection and a captured graph
on a stream that never reserved a workspace.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from oracle import tolerance
from workloads import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH_FLOATS = 1 << 21


@pytest.fixture(scope="module")
def skg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import latency_skinny_gemm_amd as m
    m.lib()
    return m


def _inputs(M, N, K, bias, seed):
    x, w, b = gen.bf16_inputs(M, N, K, bias, seed=seed)
    return x.to(DEV), w.to(DEV), (b.to(DEV) if bias else None), (x, w, b)


def _call(skg, fn, x, w, b, out, M, N, K, stream):
    return fn(x.data_ptr(), w.data_ptr(), None if b is None else b.data_ptr(), None,
              out.data_ptr(), M, N, K, ctypes.c_void_p(stream.cuda_stream))


def _pair(skg, M, N, K, bias, seed, stream):
    """(noalloc output, skinny_gemm_bf16 output, host inputs)."""
    x, w, b, host = _inputs(M, N, K, bias, seed)
    a = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    r = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    L = skg.lib()
    with torch.cuda.stream(stream):
        assert _call(skg, L.skinny_gemm_bf16_noalloc, x, w, b, a, M, N, K, stream) == 0
    stream.synchronize()
    with torch.cuda.stream(stream):
        assert _call(skg, L.skinny_gemm_bf16, x, w, b, r, M, N, K, stream) == 0
    stream.synchronize()
    return a.cpu(), r.cpu(), host


# the first call fills the whole array (S * M * N = 2^21 floats), the second
# is smaller; then a split-K plan whose last-arriver reduction is switched to
# the second kernel, then a plan with no partials (dot kernel)
SEQUENCES = [
    [(128, 4096, 7168, False), (8, 2112, 7168, True)],
    [(20, 700, 2056, True), (8, 1000, 2056, False)],
    [(10, 384, 7168, False), (3, 256, 2880, True)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "_then_".join(f"{m}x{n}x{k}" for m, n, k, _ in s))
def test_noalloc_matches_skinny_gemm_bf16_bitwise(skg, seq):
    stream = torch.cuda.Stream()
    for i, (M, N, K, bias) in enumerate(seq):
        p = skg.plan(M, N, K)
        assert p.splits * M * N <= SCRATCH_FLOATS
        a, r, (x, w, b) = _pair(skg, M, N, K, bias, 1000 * i + M + N + K, stream)
        assert torch.equal(a.view(torch.int16), r.view(torch.int16)), (M, N, K, p)
        if M * N * K <= 128 * 4096 * 7168 // 8:
            ref = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w),
                                   None if b is None else gen.bits16(b), threads=16)
            ok, msg = tolerance.check(a, ref, K)
            assert ok, f"{(M, N, K)}: {msg}"
        else:  # full decode size: sampled outputs
            rows, cols = [0, M // 2, M - 1], list(range(0, N, N // 31))[:32] + [N - 1]
            ref = oracle.gemm_bf16(gen.bits16(x[rows]), gen.bits16(w[cols]),
                                   None if b is None else gen.bits16(b[cols]), threads=16)
            ok, msg = tolerance.check(a[rows][:, cols], ref, K)
            assert ok, f"{(M, N, K)} sampled: {msg}"


def test_noalloc_rejects_partials_beyond_the_array(skg):
    M, N, K = 512, 4096, 7168
    p = skg.plan(M, N, K)
    assert p.splits > 1 and p.splits * M * N > SCRATCH_FLOATS
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((N, K), dtype=torch.bfloat16, device=DEV)
    out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.Stream()
    rc = _call(skg, skg.lib().skinny_gemm_bf16_noalloc, x, w, None, out, M, N, K, stream)
    stream.synchronize()
    assert rc == skg.ERR_WORKSPACE
    assert bool((out == 7.0).all())  # nothing was launched


def test_noalloc_in_a_graph_without_reserve(skg):
    # a fresh stream with no workspace: skinny_gemm_bf16 could not be
    # captured here (it would need to allocate); the no-allocation form can
    M, N, K = 8, 1000, 2056
    x, w, b, host = _inputs(M, N, K, True, 77)
    out = torch.zeros((M, N), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):  # a device's first call looks up its array
        assert _call(skg, skg.lib().skinny_gemm_bf16_noalloc, x, w, b, out, M, N, K, stream) == 0
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        rc = _call(skg, skg.lib().skinny_gemm_bf16_noalloc, x, w, b, out, M, N, K, stream)
    assert rc == 0
    ref = oracle.gemm_bf16(gen.bits16(host[0]), gen.bits16(host[1]), gen.bits16(host[2]), threads=16)
    first = None
    for rep in range(4):
        out.zero_()  # eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        got = out.cpu()
        ok, msg = tolerance.check(got, ref, K)
        assert ok, f"replay {rep}: {msg}"
        if first is None:
            first = got
        assert torch.equal(got.view(torch.int16), first.view(torch.int16)), f"replay {rep}"
    del g
