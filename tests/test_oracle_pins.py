"""Pins for the CPU oracle: results the mathematics fixes, reached by a route
other than the oracle's own code (closed forms, exact rational arithmetic,
torch's decoders, brute force).  CPU only.

Passage followed by the oracle: "sglang PR #30117" page, key source snippet
(out = x @ weight.T + bias, bf16 in/out, fp32 accumulation).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact
from workloads import inputs as gen

KS = (2048, 2880, 4096, 6144, 7168)


# ------------------------------------------------------------------ decoders

def test_decode_bf16_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_decode_e4m3_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.decode_e4m3(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # the format's landmarks, from its bit-field definition
    assert oracle.decode_e4m3(0x7E) == 448.0
    assert oracle.decode_e4m3(0x01) == 2.0 ** -9
    assert oracle.decode_e4m3(0x08) == 2.0 ** -6
    assert math.isnan(oracle.decode_e4m3(0x7F)) and math.isnan(oracle.decode_e4m3(0xFF))
    for c in range(256):
        e = exact.e4m3_code_to_fraction(c)
        g = oracle.decode_e4m3(c)
        assert exact.same(e if isinstance(e, float) else e, g if math.isnan(g) else Fraction(g))


def test_decode_e8m0_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.decode_e8m0(c) for c in codes])
    assert math.isnan(got[255]) and math.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert oracle.decode_e8m0(127) == 1.0 and oracle.decode_e8m0(0) == 2.0 ** -127


# ------------------------------------------------------------------ rounding

def _exact_bf16(v: float):
    return exact.round_fraction(Fraction(v), **exact.BF16)


def _check_round(v):
    code = oracle.round_bf16(v)
    got = exact.bf16_code_to_fraction(code)
    want = _exact_bf16(v)
    assert exact.same(got, want), (v, hex(code), want)
    if v == 0:
        assert (code & 0x8000) == (0x8000 if math.copysign(1, v) < 0 else 0)


def test_round_bf16_double_rounding_case():
    # 1 + 2^-8 + 2^-40 lies above the tie 1 + 2^-8: nearest bf16 is 1 + 2^-7.
    assert oracle.round_bf16(1 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    # the tie itself goes to even (1.0)
    assert oracle.round_bf16(1 + 2.0 ** -8) == 0x3F80
    assert oracle.round_bf16(1 + 3 * 2.0 ** -8) == 0x3F82


def test_round_bf16_against_exact_fractions():
    rng = np.random.default_rng(1234)
    vals = []
    # random magnitudes over the whole range, both signs
    for e in range(-140, 129, 3):
        for _ in range(6):
            vals.append(float(rng.uniform(1, 2)) * 2.0 ** e * (1 if rng.random() < .5 else -1))
    # exact ties and near-ties in several binades, incl. the subnormal range
    for e in (-133, -130, -127, -126, -100, -8, 0, 7, 100, 126, 127):
        q = 2.0 ** (max(e, -126) - 7)
        for k in (1, 2, 3, 255):
            base = k * q if e <= -126 else (2.0 ** e) + k * q
            vals += [base + q / 2, base - q / 2, base + q / 2 + q / 64, base + q / 2 - q / 64]
    # overflow boundary: max finite, the midpoint to 2^128 and just below it
    mf = (2 - 2.0 ** -7) * 2.0 ** 127
    vals += [mf, mf + 2.0 ** 119, mf + 2.0 ** 119 - 2.0 ** 100, 2.0 ** 128, -mf - 2.0 ** 119]
    vals += [0.0, -0.0, 2.0 ** -134, 2.0 ** -134 * 1.0000001, 2.0 ** -135, 3 * 2.0 ** -134]
    for v in vals:
        _check_round(v)


def test_round_bf16_matches_torch_for_fp32_values():
    # torch's fp32 -> bf16 conversion is a single RNE; for values that are
    # exactly binary32 the oracle's fp64 -> bf16 rounding must agree with it.
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_bf16(float(v)) for v in f[:50000]], dtype=np.uint16)
    assert np.array_equal(got, ref[:50000])


def test_round_nan_inf():
    assert oracle.round_bf16(float("inf")) == 0x7F80
    assert oracle.round_bf16(float("-inf")) == 0xFF80
    c = oracle.round_bf16(float("nan"))
    assert (c & 0x7F80) == 0x7F80 and (c & 0x7F) != 0


# ------------------------------------------------------------------ GEMM pins

def _decode(out16):
    return torch.from_numpy(out16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("K", KS)
def test_all_ones_gives_K(K):
    x, w = gen.ones(3, 5, K)
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w))
    assert np.all(_decode(out) == K)  # every configured K is exact in bf16


@pytest.mark.parametrize("K", KS)
def test_all_ones_plus_bias_rounds_back_to_K(K):
    # K + 1 lies strictly below the midpoint between K and the next bf16
    # (spacing 16 in [2048, 4096), 32 in [4096, 8192)): rounds back to K.
    x, w = gen.ones(2, 3, K)
    bias = torch.ones(3, dtype=torch.bfloat16)
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(bias))
    assert np.all(_decode(out) == K)
    # bias = 8 in [2048,4096) (half the spacing 16) is a tie: K is even -> K,
    # while bias = 24 lands at 1.5 spacings -> K + 32 (tie to even 2*16).
    if K < 4096:
        for b, want in ((8.0, K if (K // 16) % 2 == 0 else K + 16), (24.0, K + 32)):
            out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w),
                                   gen.bits16(torch.full((3,), b, dtype=torch.bfloat16)))
            assert np.all(_decode(out) == want), (K, b)


@pytest.mark.parametrize("K", (8, 2880, 7168))
def test_sign_alternating_gives_zero(K):
    x, w = gen.alternating(2, 4, K)
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w))
    assert np.all(_decode(out) == 0.0)


@pytest.mark.parametrize("K,N", ((2880, 128), (2048, 256), (64, 48)))
def test_one_hot_selects_x(K, N):
    x, w, pi = gen.one_hot(4, N, K, seed=11)
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w))
    xb = gen.bits16(x)
    assert np.array_equal(out, xb[:, pi.numpy()])
    # with bias: RNE(x + b), computed exactly
    b = (torch.randn(N, generator=torch.Generator().manual_seed(5)) * 0.3).to(torch.bfloat16)
    outb = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b))
    bb = gen.bits16(b)
    for m in range(4):
        for n in range(N):
            want = exact.round_fraction(exact.bf16_code_to_fraction(xb[m, pi[n]])
                                        + exact.bf16_code_to_fraction(bb[n]), **exact.BF16)
            assert exact.bf16_code_to_fraction(outb[m, n]) == want


@pytest.mark.parametrize("M,N,K,bias", ((5, 7, 2880, True), (16, 9, 7168, False), (3, 4, 8, True)))
def test_small_integer_regime_exact(M, N, K, bias):
    x, w, b = gen.small_integers(M, N, K, bias, seed=M * 1000 + K)
    xi = x.to(torch.int64).numpy()
    wi = w.to(torch.int64).numpy()
    acc = xi @ wi.T
    if bias:
        acc = acc + b.to(torch.int64).numpy()[None, :]
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), None if b is None else gen.bits16(b))
    for m in range(M):
        for n in range(N):
            want = exact.round_fraction(Fraction(int(acc[m, n])), **exact.BF16)
            assert exact.bf16_code_to_fraction(out[m, n]) == want


def test_brute_force_tiny():
    x, w = gen.brute_force_set()
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w))
    xb, wb = gen.bits16(x), gen.bits16(w)
    # The oracle accumulates in fp64.  Its result must be the exactly
    # rounded one wherever fp64 summation cannot move the sum across a bf16
    # rounding boundary; inside that error bound either neighbour is right.
    near_tie = 0
    for r in range(x.shape[0]):
        a = [exact.bf16_code_to_fraction(c) for c in xb[r]]
        for c in range(w.shape[0]):
            prods = [ai * exact.bf16_code_to_fraction(bj) for ai, bj in zip(a, wb[c])]
            s = sum(prods, Fraction(0))
            want = exact.round_fraction(s, **exact.BF16)
            got = exact.bf16_code_to_fraction(out[r, c])
            lo, hi = exact.round_range(s, exact.fp64_sum_bound(prods), exact.BF16)
            if lo == hi:
                assert exact.same(got, want), (r, c, s, hex(out[r, c]))
            else:
                near_tie += 1
                assert lo <= got <= hi, (r, c, s, hex(out[r, c]))
    # Only a product exactly on a bf16 tie plus a product below fp64's reach
    # (e.g. 1.5 * (1 + 2^-7) + 2^-133 * 2^-133) is ambiguous: 140 of the
    # 20736 combinations of this set; every other one is checked exactly.
    assert near_tie <= x.shape[0] * w.shape[0] // 100, near_tie


def test_numpy_fp64_cross_check():
    M, N, K = 8, 64, 2880
    x, w, b = gen.bf16_inputs(M, N, K, True, seed=99)
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b))
    ref = x.double().numpy() @ w.double().numpy().T + b.double().numpy()[None, :]
    got = _decode(out)
    # one bf16 rounding of nearly the same fp64 value: within half an ulp
    # (at most 2^-8 of the value) plus the fp64 summation-order noise.
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-12)
    # the roundings agree except at (practically never met) near-ties
    again = np.array([[oracle.round_bf16(v) for v in row] for row in ref], dtype=np.uint16)
    assert (again != out).sum() <= 1


def test_thread_count_does_not_change_bits():
    x, w, b = gen.bf16_inputs(7, 96, 2048, True, seed=3)
    a = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b), threads=1)
    c = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b), threads=8)
    assert np.array_equal(a, c)


def test_transposed_operand_would_be_seen():
    # x[M,K] and W[N,K] differ in role: out[m, n] uses row m of x and row n
    # of W.  A one-hot x picks columns of W: out[m, n] = W[n, m].
    K, N, M = 16, 5, 4
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    x[torch.arange(M), torch.arange(M)] = 1.0
    w = torch.arange(N * K, dtype=torch.float32).reshape(N, K).to(torch.bfloat16)
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w))
    assert np.array_equal(_decode(out), w.double().numpy()[:, :M].T)


def test_empty_K_is_bias_only():
    x = torch.zeros(2, 0, dtype=torch.bfloat16)
    w = torch.zeros(3, 0, dtype=torch.bfloat16)
    b = torch.tensor([1.5, -2.0, 0.25], dtype=torch.bfloat16)
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b))
    assert np.array_equal(_decode(out), np.tile([1.5, -2.0, 0.25], (2, 1)))


def test_fp32_output_rounds_once_from_exact():
    M, N, K = 4, 6, 64
    x, w, _ = gen.bf16_inputs(M, N, K, False, seed=21)
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), out_f32=True)
    xb, wb = gen.bits16(x), gen.bits16(w)
    for m in range(M):
        for n in range(N):
            s = sum((exact.bf16_code_to_fraction(xb[m, k]) * exact.bf16_code_to_fraction(wb[n, k])
                     for k in range(K)), Fraction(0))
            assert exact.f32_to_fraction(out[m, n]) == exact.round_fraction(s, **exact.F32)


def test_nan_and_inf_propagate():
    x = torch.ones(2, 8, dtype=torch.bfloat16)
    w = torch.ones(3, 8, dtype=torch.bfloat16)
    x[0, 3] = float("nan")
    w[2, 0] = float("inf")
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w))
    d = _decode(out)
    assert np.all(np.isnan(d[0]))
    assert d[1, 2] == math.inf and d[1, 0] == 8.0


# ------------------------------------------------------------------ FP8 pins

def _e4m3_int(q):
    """e4m3 bytes -> exact integers in units of 2^-9 (every e4m3 value is a
    multiple of the smallest subnormal 2^-9)."""
    return np.array([[int(exact.e4m3_code_to_fraction(c) * 512) for c in row] for row in q],
                    dtype=np.int64)


def test_fp8_per_tensor_exact():
    M, N, K = 3, 5, 256
    xq, wq, sx, sw = gen.fp8_inputs(M, N, K, "fp8_tensor", seed=17)
    xb, wb = gen.bits8(xq), gen.bits8(wq)
    acc = _e4m3_int(xb) @ _e4m3_int(wb).T   # exact, units of 2^-18
    for scales in ((1.0, 1.0), (float(sx), float(sw))):
        out = oracle.gemm_fp8_tensor(xb, wb, *scales)
        s = Fraction(float(np.float32(scales[0]))) * Fraction(float(np.float32(scales[1])))
        for m in range(M):
            for n in range(N):
                want = exact.round_fraction(Fraction(int(acc[m, n]), 2 ** 18) * s, **exact.BF16)
                assert exact.bf16_code_to_fraction(out[m, n]) == want


def test_fp8_mx_exact_and_invariants():
    M, N, K = 3, 4, 128
    xq, wq, xe, we = gen.fp8_inputs(M, N, K, "fp8_mx", seed=23)
    rng = np.random.default_rng(5)
    xe = torch.from_numpy(rng.integers(120, 135, size=(M, K // 32)).astype(np.uint8))
    we = torch.from_numpy(rng.integers(118, 131, size=(N, K // 32)).astype(np.uint8))
    xb, wb, xeb, web = gen.bits8(xq), gen.bits8(wq), gen.bits8(xe), gen.bits8(we)
    xi, wi = _e4m3_int(xb), _e4m3_int(wb)
    out = oracle.gemm_fp8_mx(xb, wb, xeb, web)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for blk in range(K // 32):
                part = int(np.dot(xi[m, blk * 32:(blk + 1) * 32], wi[n, blk * 32:(blk + 1) * 32]))
                s += Fraction(part, 2 ** 18) * Fraction(2) ** (int(xeb[m, blk]) - 127) \
                    * Fraction(2) ** (int(web[n, blk]) - 127)
            want = exact.round_fraction(s, **exact.BF16)
            assert exact.bf16_code_to_fraction(out[m, n]) == want
    # raising every x-block exponent of row m by j scales row m by exactly 2^j
    xe2 = xeb.copy()
    xe2[1] += 3
    out2 = oracle.gemm_fp8_mx(xb, wb, xe2, web)
    d, d2 = _decode(out), _decode(out2)
    assert np.array_equal(d2[1], d[1] * 8) and np.array_equal(d2[[0, 2]], d[[0, 2]])
    # all exponents 127 is per-tensor with unit scales
    ones_x = np.full_like(xeb, 127)
    ones_w = np.full_like(web, 127)
    assert np.array_equal(oracle.gemm_fp8_mx(xb, wb, ones_x, ones_w),
                          oracle.gemm_fp8_tensor(xb, wb, 1.0, 1.0))


# FP8 with bias.  Per-tensor: out = RNE_bf16(sx * sw * sum(xq * wq) + bias),
# the scale product applied once, to the sum only, and the bias added after
# it ("sglang PR #28333" page: the key source snippet adds the bias to the
# GEMM's output; its motivation section makes the scales belong to the
# product, applied once).  MX: the bias is added after every block's scaled
# partial ("sglang PR #34042" page).  The scales here are non-unit powers of
# two and the bias is large enough to move the rounded output, so a bias
# placed before the scale product (shrunk by sx * sw) or dropped gives other
# bits; the tests check that they would.

def _int_bias(N, seed, lo=-3, hi=3):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (N,), generator=g).to(torch.bfloat16)


def _small_int_codes(rows, K, seed):
    g = torch.Generator().manual_seed(seed)
    return gen.bits8(torch.randint(-2, 3, (rows, K), generator=g).float().to(torch.float8_e4m3fn))


def test_fp8_per_tensor_bias_after_the_scale_exact():
    sx, sw = 2.0 ** -3, 2.0 ** -2
    # (a) small e4m3 integers: every value is a small exact rational
    M, N, K = 4, 9, 64
    xb, wb = _small_int_codes(M, K, 61), _small_int_codes(N, K, 62)
    bias = _int_bias(N, 63)
    bb = gen.bits16(bias)
    out = oracle.gemm_fp8_tensor(xb, wb, sx, sw, bb)
    dot = _e4m3_int(xb) @ _e4m3_int(wb).T  # units of 2^-18
    s = Fraction(1, 32)
    moved = 0
    for m in range(M):
        for n in range(N):
            d = Fraction(int(dot[m, n]), 2 ** 18)
            b = exact.bf16_code_to_fraction(bb[n])
            want = exact.round_fraction(d * s + b, **exact.BF16)
            assert exact.bf16_code_to_fraction(out[m, n]) == want, (m, n)
            before = exact.round_fraction((d + b) * s, **exact.BF16)
            dropped = exact.round_fraction(d * s, **exact.BF16)
            moved += (before != want) and (dropped != want)
    # the pin separates the right placement from both wrong ones
    assert moved >= (M * N) // 2, moved
    # (b) codes quantised from N(0,1) with the same scales and a bias of the
    # outputs' own size
    M, N, K = 3, 7, 256
    xq, wq, _, _ = gen.fp8_inputs(M, N, K, "fp8_tensor", seed=64)
    xb, wb = gen.bits8(xq), gen.bits8(wq)
    dot = _e4m3_int(xb) @ _e4m3_int(wb).T
    g = torch.Generator().manual_seed(65)
    bias = (torch.randn(N, generator=g) * float(np.abs(dot).mean()) * 2.0 ** -23).to(torch.bfloat16)
    bb = gen.bits16(bias)
    out = oracle.gemm_fp8_tensor(xb, wb, sx, sw, bb)
    for m in range(M):
        for n in range(N):
            want = exact.round_fraction(Fraction(int(dot[m, n]), 2 ** 18) * s
                                        + exact.bf16_code_to_fraction(bb[n]), **exact.BF16)
            assert exact.bf16_code_to_fraction(out[m, n]) == want, (m, n)


def test_fp8_mx_bias_after_every_block_exact():
    M, N, K = 3, 6, 128
    # (a) small e4m3 integers, exponents 125..129: exact values
    xb, wb = _small_int_codes(M, K, 71), _small_int_codes(N, K, 72)
    rng = np.random.default_rng(73)
    xe = rng.integers(125, 130, size=(M, K // 32)).astype(np.uint8)
    we = rng.integers(125, 130, size=(N, K // 32)).astype(np.uint8)
    bias = _int_bias(N, 74)
    bb = gen.bits16(bias)
    xi, wi = _e4m3_int(xb), _e4m3_int(wb)

    def scaled(m, n, xe_, we_):
        s = Fraction(0)
        for blk in range(K // 32):
            part = int(np.dot(xi[m, blk * 32:(blk + 1) * 32], wi[n, blk * 32:(blk + 1) * 32]))
            s += Fraction(part, 2 ** 18) * Fraction(2) ** (int(xe_[m, blk]) - 127) \
                * Fraction(2) ** (int(we_[n, blk]) - 127)
        return s

    out = oracle.gemm_fp8_mx(xb, wb, xe, we, bb)
    moved = 0
    for m in range(M):
        for n in range(N):
            b = exact.bf16_code_to_fraction(bb[n])
            want = exact.round_fraction(scaled(m, n, xe, we) + b, **exact.BF16)
            assert exact.bf16_code_to_fraction(out[m, n]) == want, (m, n)
            moved += exact.round_fraction(scaled(m, n, xe, we), **exact.BF16) != want
    assert moved >= (M * N) // 2, moved
    # (b) codes quantised from N(0,1) with their own block exponents and a
    # bias of the outputs' size
    xq, wq, xe2, we2 = gen.fp8_inputs(M, N, K, "fp8_mx", seed=75)
    xb, wb, xe2, we2 = gen.bits8(xq), gen.bits8(wq), gen.bits8(xe2), gen.bits8(we2)
    xi, wi = _e4m3_int(xb), _e4m3_int(wb)
    mag = float(np.mean([abs(float(scaled(m, n, xe2, we2))) for m in range(M) for n in range(N)]))
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(76)) * mag).to(torch.bfloat16)
    bb = gen.bits16(bias)
    out = oracle.gemm_fp8_mx(xb, wb, xe2, we2, bb)
    for m in range(M):
        for n in range(N):
            want = exact.round_fraction(scaled(m, n, xe2, we2) + exact.bf16_code_to_fraction(bb[n]),
                                        **exact.BF16)
            assert exact.bf16_code_to_fraction(out[m, n]) == want, (m, n)


def test_no_intermediate_fp32_rounding():
    # 1.5 * (1 + 2^-7) = 1.51171875 is exactly the midpoint of the bf16
    # neighbours 1.5078125 and 1.515625.  Subtracting 2^-30 (from
    # 2^-15 * -2^-15) puts the exact sum just below it, so one correct
    # rounding gives 1.5078125.  An fp32 intermediate would snap the sum
    # back onto the midpoint and the tie would go to 1.515625.
    x = torch.tensor([[1.5, 2.0 ** -15]], dtype=torch.bfloat16)
    w = torch.tensor([[1.0078125, -(2.0 ** -15)]], dtype=torch.bfloat16)
    out = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w))
    assert out[0, 0] == 0x3FC1
    w2 = torch.tensor([[1.0078125, 2.0 ** -15]], dtype=torch.bfloat16)
    assert oracle.gemm_bf16(gen.bits16(x), gen.bits16(w2))[0, 0] == 0x3FC2


# ------------------------------------------------ static FP8 quantisation
# "sglang PR #28333" page, static FP8 quant kernel: q = e4m3(clamp(x * (1/s),
# -448, 448)) in binary32.  The encoder is pinned to the e4m3 bit fields
# (exact rationals, independent of the oracle's code) and the quantiser to
# torch's own binary32 arithmetic and float8_e4m3fn cast.

def _finite_e4m3_values():
    vals = []
    for code in range(256):
        f = exact.e4m3_code_to_fraction(code)
        if isinstance(f, Fraction):  # NaN codes are checked on their own
            vals.append((f, code))
    return vals


def test_encode_e4m3_round_trips_every_code():
    for f, code in _finite_e4m3_values():
        got = oracle.encode_e4m3(float(f)) if f != 0 else oracle.encode_e4m3(-0.0 if code & 0x80 else 0.0)
        assert got == code, (code, f, got)


def test_encode_e4m3_midpoints_round_to_even():
    pos = sorted({f for f, c in _finite_e4m3_values() if f >= 0})
    code_of = {f: c for f, c in _finite_e4m3_values() if not (c & 0x80)}
    for lo, hi in zip(pos, pos[1:]):
        mid = (lo + hi) / 2
        even = lo if code_of[lo] % 2 == 0 else hi
        assert float(mid) == mid  # midpoints of e4m3 neighbours are binary32 values
        assert oracle.encode_e4m3(float(mid)) == code_of[even], (lo, hi)
        assert oracle.encode_e4m3(-float(mid)) == code_of[even] | 0x80
        # just off the midpoint, by one binary32 ulp, the nearer neighbour wins
        below = float(np.nextafter(np.float32(mid), np.float32(0)))
        above = float(np.nextafter(np.float32(mid), np.float32(1e9)))
        assert oracle.encode_e4m3(below) == code_of[lo]
        assert oracle.encode_e4m3(above) == code_of[hi]
    assert oracle.encode_e4m3(float("nan")) == 0x7F
    assert oracle.encode_e4m3(-float("nan")) == 0xFF


@pytest.mark.parametrize("s", [1.0, 0.037, 3.5, 2.0 ** -4, 1e-3, 448.0 / 7.25])
def test_quant_matches_torch_for_every_bf16_code(s):
    codes = np.arange(65536, dtype=np.uint16)
    q = oracle.quant_e4m3(codes, s)
    x = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float()
    inv = 1.0 / torch.tensor(s, dtype=torch.float32)
    ref = (x * inv).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = torch.isnan(x).numpy()
    assert np.array_equal(q[~nan], ref[~nan])
    assert np.all((q[nan] & 0x7F) == 0x7F)


def _bf16_as_f32(code):
    return np.array([code], np.uint16).astype(np.uint32).__lshift__(16).view(np.float32)[0]


def test_quant_uses_the_reciprocal_not_a_division():
    # x * (1/s) and x / s are different binary32 roundings; with this scale
    # and x = 1.0546875 (a bf16 value) they straddle the e4m3 midpoint 1.0625
    # between 1.0 and 1.125.  The page's kernel multiplies by the reciprocal.
    s = np.float32(0.9926469922065735)
    xv = np.float32(1.0546875)
    a, b = np.float32(xv * (np.float32(1.0) / s)), np.float32(xv / s)
    assert a != b
    code = int(np.array([xv], np.float32).view(np.uint32)[0] >> 16)
    q = oracle.quant_e4m3(np.array([code], np.uint16), float(s))[0]
    ref = torch.tensor([float(a)], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()
    wrong = torch.tensor([float(b)], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()
    assert ref != wrong and q == ref


def test_gemm_fp8_quant_composes_quant_and_gemm():
    x, _, _ = gen.bf16_inputs(3, 8, 64, False, seed=4)
    g = torch.Generator().manual_seed(5)
    wcodes = gen.bits8(torch.randint(-2, 3, (8, 64), generator=g).float().to(torch.float8_e4m3fn))
    xq = oracle.quant_e4m3(gen.bits16(x), 0.02)
    a = oracle.gemm_fp8_quant(gen.bits16(x), wcodes, 0.02, 0.5, out_f32=True)
    b = oracle.gemm_fp8_tensor(xq, wcodes, 0.02, 0.5, out_f32=True)
    assert np.array_equal(a, b)
    # and the codes are the ones the quantiser pins fix: spot-check by torch
    ref = (x.float() * (1.0 / torch.tensor(0.02, dtype=torch.float32))).clamp(-448, 448)
    assert np.array_equal(xq, gen.bits8(ref.to(torch.float8_e4m3fn)))
