"""Seeded input generators.

Every input is synthetic and reproducible: a torch CPU generator seeded with
the first 4 bytes (little-endian) of SHA-256 of the point's canonical string.
Draw order: x, then W, then bias.  Values are drawn as fp32 and converted to
bf16 by torch (a single round-to-nearest-even from fp32).

Distributions (the second parameter of N(., .) is the variance):
  x ~ N(0, 1), W ~ N(0, 1/K), bias ~ N(0, 0.1)   (bf16 points)
  x0, W0 ~ N(0, 1) fp32, then quantised to e4m3fn  (FP8 points)

FP8 quantisation of the generated inputs (input preparation, not the GEMM):
  per-tensor: s = amax / 448 (fp32); q = e4m3(clamp(v * (1/s), -448, 448)),
              multiplying by the reciprocal as the quantisation kernel on the
              "sglang PR #28333" page does.
  MX:         per row and per 32-element K block, e = ceil(log2(amax_b/448))
              clamped to [-127, 127] plus the bias 127 (an all-zero block
              takes e = 127); q = e4m3(clamp(v * 2^-(e-127), -448, 448)).
The casts to e4m3fn are torch's own (round-to-nearest-even).

Also here: the structured inputs the oracle's pins and the exact-regime GPU
tests use (all-ones, sign-alternating, one-hot, small integers, and the
brute-force enumeration set).  All tensors returned are CPU tensors.
"""
import hashlib
import math

import torch

BF16 = torch.bfloat16
E4M3 = torch.float8_e4m3fn


def seed_of(key: str) -> int:
    return int.from_bytes(hashlib.sha256(key.encode()).digest()[:4], "little")


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def bf16_inputs(M, N, K, bias, seed):
    """Returns (x[M,K], W[N,K], bias[N] or None) as bf16 CPU tensors."""
    g = _gen(seed)
    x = torch.randn(M, K, generator=g, dtype=torch.float32).to(BF16)
    w = (torch.randn(N, K, generator=g, dtype=torch.float32)
         * torch.tensor(1.0 / math.sqrt(K), dtype=torch.float32)).to(BF16)
    b = None
    if bias:
        b = (torch.randn(N, generator=g, dtype=torch.float32)
             * torch.tensor(math.sqrt(0.1), dtype=torch.float32)).to(BF16)
    return x, w, b


def quantise_per_tensor(v):
    """v fp32 -> (q e4m3fn, s fp32 scalar tensor)."""
    amax = v.abs().max().to(torch.float32)
    s = (amax / 448.0).to(torch.float32) if amax > 0 else torch.tensor(1.0)
    inv = (1.0 / s).to(torch.float32)
    q = (v * inv).clamp(-448.0, 448.0).to(E4M3)
    return q, s.reshape(1)


def quantise_mx(v):
    """v fp32 [R, K] -> (q e4m3fn [R,K], e uint8 [R, K/32])."""
    R, K = v.shape
    assert K % 32 == 0
    blocks = v.reshape(R, K // 32, 32)
    amax = blocks.abs().amax(dim=2).to(torch.float64)
    e = torch.full(amax.shape, 127, dtype=torch.int64)
    nz = amax > 0
    e[nz] = torch.ceil(torch.log2(amax[nz] / 448.0)).clamp(-127, 127).to(torch.int64) + 127
    scale_inv = torch.ldexp(torch.ones_like(amax), -(e - 127)).to(torch.float32)
    q = (blocks * scale_inv.unsqueeze(2)).clamp(-448.0, 448.0).to(E4M3).reshape(R, K)
    return q, e.to(torch.uint8)


def fp8_inputs(M, N, K, mode, seed):
    """FP8 point inputs.  mode "fp8_tensor": (xq, wq, sx[1], sw[1]);
    mode "fp8_mx": (xq, wq, xe[M,K/32], we[N,K/32])."""
    g = _gen(seed)
    x0 = torch.randn(M, K, generator=g, dtype=torch.float32)
    w0 = torch.randn(N, K, generator=g, dtype=torch.float32)
    if mode == "fp8_tensor":
        xq, sx = quantise_per_tensor(x0)
        wq, sw = quantise_per_tensor(w0)
        return xq, wq, sx, sw
    if mode == "fp8_mx":
        xq, xe = quantise_mx(x0)
        wq, we = quantise_mx(w0)
        return xq, wq, xe, we
    raise ValueError(mode)


def point_inputs(p):
    """Inputs for a workloads.configs.Point."""
    if p.dtype == "bf16":
        return bf16_inputs(p.M, p.N, p.K, p.bias, seed_of(p.key()))
    return fp8_inputs(p.M, p.N, p.K, p.dtype, seed_of(p.key()))


# ------------------------------------------------------------ structured inputs

def ones(M, N, K):
    return torch.ones(M, K, dtype=BF16), torch.ones(N, K, dtype=BF16)


def alternating(M, N, K):
    """x = 1, W[n,k] = (-1)^k."""
    w = torch.ones(N, K, dtype=torch.float32)
    w[:, 1::2] = -1.0
    return torch.ones(M, K, dtype=BF16), w.to(BF16)


def one_hot_map(N, K, seed):
    """pi(n): N distinct positions in [0, K), N <= K.  The last columns are
    sent to positions near the end of K, where any tail handling lives."""
    assert N <= K
    perm = torch.randperm(K, generator=_gen(seed))
    targets = [K - 1 - 3 * i for i in range(min(N, 8)) if K - 1 - 3 * i >= 0]
    for i, t in enumerate(targets):
        pos = int((perm == t).nonzero()[0, 0])
        j = N - 1 - i
        perm[pos], perm[j] = perm[j].clone(), perm[pos].clone()
    return perm[:N].clone()


def one_hot(M, N, K, seed):
    """x ~ N(0,1) bf16, W[n, k] = [k == pi(n)].  Returns (x, W, pi)."""
    g = _gen(seed)
    x = torch.randn(M, K, generator=g, dtype=torch.float32).to(BF16)
    pi = one_hot_map(N, K, seed + 1)
    w = torch.zeros(N, K, dtype=BF16)
    w[torch.arange(N), pi] = 1.0
    return x, w, pi


def small_integers(M, N, K, bias, seed, lo=-2, hi=2):
    """x, W, bias drawn uniformly from the integers lo..hi, as bf16."""
    g = _gen(seed)
    x = torch.randint(lo, hi + 1, (M, K), generator=g).to(BF16)
    w = torch.randint(lo, hi + 1, (N, K), generator=g).to(BF16)
    b = torch.randint(lo, hi + 1, (N,), generator=g).to(BF16) if bias else None
    return x, w, b


def brute_values():
    """A 12-value bf16 set spanning signs, zero, exact/inexact products,
    the smallest subnormal and the largest finite value."""
    codes = [0x0000, 0x8000, 0x3F80, 0xBF80, 0x3FC0, 0x4040, 0x3F81,
             0x3C00, 0x0001, 0x7F7F, 0xC0A0, 0x3EAB]
    return torch.tensor(codes, dtype=torch.int32).to(torch.int16).view(BF16)


def brute_force_set(K=8, positions=(1, 6)):
    """Every pair (a0, a1) x (b0, b1) of brute_values() at two active K
    positions, the rest zero.  M = 1 row per x-combination is too many rows
    for one call, so the enumeration is laid out as:
      x[M, K]: M = len(values)^2 rows, row r holds (a0, a1) = divmod(r, V);
      W[N, K]: N = len(values)^2 rows, row c holds (b0, b1) = divmod(c, V).
    out[r, c] = a0*b0 + a1*b1 covers every combination exactly once."""
    v = brute_values()
    V = v.numel()
    x = torch.zeros(V * V, K, dtype=BF16)
    w = torch.zeros(V * V, K, dtype=BF16)
    idx = torch.arange(V * V)
    x[:, positions[0]] = v[idx // V]
    x[:, positions[1]] = v[idx % V]
    w[:, positions[0]] = v[idx // V]
    w[:, positions[1]] = v[idx % V]
    return x, w


def bits16(t):
    """bf16 tensor -> numpy uint16 bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def bits8(t):
    """e4m3fn / uint8 tensor -> numpy uint8."""
    if t.dtype == torch.uint8:
        return t.contiguous().numpy()
    return t.contiguous().view(torch.uint8).numpy()
