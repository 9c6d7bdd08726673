"""The workload points of the small-M GEMM, by name and size.

Shapes follow the router and decode-linear layers the pages describe:
router (K, N) pairs of 7168 x 256/384 experts ("vllm PR #42562" page,
motivation), the tuned router shapes (4096,256), (6144,256), (7168,256),
(7168,384) ("vllm PR #48774" page, tuned tables), the non-tile-aligned
K = 2880 of the router kernel's tests ("vllm PR #42562" page, impl. item 6),
dense decode linears with M up to 128, and FP8 K = N = 4096 GEMMs.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Point:
    group: str          # workload family name
    dtype: str          # "bf16" | "fp8_tensor" | "fp8_mx"
    M: int
    N: int
    K: int
    bias: bool

    def key(self) -> str:
        """Canonical string; its SHA-256 seeds the generator."""
        return f"{self.dtype}|M={self.M}|N={self.N}|K={self.K}|bias={int(self.bias)}"


def small_bf16():
    """bf16, M=1, K=2048, N=256, no bias: the case the oracle finishes fastest."""
    return [Point("small_bf16", "bf16", 1, 256, 2048, False)]


def router_k7168():
    """bf16 router sweep: M = 1..16, K = 7168, N in {256, 384}, no bias."""
    return [Point("router_k7168", "bf16", M, N, 7168, False)
            for N in (256, 384) for M in range(1, 17)]


def router_shapes():
    """bf16 router shapes (4096,256), (6144,256), (2880,128) at
    M in {1,3,4,5,8,9,12,16}, with and without bias."""
    return [Point("router_shapes", "bf16", M, N, K, b)
            for (K, N) in ((4096, 256), (6144, 256), (2880, 128))
            for M in (1, 3, 4, 5, 8, 9, 12, 16)
            for b in (False, True)]


def decode_linear():
    """bf16 dense decode linear: M in {1,8,32,64,128}, K = 7168,
    N in {2112, 576, 4096}, with and without bias."""
    return [Point("decode_linear", "bf16", M, N, 7168, b)
            for N in (2112, 576, 4096)
            for M in (1, 8, 32, 64, 128)
            for b in (False, True)]


def fp8_square(mode):
    """FP8 e4m3, M in {1,16,64,128}, K = N = 4096, no bias;
    mode "fp8_tensor" (per-tensor fp32 scales) or "fp8_mx" (e8m0 per 32 K)."""
    return [Point("fp8_" + mode.split("_")[1], mode, M, 4096, 4096, False)
            for M in (1, 16, 64, 128)]


def larger_m():
    """The larger-M regime (M = 129-512, row blocks of 128), at sizes the
    oracle finishes in seconds: bf16 with and without bias, FP8 in both
    scale modes."""
    return ([Point("larger_m", "bf16", 129, 96, 1024, True),
             Point("larger_m", "bf16", 256, 576, 2048, False),
             Point("larger_m", "bf16", 512, 512, 2048, True)]
            + [Point("larger_m", mode, M, 512, 2048, False)
               for mode in ("fp8_tensor", "fp8_mx") for M in (200, 512)])


def larger_m_full():
    """The larger-M regime at full size (swept and benchmarked; parity is
    checked on sampled outputs): bf16 dense decode K = 7168, N = 4096 and
    FP8 K = N = 4096, M in {256, 512}."""
    return ([Point("larger_m_full", "bf16", M, 4096, 7168, False) for M in (256, 512)]
            + [Point("larger_m_full", mode, M, 4096, 4096, False)
               for mode in ("fp8_tensor", "fp8_mx") for M in (256, 512)])


def all_points():
    return (small_bf16() + router_k7168() + router_shapes() + decode_linear()
            + fp8_square("fp8_tensor") + fp8_square("fp8_mx") + larger_m())


# The headline workload: bf16, K = 7168, N = 256, M = 1..16.
HEADLINE = [p for p in router_k7168() if p.N == 256]
