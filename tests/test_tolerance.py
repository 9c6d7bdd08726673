"""The acceptance test itself, on the CPU: it must reject a planted error a
little above the bound and accept the oracle's own output."""
import numpy as np
import torch

import oracle
from oracle import tolerance
from workloads import inputs as gen


def test_accepts_reference_and_rejects_planted_errors():
    x, w, b = gen.bf16_inputs(4, 64, 2880, True, seed=8)
    ref = oracle.gemm_bf16(gen.bits16(x), gen.bits16(w), gen.bits16(b))
    ok, _ = tolerance.check(ref, ref, 2880)
    assert ok
    r = tolerance.widen(ref)
    bnd = tolerance.bound(r, 2880)
    bad = r.copy()
    bad[2, 17] += 3.0 * bnd[2, 17]  # survives the bf16 conversion below
    ok, msg = tolerance.check(torch.from_numpy(bad).to(torch.bfloat16), ref, 2880)
    assert not ok and "(2, 17)" in msg
    nanned = r.copy()
    nanned[0, 0] = np.nan
    ok, msg = tolerance.check(torch.from_numpy(nanned).to(torch.bfloat16), ref, 2880)
    assert not ok and "NaN" in msg


def test_all_zero_reference_demands_exact_zero():
    z = np.zeros((2, 3), dtype=np.uint16)
    ok, _ = tolerance.check(z, z, 4096)
    assert ok
    one = z.copy()
    one[1, 1] = 0x0001  # smallest subnormal
    ok, _ = tolerance.check(one, z, 4096)
    assert not ok
