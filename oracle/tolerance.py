"""Elementwise acceptance test for GPU results against the oracle.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check, the benchmark's
CPU-baseline leg).

Bound, per element:  |gpu - ref| <= 2^-7 * |ref| + 1e-3 * sqrt(K) * rms(ref)
where ref is the oracle's output widened to fp64 and rms(ref) is taken over
every finite element of that call's output.  NaN and +-Inf must match
exactly (same class, same sign for Inf).  With an all-zero reference the
bound reduces to exact equality.
"""
import math

import numpy as np
import torch


def widen(out, out_f32=False):
    """bf16 bit patterns (uint16/int16 numpy or torch) or float32 -> float64 numpy."""
    if isinstance(out, torch.Tensor):
        out = out.detach().cpu()
        if out.dtype == torch.bfloat16:
            return out.to(torch.float64).numpy()
        out = out.numpy()
    out = np.asarray(out)
    if out_f32 or out.dtype == np.float32:
        return out.astype(np.float64)
    return torch.from_numpy(out.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def bound(ref, K):
    fin = np.isfinite(ref)
    rms = math.sqrt(float(np.mean(ref[fin] ** 2))) if fin.any() else 0.0
    return 2.0 ** -7 * np.abs(ref) + 1e-3 * math.sqrt(K) * rms


def check(gpu, ref, K, out_f32=False):
    """Returns (ok, message).  gpu/ref: bf16 bit patterns or float32 arrays."""
    g = widen(gpu, out_f32)
    r = widen(ref, out_f32)
    if g.shape != r.shape:
        return False, f"shape {g.shape} != {r.shape}"
    nan_r, nan_g = np.isnan(r), np.isnan(g)
    if not np.array_equal(nan_r, nan_g):
        i = tuple(int(v) for v in np.argwhere(nan_r != nan_g)[0])
        return False, f"NaN mismatch at {i}: gpu={g[i]} ref={r[i]}"
    inf_r = np.isinf(r)
    if not np.array_equal(inf_r, np.isinf(g)) or not np.array_equal(r[inf_r], g[inf_r]):
        return False, "Inf mismatch"
    fin = np.isfinite(r)
    b = bound(r, K)
    err = np.abs(g - r)
    bad = fin & ~(err <= b)
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        return False, (f"{int(bad.sum())} of {r.size} elements out of tolerance; first at {i}: "
                       f"gpu={g[i]!r} ref={r[i]!r} err={err[i]:.3e} bound={b[i]:.3e}")
    worst = float(np.max(err[fin] / np.maximum(b[fin], 1e-300))) if fin.any() else 0.0
    return True, f"ok (worst err/bound = {worst:.3f})"
