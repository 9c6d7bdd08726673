"""CPU oracle for the small-M GEMM -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (latency_skinny_gemm_amd) never imports it and
shares no code with it.

The arithmetic lives in skinny_oracle.c (plain fp64 triple loop over exactly
decoded inputs, one direct fp64 -> bf16 round-to-nearest-even).  This module
only loads the compiled library and marshals numpy arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    """Load liboracle.so, building it with gcc first if it is absent."""
    global _lib
    if _lib is None:
        # SKINNY_ORACLE_LIB points the pins at another build of the oracle
        # source (the mutation test uses it); the default is the one here.
        path = os.environ.get("SKINNY_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_long
        L.oracle_decode_bf16.restype = ctypes.c_double
        L.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_e4m3.restype = ctypes.c_double
        L.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
        L.oracle_decode_e8m0.restype = ctypes.c_double
        L.oracle_decode_e8m0.argtypes = [ctypes.c_uint8]
        L.oracle_round_bf16.restype = ctypes.c_uint16
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_round_f32.restype = ctypes.c_float
        L.oracle_round_f32.argtypes = [ctypes.c_double]
        L.oracle_gemm_bf16.restype = None
        L.oracle_gemm_bf16.argtypes = [P, P, P, P, P, i64, i64, i64, ctypes.c_int]
        L.oracle_gemm_fp8_tensor.restype = None
        L.oracle_gemm_fp8_tensor.argtypes = [P, P, ctypes.c_float, ctypes.c_float, P, P, P,
                                             i64, i64, i64, ctypes.c_int]
        L.oracle_gemm_fp8_mx.restype = None
        L.oracle_gemm_fp8_mx.argtypes = [P, P, P, P, P, P, P, i64, i64, i64, ctypes.c_int]
        L.oracle_encode_e4m3.restype = ctypes.c_uint8
        L.oracle_encode_e4m3.argtypes = [ctypes.c_float]
        L.oracle_quant_e4m3.restype = None
        L.oracle_quant_e4m3.argtypes = [P, i64, ctypes.c_float, P]
        L.oracle_threads_used.restype = ctypes.c_int
        L.oracle_threads_used.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype in (np.uint16, np.int16), a.dtype
    return a.view(np.uint16)


def _u8(a):
    a = np.ascontiguousarray(a)
    assert a.dtype in (np.uint8, np.int8), a.dtype
    return a.view(np.uint8)


def _out(M, N, out_f32):
    if out_f32:
        return np.zeros((M, N), dtype=np.float32)
    return np.zeros((M, N), dtype=np.uint16)


def gemm_bf16(x, w, bias=None, out_f32=False, threads=1):
    """x[M,K], w[N,K], bias[N] as bf16 bit patterns (uint16).

    Returns out[M,N] as bf16 bit patterns (uint16), or float32 if out_f32."""
    x, w = _u16(x), _u16(w)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    b = None if bias is None else _u16(bias)
    assert b is None or b.shape == (N,)
    out = _out(M, N, out_f32)
    o16 = None if out_f32 else out
    o32 = out if out_f32 else None
    lib().oracle_gemm_bf16(_ptr(x), _ptr(w), _ptr(b), _ptr(o16), _ptr(o32), M, N, K, threads)
    return out


def gemm_fp8_tensor(xq, wq, sx, sw, bias=None, out_f32=False, threads=1):
    """xq[M,K], wq[N,K] as e4m3fn bytes (uint8); sx, sw python/np float32."""
    xq, wq = _u8(xq), _u8(wq)
    M, K = xq.shape
    N, K2 = wq.shape
    assert K == K2
    b = None if bias is None else _u16(bias)
    out = _out(M, N, out_f32)
    o16 = None if out_f32 else out
    o32 = out if out_f32 else None
    lib().oracle_gemm_fp8_tensor(_ptr(xq), _ptr(wq), float(np.float32(sx)), float(np.float32(sw)),
                                 _ptr(b), _ptr(o16), _ptr(o32), M, N, K, threads)
    return out


def encode_e4m3(v):
    """Nearest e4m3fn code (ties to even) of a binary32 value in [-448, 448]."""
    return int(lib().oracle_encode_e4m3(float(np.float32(v))))


def quant_e4m3(x, s):
    """Static per-tensor quantisation of bf16 codes x (any shape) with the
    fp32 scale s: e4m3 codes of clamp(x * (1/s), -448, 448), in binary32."""
    x = _u16(x)
    q = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_quant_e4m3(_ptr(x), x.size, float(np.float32(s)), _ptr(q))
    return q


def gemm_fp8_quant(x, wq, sx, sw, bias=None, out_f32=False, threads=1):
    """bf16 x[M,K] quantised statically with sx, then the per-tensor FP8 GEMM
    with e4m3 wq[N,K] and sw."""
    return gemm_fp8_tensor(quant_e4m3(x, sx), wq, sx, sw, bias, out_f32, threads)


def gemm_fp8_mx(xq, wq, xe, we, bias=None, out_f32=False, threads=1):
    """xq[M,K], wq[N,K] e4m3fn bytes; xe[M,K/32], we[N,K/32] e8m0 bytes."""
    xq, wq, xe, we = _u8(xq), _u8(wq), _u8(xe), _u8(we)
    M, K = xq.shape
    N, K2 = wq.shape
    assert K == K2 and K % 32 == 0
    assert xe.shape == (M, K // 32) and we.shape == (N, K // 32)
    b = None if bias is None else _u16(bias)
    out = _out(M, N, out_f32)
    o16 = None if out_f32 else out
    o32 = out if out_f32 else None
    lib().oracle_gemm_fp8_mx(_ptr(xq), _ptr(wq), _ptr(xe), _ptr(we), _ptr(b), _ptr(o16),
                             _ptr(o32), M, N, K, threads)
    return out


def decode_bf16(code):
    return lib().oracle_decode_bf16(int(code))


def decode_e4m3(code):
    return lib().oracle_decode_e4m3(int(code))


def decode_e8m0(code):
    return lib().oracle_decode_e8m0(int(code))


def round_bf16(v):
    return int(lib().oracle_round_bf16(float(v)))


def threads_used(requested):
    return int(lib().oracle_threads_used(int(requested)))
