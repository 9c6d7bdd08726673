"""Python binding of the small-M GEMM library (libskinny_gemm.so).

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  When the
library is not built, every call raises: there is no fallback.

    out[M, N] = bf16( x[M, K] @ W[N, K]^T (+ bias[N]) ), fp32 accumulation.
"""
import ctypes
import os

import torch

__all__ = ["SkgPlan", "SkinnyGemmError", "gemm_bf16", "gemm_bf16_planned", "gemm_fp8",
           "gemm_fp8_planned", "plan", "plan_on",
           "plan_complete", "reserve", "release_all", "status_string", "library_path",
           "KIND_DOT", "KIND_SPLITK", "KIND_TILED", "KIND_ROWS", "REDUCE_NONE", "REDUCE_LAST", "REDUCE_KERNEL", "FLAG_DOT2", "FLAG_TILED_WIDE", "FLAG_DOT_XLDS", "FLAG_ROWS_HALF", "FLAG_DOT_WFIRST",
           "DTYPE_BF16", "DTYPE_FP8", "DTYPE_F32", "DTYPE_FP8_MX", "gemm_bf16_f32", "gemm_fp8_quant",
           "quant_e4m3"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libskinny_gemm.so")

# mirrors of include/skinny_gemm.h
OK = 0
ERR_INVALID_ARG = -1
ERR_ALIGNMENT = -2
ERR_UNSUPPORTED = -3
ERR_WORKSPACE = -4
ERR_HIP = -5
DTYPE_BF16 = 0
DTYPE_FP8 = 1
DTYPE_F32 = 2  # output dtype only
DTYPE_FP8_MX = 3  # planning only: FP8 with MX block scales (its own table entries)
FP8_PER_TENSOR = 1
FP8_MX32 = 2
KIND_DOT = 1
KIND_SPLITK = 2
KIND_TILED = 3
KIND_ROWS = 4
REDUCE_NONE = 0
REDUCE_LAST = 1
REDUCE_KERNEL = 2
FLAG_DOT2 = 1
FLAG_TILED_WIDE = 2
FLAG_DOT_XLDS = 4
FLAG_ROWS_HALF = 8
FLAG_DOT_WFIRST = 16
MAX_M = 512


class SkgPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("kind", "threads", "cols", "splits", "depth", "waves_m", "reduce", "flags",
                 "k_chunk", "m_tiles", "grid", "from_table")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}

    def __repr__(self):
        return "SkgPlan(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"


class SkinnyGemmError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class Fp8Scales(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("sx", ctypes.c_void_p), ("sw", ctypes.c_void_p),
                ("x_e8m0", ctypes.c_void_p), ("w_e8m0", ctypes.c_void_p)]


_lib = None


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                           "(hipcc for gfx950).  There is no fallback implementation.")
    L = ctypes.CDLL(_LIB_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    PP = ctypes.POINTER(SkgPlan)
    L.skinny_gemm_bf16.argtypes = [P, P, P, P, P, I, I, I, P]
    L.skinny_gemm_bf16.restype = I
    L.skinny_gemm_bf16_noalloc.argtypes = [P, P, P, P, P, I, I, I, P]
    L.skinny_gemm_bf16_noalloc.restype = I
    L.skinny_gemm_bf16_planned.argtypes = [P, P, P, P, I, I, I, PP, P]
    L.skinny_gemm_bf16_planned.restype = I
    L.skinny_gemm_fp8.argtypes = [P, P, P, ctypes.POINTER(Fp8Scales), P, I, I, I, P]
    L.skinny_gemm_fp8.restype = I
    L.skinny_gemm_fp8_planned.argtypes = [P, P, P, ctypes.POINTER(Fp8Scales), P, I, I, I, PP, P]
    L.skinny_gemm_fp8_planned.restype = I
    L.skinny_gemm_bf16_f32.argtypes = [P, P, P, P, I, I, I, P]
    L.skinny_gemm_bf16_f32.restype = I
    L.skinny_gemm_bf16_f32_planned.argtypes = [P, P, P, P, I, I, I, PP, P]
    L.skinny_gemm_bf16_f32_planned.restype = I
    L.skinny_gemm_fp8_quant.argtypes = [P, P, P, P, P, P, I, I, I, I, P]
    L.skinny_gemm_fp8_quant.restype = I
    L.skinny_gemm_fp8_quant_planned.argtypes = [P, P, P, P, P, P, I, I, I, I, PP, P]
    L.skinny_gemm_fp8_quant_planned.restype = I
    L.skinny_quant_e4m3.argtypes = [P, P, P, ctypes.c_long, P]
    L.skinny_quant_e4m3.restype = I
    L.skinny_gemm_plan.argtypes = [I, I, I, I, PP]
    L.skinny_gemm_plan.restype = I
    L.skinny_gemm_plan_on.argtypes = [I, I, I, I, I, PP]
    L.skinny_gemm_plan_on.restype = I
    L.skinny_gemm_plan_complete.argtypes = [I, I, I, I, PP]
    L.skinny_gemm_plan_complete.restype = I
    L.skinny_gemm_reserve.argtypes = [I, I, I, I, P]
    L.skinny_gemm_reserve.restype = I
    L.skinny_gemm_release_all.argtypes = []
    L.skinny_gemm_release_all.restype = I
    L.skinny_gemm_status_string.argtypes = [I]
    L.skinny_gemm_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def status_string(status):
    return _load().skinny_gemm_status_string(int(status)).decode()


def _check(status, what):
    if status != OK:
        raise SkinnyGemmError(status, what)


def _one_device(*ts):
    """The device of the given tensors (None entries skipped); all must share it."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"all tensors must be on one device, got {dev} and {t.device}")
    return dev


def _launch(dev, stream, fn, *args):
    """fn(*args, stream) with `dev` current (the library keeps its workspaces
    per current device) on `stream`, else dev's current stream."""
    with torch.cuda.device(dev):
        s = torch.cuda.current_stream() if stream is None else stream
        if s.device != dev:
            raise ValueError(f"stream is on {s.device}, the tensors on {dev}")
        return fn(*args, ctypes.c_void_p(s.cuda_stream))


def _empty(shape, dtype, device, stream):
    """A new output tensor, allocated for the stream the call runs on (so the
    caching allocator does not hand its memory to other work on another
    stream while the call may still write it)."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensors(x, W, bias, out, dtype):
    if x.dim() != 2 or W.dim() != 2 or x.shape[1] != W.shape[1]:
        raise ValueError(f"x[M,K] and W[N,K] expected, got {tuple(x.shape)} and {tuple(W.shape)}")
    M, K = x.shape
    N = W.shape[0]
    for name, t in (("x", x), ("W", W), ("bias", bias), ("out", out)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (the library takes no strides)")
    if x.dtype != dtype or W.dtype != dtype:
        raise TypeError(f"x and W must be {dtype}, got {x.dtype} and {W.dtype}")
    if bias is not None and (bias.dtype != torch.bfloat16 or tuple(bias.shape) != (N,)):
        raise TypeError("bias must be bf16 [N]")
    if out is not None and (out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N)):
        raise TypeError("out must be bf16 [M, N]")
    return M, N, K


def gemm_bf16(x, W, bias=None, out=None, stream=None):
    """out[M,N] = x[M,K] @ W[N,K]^T (+ bias), bf16, on the library's plan."""
    M, N, K = _check_tensors(x, W, bias, out, torch.bfloat16)
    if out is None:
        out = _empty((M, N), torch.bfloat16, x.device, stream)
    rc = _launch(_one_device(x, W, bias, out), stream, _load().skinny_gemm_bf16, _ptr(x), _ptr(W),
                 _ptr(bias), None, _ptr(out), M, N, K)
    _check(rc, f"skinny_gemm_bf16(M={M}, N={N}, K={K})")
    return out


def gemm_bf16_noalloc(x, W, bias, out, stream=None):
    """As gemm_bf16 through skinny_gemm_bf16_noalloc: `out` must be given
    (nothing is allocated); split partials use the library's fixed per-GPU
    array, so calls that overlap in time on one GPU race."""
    M, N, K = _check_tensors(x, W, bias, out, torch.bfloat16)
    if out is None:
        raise TypeError("gemm_bf16_noalloc needs an output tensor")
    rc = _launch(_one_device(x, W, bias, out), stream, _load().skinny_gemm_bf16_noalloc, _ptr(x),
                 _ptr(W), _ptr(bias), None, _ptr(out), M, N, K)
    _check(rc, f"skinny_gemm_bf16_noalloc(M={M}, N={N}, K={K})")
    return out


def gemm_bf16_planned(x, W, p, bias=None, out=None, stream=None):
    """As gemm_bf16, with a caller-made SkgPlan (completed by the library)."""
    M, N, K = _check_tensors(x, W, bias, out, torch.bfloat16)
    if out is None:
        out = _empty((M, N), torch.bfloat16, x.device, stream)
    rc = _launch(_one_device(x, W, bias, out), stream, _load().skinny_gemm_bf16_planned, _ptr(x),
                 _ptr(W), _ptr(bias), _ptr(out), M, N, K, ctypes.byref(p))
    _check(rc, f"skinny_gemm_bf16_planned(M={M}, N={N}, K={K}, {p})")
    return out


def gemm_bf16_f32(x, W, bias=None, out=None, plan=None, stream=None):
    """fp32 logits: out[M,N] = x[M,K] @ W[N,K]^T (+ bias) in fp32 (no bf16
    rounding); the library's plan, or a caller-made one."""
    M, N, K = _check_tensors(x, W, bias, None, torch.bfloat16)
    if out is None:
        out = _empty((M, N), torch.float32, x.device, stream)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise TypeError("out must be contiguous float32 [M, N]")
    dev = _one_device(x, W, bias, out)
    if plan is None:
        rc = _launch(dev, stream, _load().skinny_gemm_bf16_f32, _ptr(x), _ptr(W), _ptr(bias),
                     _ptr(out), M, N, K)
    else:
        rc = _launch(dev, stream, _load().skinny_gemm_bf16_f32_planned, _ptr(x), _ptr(W),
                     _ptr(bias), _ptr(out), M, N, K, ctypes.byref(plan))
    _check(rc, f"skinny_gemm_bf16_f32(M={M}, N={N}, K={K}, {plan})")
    return out


def _scalar_f32(name, t):
    if t is None or t.dtype != torch.float32 or t.numel() != 1 or not t.is_cuda:
        raise TypeError(f"{name} must be a one-element float32 device tensor")


def gemm_fp8_quant(x, wq, sx, sw, bias=None, out_dtype=torch.bfloat16, out=None, plan=None,
                   stream=None):
    """bf16 x quantised statically to e4m3 with sx, times e4m3 wq with sw
    (per-tensor): out = sx*sw*sum(q*w) (+ bias), bf16 or fp32."""
    if x.dim() != 2 or not x.is_cuda or not x.is_contiguous() or x.dtype != torch.bfloat16:
        raise TypeError("x must be a contiguous bf16 [M, K] device tensor")
    if wq.dim() != 2 or not wq.is_cuda or not wq.is_contiguous() or \
            wq.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError("wq must be a contiguous float8_e4m3fn [N, K] device tensor")
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("x[M,K] and wq[N,K] expected")
    _scalar_f32("sx", sx)
    _scalar_f32("sw", sw)
    if bias is not None and (bias.dtype != torch.bfloat16 or tuple(bias.shape) != (N,)
                             or not bias.is_cuda):
        raise TypeError("bias must be bf16 [N] on the device")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    code = DTYPE_F32 if out_dtype == torch.float32 else DTYPE_BF16
    if out is None:
        out = _empty((M, N), out_dtype, x.device, stream)
    elif out.dtype != out_dtype or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise TypeError(f"out must be contiguous {out_dtype} [M, N]")
    args = (_ptr(x), _ptr(wq), _ptr(bias), _ptr(sx), _ptr(sw), _ptr(out), code, M, N, K)
    dev = _one_device(x, wq, bias, sx, sw, out)
    if plan is None:
        rc = _launch(dev, stream, _load().skinny_gemm_fp8_quant, *args)
    else:
        rc = _launch(dev, stream, _load().skinny_gemm_fp8_quant_planned, *args, ctypes.byref(plan))
    _check(rc, f"skinny_gemm_fp8_quant(M={M}, N={N}, K={K}, {plan})")
    return out


def quant_e4m3(x, s, out=None, stream=None):
    """Static e4m3 quantisation of a contiguous bf16 device tensor with the
    one-element fp32 scale s; returns float8_e4m3fn of x's shape."""
    if not x.is_cuda or not x.is_contiguous() or x.dtype != torch.bfloat16:
        raise TypeError("x must be a contiguous bf16 device tensor")
    _scalar_f32("s", s)
    if out is None:
        out = _empty(x.shape, torch.float8_e4m3fn, x.device, stream)
    elif out.dtype not in (torch.float8_e4m3fn, torch.uint8) or out.shape != x.shape \
            or not out.is_contiguous():
        raise TypeError("out must be a contiguous float8_e4m3fn tensor of x's shape")
    rc = _launch(_one_device(x, s, out), stream, _load().skinny_quant_e4m3, _ptr(x), _ptr(s),
                 _ptr(out), x.numel())
    _check(rc, f"skinny_quant_e4m3(n={x.numel()})")
    return out


def _fp8_args(xq, wq, sx, sw, xe, we, bias, out, stream):
    """Checks FP8 operands; returns (M, N, K, Fp8Scales, out)."""
    for name, t in (("xq", xq), ("wq", wq)):
        if t.dim() != 2 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D device tensor")
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError(f"{name} must be float8_e4m3fn (or its bytes as uint8)")
    M, K = xq.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError("xq[M,K] and wq[N,K] expected")
    sc = Fp8Scales()
    if sx is not None or sw is not None:
        if xe is not None or we is not None:
            raise ValueError("give per-tensor scales (sx, sw) or MX exponents (xe, we), not both")
        for name, t in (("sx", sx), ("sw", sw)):
            if t is None or t.dtype != torch.float32 or t.numel() != 1 or not t.is_cuda:
                raise TypeError(f"{name} must be a one-element float32 device tensor")
        sc.mode, sc.sx, sc.sw = FP8_PER_TENSOR, sx.data_ptr(), sw.data_ptr()
    else:
        for name, t, rows in (("xe", xe, M), ("we", we, N)):
            if t is None or t.dtype not in (torch.uint8, torch.float8_e8m0fnu) or not t.is_cuda \
                    or not t.is_contiguous() or tuple(t.shape) != (rows, K // 32):
                raise TypeError(f"{name} must be a contiguous uint8 [{rows}, K/32] device tensor")
        sc.mode, sc.x_e8m0, sc.w_e8m0 = FP8_MX32, xe.data_ptr(), we.data_ptr()
    if bias is not None and (bias.dtype != torch.bfloat16 or tuple(bias.shape) != (N,)
                             or not bias.is_cuda):
        raise TypeError("bias must be bf16 [N] on the device")
    if out is None:
        out = _empty((M, N), torch.bfloat16, xq.device, stream)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise TypeError("out must be contiguous bf16 [M, N]")
    return M, N, K, sc, out


def gemm_fp8(xq, wq, sx=None, sw=None, xe=None, we=None, bias=None, out=None, stream=None):
    """FP8 e4m3 GEMM, bf16 out: per-tensor (sx, sw) or MX (xe, we) scales."""
    M, N, K, sc, out = _fp8_args(xq, wq, sx, sw, xe, we, bias, out, stream)
    rc = _launch(_one_device(xq, wq, sx, sw, xe, we, bias, out), stream, _load().skinny_gemm_fp8,
                 _ptr(xq), _ptr(wq), _ptr(bias), ctypes.byref(sc), _ptr(out), M, N, K)
    _check(rc, f"skinny_gemm_fp8(M={M}, N={N}, K={K}, mode={sc.mode})")
    return out


def gemm_fp8_planned(xq, wq, p, sx=None, sw=None, xe=None, we=None, bias=None, out=None,
                     stream=None):
    M, N, K, sc, out = _fp8_args(xq, wq, sx, sw, xe, we, bias, out, stream)
    rc = _launch(_one_device(xq, wq, sx, sw, xe, we, bias, out), stream,
                 _load().skinny_gemm_fp8_planned, _ptr(xq), _ptr(wq), _ptr(bias), ctypes.byref(sc),
                 _ptr(out), M, N, K, ctypes.byref(p))
    _check(rc, f"skinny_gemm_fp8_planned(M={M}, N={N}, K={K}, {p})")
    return out


def make_plan(kind, threads, cols=1, splits=1, depth=0, reduce=REDUCE_NONE, flags=0, waves_m=0,
              m_tiles=0):
    p = SkgPlan()
    p.kind, p.threads, p.cols, p.splits, p.depth, p.reduce = kind, threads, cols, splits, depth, reduce
    p.flags, p.waves_m, p.m_tiles = flags, waves_m, m_tiles
    return p


def plan(M, N, K, dtype=DTYPE_BF16):
    p = SkgPlan()
    _check(_load().skinny_gemm_plan(M, N, K, dtype, ctypes.byref(p)), "skinny_gemm_plan")
    return p


def plan_on(M, N, K, num_cus, dtype=DTYPE_BF16):
    p = SkgPlan()
    _check(_load().skinny_gemm_plan_on(M, N, K, dtype, num_cus, ctypes.byref(p)),
           "skinny_gemm_plan_on")
    return p


def plan_complete(M, N, K, p, dtype=DTYPE_BF16):
    """Completes a copy of p; raises SkinnyGemmError if it is not valid."""
    q = SkgPlan.from_buffer_copy(p)
    _check(_load().skinny_gemm_plan_complete(M, N, K, dtype, ctypes.byref(q)),
           "skinny_gemm_plan_complete")
    return q


def reserve(max_M, max_N, max_K, max_S, stream=None):
    """Reserves workspace for `stream` (else the current stream) on the
    stream's device: for calls with M <= max_M, N <= max_N, K <= max_K and
    at most max_S splits (max_K = 0: no room for gemm_fp8_quant's quantised
    x)."""
    s = torch.cuda.current_stream() if stream is None else stream
    with torch.cuda.device(s.device):
        _check(_load().skinny_gemm_reserve(max_M, max_N, max_K, max_S,
                                           ctypes.c_void_p(s.cuda_stream)),
               "skinny_gemm_reserve")


def release_all():
    _check(_load().skinny_gemm_release_all(), "skinny_gemm_release_all")
