"""The C ABI on the CPU: the library loads, exports everything its headers
declare, rejects bad arguments before any HIP call, and plans exactly.
No call here reaches the GPU (every GEMM call is one the library must
reject during host-side validation)."""
import ctypes
import os
import re

import pytest

import latency_skinny_gemm_amd as skg
from latency_skinny_gemm_amd import build as lib_build
from workloads import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(skg.library_path()):
        lib_build.build()
    return skg.lib()


def _declared(header):
    txt = open(os.path.join(ROOT, "include", header)).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(skinny_\w+)\s*\(", txt, flags=re.M))


def test_every_declared_symbol_is_exported(lib):
    names = _declared("skinny_gemm.h")
    assert {"skinny_gemm_bf16", "skinny_gemm_fp8", "skinny_gemm_plan", "skinny_gemm_reserve",
            "skinny_gemm_release_all", "skinny_gemm_status_string"} <= names
    for n in names:
        assert hasattr(lib, n), n
    floors = ctypes.CDLL(os.path.join(os.path.dirname(skg.library_path()), "libskinny_floors.so"))
    for n in _declared("skinny_floors.h"):
        assert hasattr(floors, n), n


# fake, never dereferenced device addresses (validation rejects first)
X, W, OUT, B = 0x10000, 0x200000, 0x4000000, 0x8000000


BF16_BAD_ARGS = [
    ((X, W, 0, 0, OUT, -1, 8, 64), skg.ERR_INVALID_ARG),
    ((X, W, 0, 0, OUT, 2, -8, 64), skg.ERR_INVALID_ARG),
    ((X, W, 0, 0, OUT, 2, 8, -64), skg.ERR_INVALID_ARG),
    ((X, W, 0, 0, OUT, 0, 8, 64), skg.OK),          # empty: no launch
    ((0, 0, 0, 0, 0, 5, 0, 64), skg.OK),            # empty: no launch
    ((X, W, 0, 0, OUT, 513, 8, 64), skg.ERR_UNSUPPORTED),
    ((X, W, 0, 0, OUT, 129, 8, 72), skg.ERR_UNSUPPORTED),   # > 128 rows: K % 32
    ((X, W, 0, 0, OUT, 2, 8, 60), skg.ERR_UNSUPPORTED),
    ((X, W, 0, 0, OUT, 2, 8, 0), skg.ERR_UNSUPPORTED),
    ((X, W, 0, 0, OUT, 2, 8, 4), skg.ERR_UNSUPPORTED),
    ((0, W, 0, 0, OUT, 2, 8, 64), skg.ERR_INVALID_ARG),
    ((X, 0, 0, 0, OUT, 2, 8, 64), skg.ERR_INVALID_ARG),
    ((X, W, 0, 0, 0, 2, 8, 64), skg.ERR_INVALID_ARG),
    ((X, W, 0, 0x1234, OUT, 2, 8, 64), skg.ERR_INVALID_ARG),  # scales must be NULL
    ((X + 2, W, 0, 0, OUT, 2, 8, 64), skg.ERR_ALIGNMENT),
    ((X, W + 8, 0, 0, OUT, 2, 8, 64), skg.ERR_ALIGNMENT),
    ((X, W, 0, 0, OUT + 1, 2, 8, 64), skg.ERR_ALIGNMENT),
    ((X, W, B + 1, 0, OUT, 2, 8, 64), skg.ERR_ALIGNMENT),
    ((X, W, 0, 0, X + 64, 2, 8, 64), skg.ERR_INVALID_ARG),   # out overlaps x
    ((X, W, 0, 0, W + 1000, 2, 8, 64), skg.ERR_INVALID_ARG), # out overlaps W
    ((X, W, B, 0, B - 2, 2, 8, 64), skg.ERR_INVALID_ARG),    # out overlaps bias
]


@pytest.mark.parametrize("args,status", BF16_BAD_ARGS)
def test_bf16_validation_before_any_device_call(lib, args, status):
    x, w, b, sc, o, M, N, K = args
    assert lib.skinny_gemm_bf16(x or None, w or None, b or None, sc or None, o or None,
                                M, N, K, None) == status


def test_noalloc_validates_as_skinny_gemm_bf16(lib):
    # the same host-side checks, in the same order, before any HIP call
    for args, status in BF16_BAD_ARGS:
        x, w, b, sc, o, M, N, K = args
        assert lib.skinny_gemm_bf16_noalloc(x or None, w or None, b or None, sc or None, o or None,
                                            M, N, K, None) == status, args
    # partials beyond the fixed 2^21-float array: rejected before any HIP
    # call (M = 512, N = 4096, K = 7168 plans 2 splits: 2^22 floats)
    x, w, o = 1 << 40, 2 << 40, 3 << 40
    p = skg.plan(512, 4096, 7168)
    assert p.splits * 512 * 4096 > 1 << 21
    assert lib.skinny_gemm_bf16_noalloc(x, w, None, None, o, 512, 4096, 7168, None) == \
        skg.ERR_WORKSPACE


def test_release_all_with_nothing_held_makes_no_device_call(lib):
    # no workspace was ever made in this process (no GPU here): nothing to
    # free, and no HIP call that would fail without a device
    assert lib.skinny_gemm_release_all() == skg.OK


def test_fp8_validation(lib):
    sc = skg.Fp8Scales()
    sc.mode = 7
    assert lib.skinny_gemm_fp8(X, W, None, ctypes.byref(sc), OUT, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    assert lib.skinny_gemm_fp8(X, W, None, None, OUT, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    sc.mode = skg.FP8_PER_TENSOR   # scale pointers missing
    assert lib.skinny_gemm_fp8(X, W, None, ctypes.byref(sc), OUT, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    sc.mode = skg.FP8_MX32         # exponent pointers missing
    assert lib.skinny_gemm_fp8(X, W, None, ctypes.byref(sc), OUT, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    sc.x_e8m0, sc.w_e8m0 = 0x30000, 0x40000
    assert lib.skinny_gemm_fp8(X, W, None, ctypes.byref(sc), OUT, 2, 8, 48, None) == skg.ERR_UNSUPPORTED
    assert lib.skinny_gemm_fp8(X, W, None, ctypes.byref(sc), OUT, 2, 8, 40, None) == skg.ERR_UNSUPPORTED
    assert lib.skinny_gemm_fp8(X + 8, W, None, ctypes.byref(sc), OUT, 2, 8, 64, None) == skg.ERR_ALIGNMENT
    assert lib.skinny_gemm_fp8(X, W, None, ctypes.byref(sc), X + 32, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    assert lib.skinny_gemm_fp8(X, W, None, ctypes.byref(sc), OUT, 0, 8, 64, None) == skg.OK
    sc.mode, sc.sx, sc.sw = skg.FP8_PER_TENSOR, 0x50002, 0x60000
    assert lib.skinny_gemm_fp8(X, W, None, ctypes.byref(sc), OUT, 2, 8, 64, None) == skg.ERR_ALIGNMENT


def test_bf16_f32_validation(lib):
    f = lib.skinny_gemm_bf16_f32
    assert f(X, W, None, OUT + 2, 2, 8, 64, None) == skg.ERR_ALIGNMENT       # fp32: 4-byte aligned
    assert f(X, W, None, None, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    assert f(X, W, None, X + 64, 2, 8, 64, None) == skg.ERR_INVALID_ARG      # overlaps x
    # an fp32 out is twice as long: it reaches x 16 bytes beyond a bf16 out's end
    assert f(X, W, None, X - 2 * 8 * 4 + 16, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    assert f(X, W, None, OUT, 0, 8, 64, None) == skg.OK
    assert f(X, W, None, OUT, 2, 8, 60, None) == skg.ERR_UNSUPPORTED
    assert lib.skinny_gemm_bf16_f32_planned(X, W, None, OUT, 2, 8, 64, None, None) == skg.ERR_INVALID_ARG


def test_fp8_quant_validation(lib):
    f = lib.skinny_gemm_fp8_quant
    SX, SW = 0x50000, 0x60000
    assert f(X, W, None, SX, SW, OUT, 5, 2, 8, 64, None) == skg.ERR_INVALID_ARG    # out dtype
    assert f(X, W, None, SX, SW, OUT, skg.DTYPE_FP8, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    assert f(X, W, None, None, SW, OUT, skg.DTYPE_BF16, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    assert f(X, W, None, SX, None, OUT, skg.DTYPE_BF16, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    assert f(X, W, None, SX, SW, OUT, skg.DTYPE_BF16, 2, 8, 40, None) == skg.ERR_UNSUPPORTED
    assert f(X + 8, W, None, SX, SW, OUT, skg.DTYPE_BF16, 2, 8, 64, None) == skg.ERR_ALIGNMENT
    assert f(X, W, None, SX + 2, SW, OUT, skg.DTYPE_BF16, 2, 8, 64, None) == skg.ERR_ALIGNMENT
    assert f(X, W, None, SX, SW, OUT + 2, skg.DTYPE_F32, 2, 8, 64, None) == skg.ERR_ALIGNMENT
    # x is bf16 here: 2 bytes per element, so out at x + M*K bytes still overlaps
    assert f(X, W, None, SX, SW, X + 2 * 64, skg.DTYPE_BF16, 2, 8, 64, None) == skg.ERR_INVALID_ARG
    assert f(X, W, None, SX, SW, OUT, skg.DTYPE_BF16, 0, 8, 64, None) == skg.OK
    assert lib.skinny_gemm_fp8_quant_planned(X, W, None, SX, SW, OUT, skg.DTYPE_BF16, 2, 8, 64,
                                             None, None) == skg.ERR_INVALID_ARG


def test_quant_validation(lib):
    f = lib.skinny_quant_e4m3
    S = 0x50000
    assert f(X, S, OUT, -1, None) == skg.ERR_INVALID_ARG
    assert f(X, S, OUT, 0, None) == skg.OK
    assert f(0, S, OUT, 0, None) == skg.OK
    assert f(None, S, OUT, 16, None) == skg.ERR_INVALID_ARG
    assert f(X, None, OUT, 16, None) == skg.ERR_INVALID_ARG
    assert f(X + 2, S, OUT, 16, None) == skg.ERR_ALIGNMENT
    assert f(X, S, OUT + 8, 16, None) == skg.ERR_ALIGNMENT
    assert f(X, S + 1, OUT, 16, None) == skg.ERR_ALIGNMENT
    assert f(X, S, X + 16, 16, None) == skg.ERR_INVALID_ARG   # q inside x's 32 bytes
    assert f(X, S, OUT, 1 << 31, None) == skg.ERR_UNSUPPORTED


FP8 = [p for p in configs.all_points() if p.dtype != "bf16"]


@pytest.mark.parametrize("M,N,K,NB,wm,NS,U,S", [
    (128, 4096, 4096, 8, 2, 3, 1, 8), (64, 4096, 4096, 4, 0, 4, 2, 4), (16, 4096, 4096, 8, 1, 6, 1, 4),
    (1, 1024, 4096, 16, 0, 2, 1, 2), (37, 200, 1024, 2, 4, 4, 2, 3), (128, 96, 4096, 2, 2, 3, 2, 1),
    (512, 4096, 4096, 2, 4, 3, 2, 2), (300, 200, 1024, 4, 2, 3, 1, 4)])
def test_fp8_tiled_plans_cover(lib, M, N, K, NB, wm, NS, U, S):
    p = skg.make_plan(skg.KIND_TILED, 256, NB, S, NS, skg.REDUCE_KERNEL, waves_m=wm,
                      flags=skg.FLAG_TILED_WIDE if U == 2 else 0)
    q = skg.plan_complete(M, N, K, p, skg.DTYPE_FP8)
    assert q.kind == skg.KIND_TILED
    _check_fp8_coverage(q, M, N, K)


def test_large_M_takes_tiled_plans_only(lib):
    for dt, K in ((skg.DTYPE_BF16, 7168), (skg.DTYPE_FP8, 4096)):
        for M in (129, 256, 512):
            assert skg.plan(M, 4096, K, dt).kind == skg.KIND_TILED
            with pytest.raises(skg.SkinnyGemmError):
                skg.plan_complete(M, 4096, K, skg.make_plan(skg.KIND_SPLITK, 256, 1, 4, 1), dt)
            with pytest.raises(skg.SkinnyGemmError):  # last arriver: one row block only
                skg.plan_complete(M, 4096, K, skg.make_plan(skg.KIND_TILED, 256, 4, 2, 2,
                                                            skg.REDUCE_LAST), dt)
            q = skg.plan_complete(M, 4096, K, skg.make_plan(skg.KIND_TILED, 256, 4, 2, 2), dt)
            assert q.reduce == skg.REDUCE_KERNEL and q.m_tiles == 8
    with pytest.raises(skg.SkinnyGemmError):
        skg.plan(513, 64, 1024)


def test_fp8_tiled_rejects(lib):
    with pytest.raises(skg.SkinnyGemmError):  # whole 128-wide steps only
        skg.plan_complete(16, 256, 4112, skg.make_plan(skg.KIND_TILED, 256, 4, 2, 3), skg.DTYPE_FP8)
    with pytest.raises(skg.SkinnyGemmError):  # LDS: 8 stages of 16 blocks of 4 KB
        skg.plan_complete(128, 4096, 4096, skg.make_plan(skg.KIND_TILED, 256, 8, 2, 8,
                                                         flags=skg.FLAG_TILED_WIDE), skg.DTYPE_FP8)


def _fp8_dtype(p):
    return skg.DTYPE_FP8_MX if p.dtype == "fp8_mx" else skg.DTYPE_FP8


@pytest.mark.parametrize("p", FP8, ids=lambda p: p.key())
def test_fp8_plans_valid_and_cover(lib, p):
    dt = _fp8_dtype(p)
    q = skg.plan(p.M, p.N, p.K, dt)
    again = skg.plan_complete(p.M, p.N, p.K, q, dt)
    assert (again.kind, again.grid, again.splits, again.k_chunk) == (q.kind, q.grid, q.splits, q.k_chunk)
    _check_fp8_coverage(q, p.M, p.N, p.K, dt == skg.DTYPE_FP8_MX)
    if p.group.startswith("fp8_"):  # the swept FP8 points: one table entry per scale mode
        assert q.from_table == 1, p.key()


def test_fp8_mx_planning_dtype(lib):
    # the same kernels and limits as per-tensor FP8, K % 32 == 0, and its own
    # table entries (at M = 1 the two modes are fastest with different plans)
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.plan(4, 256, 4112, skg.DTYPE_FP8_MX)
    assert e.value.status == skg.ERR_UNSUPPORTED
    assert skg.plan(4, 256, 4112, skg.DTYPE_FP8).kind in (skg.KIND_DOT, skg.KIND_SPLITK)
    for kind, T, NB, S, D in ((skg.KIND_DOT, 256, 1, 1, 0), (skg.KIND_SPLITK, 256, 1, 4, 2),
                              (skg.KIND_TILED, 256, 4, 2, 3)):
        a = skg.plan_complete(16, 4096, 4096, skg.make_plan(kind, T, NB, S, D, skg.REDUCE_KERNEL if S > 1
                                                            else skg.REDUCE_NONE), skg.DTYPE_FP8)
        b = skg.plan_complete(16, 4096, 4096, skg.make_plan(kind, T, NB, S, D, skg.REDUCE_KERNEL if S > 1
                                                            else skg.REDUCE_NONE), skg.DTYPE_FP8_MX)
        assert a.as_dict() == b.as_dict()
    t = skg.plan(1, 4096, 4096, skg.DTYPE_FP8)
    m = skg.plan(1, 4096, 4096, skg.DTYPE_FP8_MX)
    assert t.from_table == m.from_table == 1
    assert (t.kind, t.threads, t.depth) != (m.kind, m.threads, m.depth)
    # off the table both fall back to the same rule
    assert skg.plan(16, 4096, 2048, skg.DTYPE_FP8).as_dict() == \
        skg.plan(16, 4096, 2048, skg.DTYPE_FP8_MX).as_dict()


def _tiled_position(b, MB, S, G):
    """The tiled kernels' workgroup -> (row block, K chunk, column group)."""
    if MB > 1 and G % 8 == 0:
        q, r = divmod(b, 8 * MB)
        mb, sj = r // 8, q * 8 + r % 8
    else:
        mb, sj = b % MB, b // MB
    return mb, sj % S, sj // S


def _check_fp8_tiled_coverage(p, M, N, K):
    S, NB, NS, kc, WM = p.splits, p.cols, p.depth, p.k_chunk, p.waves_m
    U = 2 if p.flags & skg.FLAG_TILED_WIDE else 1
    WN = 4 // WM
    natural = next((v for v in (1, 2, 4, 8) if v >= -(-M // 16)), 8)
    MT = p.m_tiles  # the rows' own power of two, or a smaller one (row blocks)
    assert MT in (1, 2, 4, 8) and MT <= natural and MT % WM == 0 and NB % WN == 0
    assert p.threads == 256 and K % 128 == 0 and kc % 128 == 0 and (S - 1) * kc < K <= S * kc
    groups = -(-N // (16 * NB))
    MB = -(-M // (MT * 16))
    assert MB == 1 or S == 1 or p.reduce != skg.REDUCE_LAST
    rows = sorted(mb * MT * 16 + r for mb in range(MB) for r in range(min(MT * 16, M - mb * MT * 16)))
    assert rows == list(range(M))
    assert p.grid == MB * groups * S
    dec = [_tiled_position(b, MB, S, p.grid // MB) for b in range(p.grid)]
    assert sorted(dec) == sorted((mb, s, j) for mb in range(MB) for s in range(S) for j in range(groups))
    CPR = 8 * U

    def swz(r):
        return (r // (16 // CPR)) & (CPR - 1)

    # a block: 16 rows x CPR chunks; part i of 2U fills positions 64i..64i+63
    stored = {}
    for part in range(2 * U):
        for lane in range(64):
            lin = part * 64 + lane
            r, c = lin // CPR, (lin % CPR) ^ swz(lin // CPR)
            assert (r, c) not in stored
            stored[(r, c)] = lin
    assert sorted(stored) == [(r, c) for r in range(16) for c in range(CPR)]
    # the MFMA operand of lane l in step u: row l % 16, K offsets 16g and
    # 64 + 16g of the step (g = l // 16) = chunks 8u + g and 8u + 4 + g
    for u in range(U):
        for g in range(4):
            for c in (8 * u + g, 8 * u + 4 + g):
                assert 16 * c in (128 * u + 16 * g, 128 * u + 64 + 16 * g)
                pos = [stored[(r, c)] for r in range(16)]
                assert len({(q * 16 % 256) // 16 for q in pos}) == 16   # 16 bank groups
    # MX scales: wave w's load, lane p -> row (64/U) w + p // U, dword p % U,
    # LDS byte 256 w + 4 p = row * 4U + 4 * dword; lane l of step u reads byte
    # row * 4U + 4u + g, the exponent of block 4u + g of the stage
    for tiles in (MT, NB):
        rows = tiles * 16
        nload = -(-(rows * 4 * U) // 256)
        assert nload <= 4
        seen_rows = {}
        for w in range(nload):
            for lane in range(64):
                row, dw = (64 // U) * w + lane // U, lane % U
                assert 256 * w + 4 * lane == row * 4 * U + 4 * dw
                seen_rows.setdefault(row, set()).add(dw)
        assert all(seen_rows.get(r) == set(range(U)) for r in range(rows))
        for u in range(U):
            for g in range(4):
                assert (4 * u + g) * 32 == 128 * u + 32 * g
    # every K of every split computed once (rotation a permutation)
    for j in range(groups):
        for s in range(S):
            nst = -(-((min(K, (s + 1) * kc) - s * kc) // 128) // U)
            assert sorted((st + j % nst) % nst for st in range(nst)) == list(range(nst))
    seen = [0] * K
    for s in range(S):
        kbeg = s * kc
        nsteps = (min(K, kbeg + kc) - kbeg) // 128
        for st in range(-(-nsteps // U)):
            for u in range(U):
                if st * U + u < nsteps:
                    for kk in range(128):
                        seen[kbeg + (st * U + u) * 128 + kk] += 1
    assert seen == [1] * K
    XPW, WPW = -(-(MT * 2 * U) // 4), -(-(NB * 2 * U) // 4)
    assert (NS - 2) * (XPW + WPW + 2) < 64


def _check_fp8_rows_coverage(p, M, N, K, mx):
    # the FP8 whole-row ring: stages of SB K (1 byte each); a load fills
    # 1 KB (row j*RPL + p/CPR, position p%CPR holding chunk (p%CPR) ^ (LDS
    # row % 16)); MX: wave w < WSL loads W scale rows RPS*w.., the next XSL
    # waves the x ones (lane p: row p/CS, chunk p%CS); MFMA step u (128 K)
    # reads chunks 8u + g and 8u + 4 + g and scale byte 4u + g
    R, NW, NS = p.cols, p.threads // 64, p.depth
    SB = 512 if p.flags & skg.FLAG_ROWS_HALF else 1024
    MP = next(v for v in (1, 2, 4, 8, 16, 32) if v >= M)
    CPR, RPL = SB // 16, 1024 // SB
    XR = -(-MP // RPL) * RPL
    SPR = SB // 32
    CS = SPR // 16
    RPS = 64 // CS
    WSL, XSL = -(-R // RPS), -(-XR // RPS)
    assert R in (8, 16) and NW in (4, 8) and 3 <= NS <= 6 and M <= 32 and p.splits == 1
    assert (SB // 128) % NW == 0 and p.grid == -(-N // R)
    assert sorted(n for b in range(p.grid) for c in range(R) if (n := b * R + c) < N) == list(range(N))
    wl, xl = R // RPL, XR // RPL
    lpw = -(-wl // NW) + -(-xl // NW) + 1  # the MX layout, which every plan must fit
    stage = (R + XR) * SB + 1024 + (WSL + XSL) * 1024
    assert NS * stage <= 160 * 1024 - 256 and (NS - 2) * lpw < 64 and WSL + XSL <= NW
    for blk_rows, nl, base in ((R, wl, 0), (XR, xl, R)):
        filled = {}
        for j in range(nl):
            for l in range(64):
                r, pos = j * RPL + l // CPR, l % CPR
                key = (r, pos ^ ((base + r) & 15))
                filled[key] = filled.get(key, 0) + 1
        assert filled == {(r, c): 1 for r in range(blk_rows) for c in range(CPR)}
    # scale loads: every (row, 16-byte chunk) of each operand's stage scales once
    for rows, nsl in ((R, WSL), (XR, XSL)):
        got = sorted((i * RPS + l // CS, l % CS) for i in range(nsl) for l in range(64)
                     if i * RPS + l // CS < rows)
        assert got == [(r, c) for r in range(rows) for c in range(CS)]
    # operand chunks of a 128-K step: lane group g takes bytes [16g, 16g+16)
    # and [64+16g, 64+16g+16); every byte of the stage once over the steps
    bytes_ = sorted(128 * u + 16 * c + e for u in range(SB // 128) for g in range(4)
                    for c in (g, 4 + g) for e in range(16))
    assert bytes_ == list(range(SB))
    if mx:
        assert K % 512 == 0
    nst = -(-K // SB)
    steps = sorted(w + NW * q for w in range(NW) for q in range(SB // 128 // NW))
    assert steps == list(range(SB // 128)) and nst * SB >= K


def _check_fp8_coverage(p, M, N, K, mx=False):
    if p.kind == skg.KIND_ROWS:
        _check_fp8_rows_coverage(p, M, N, K, mx)
        return
    if p.kind == skg.KIND_TILED:
        _check_fp8_tiled_coverage(p, M, N, K)
        return
    if p.kind == skg.KIND_DOT:
        T, V = p.threads, p.depth
        K16 = K // 16
        vecs = sorted(t + i * T for t in range(T) for i in range(V) if t + i * T < K16)
        assert vecs == list(range(K16)) and p.cols in (1, 2, 4)
        C = p.cols
        assert p.grid == -(-N // C)
        cols = [n for b in range(p.grid) for c in range(C) if (n := b * C + c) < N]
        assert cols == list(range(N))
        # the cross-wave sums for C * M outputs fit in one pass of the threads
        assert C * M <= T
        return
    assert p.kind == skg.KIND_SPLITK
    S, NB, D, kc = p.splits, p.cols, p.depth, p.k_chunk
    nw = p.threads // 64
    assert kc % 128 == 0 and (S - 1) * kc < K <= S * kc and p.grid == -(-N // (16 * NB)) * S
    seen = [0] * K
    for s in range(S):
        kbeg, kend = s * kc, min(K, (s + 1) * kc)
        nsteps = -(-(kend - kbeg) // 128)
        spw = -(-nsteps // nw)
        for w in range(nw):
            first = w * spw
            my = max(0, min(spw, nsteps - first))
            nch = -(-my // D)
            consumed = [0] if nch <= 1 else [c for c0 in range(0, nch, 2) for c in (c0, c0 + 1)]
            for ch in consumed:
                for d in range(D):
                    i = ch * D + d
                    for g in range(4):      # lane group g: chunks at 16g and 64 + 16g
                        k0 = kbeg + (first + i) * 128
                        for kk0 in (k0 + 16 * g, k0 + 64 + 16 * g):
                            if i < my and kk0 < kend:
                                for kk in range(kk0, kk0 + 16):
                                    seen[kk] += 1
    assert seen == [1] * K


@pytest.mark.parametrize("M,N,K,T,C", [
    (1, 4096, 4096, 256, 2), (1, 4097, 4096, 256, 4), (16, 4096, 4096, 512, 4), (3, 5, 4112, 256, 4),
    (8, 2, 7168, 1024, 2)])
def test_fp8_dot_columns_cover(lib, M, N, K, T, C):
    try:
        q = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_DOT, T, C), skg.DTYPE_FP8)
    except skg.SkinnyGemmError:
        # only a register budget may refuse: one column fits where C does not
        skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_DOT, min(T, 512), 1), skg.DTYPE_FP8)
        return
    _check_fp8_coverage(q, M, N, K)


def test_fp8_dot_column_counts(lib):
    with pytest.raises(skg.SkinnyGemmError):
        skg.plan_complete(1, 4096, 4096, skg.make_plan(skg.KIND_DOT, 256, 3), skg.DTYPE_FP8)
    q = skg.plan_complete(1, 4097, 4096, skg.make_plan(skg.KIND_DOT, 256, 4), skg.DTYPE_FP8)
    assert q.grid == 1025 and q.cols == 4


def test_fp8_straddling_K_covered(lib):
    # per-tensor K = 4112 ends halfway through a 32-element block
    for kind, T, NB, S, D in ((skg.KIND_SPLITK, 256, 1, 3, 2), (skg.KIND_SPLITK, 128, 2, 1, 4)):
        q = skg.plan_complete(5, 48, 4112, skg.make_plan(kind, T, NB, S, D, skg.REDUCE_LAST), skg.DTYPE_FP8)
        _check_fp8_coverage(q, 5, 48, 4112)


def test_status_strings(lib):
    for st in (skg.OK, skg.ERR_INVALID_ARG, skg.ERR_ALIGNMENT, skg.ERR_UNSUPPORTED,
               skg.ERR_WORKSPACE, skg.ERR_HIP):
        assert skg.status_string(st).startswith("SKG_")
    assert skg.status_string(-99) == "SKG_ERR_UNKNOWN"


def test_reserve_rejects_bad_sizes(lib):
    assert lib.skinny_gemm_reserve(0, 10, 64, 1, None) == skg.ERR_INVALID_ARG
    assert lib.skinny_gemm_reserve(513, 10, 64, 1, None) == skg.ERR_INVALID_ARG
    assert lib.skinny_gemm_reserve(4, 10, 64, 10000, None) == skg.ERR_INVALID_ARG
    assert lib.skinny_gemm_reserve(4, 10, 64, 257, None) == skg.ERR_INVALID_ARG
    assert lib.skinny_gemm_reserve(4, 0, 64, 1, None) == skg.ERR_INVALID_ARG
    assert lib.skinny_gemm_reserve(4, 10, -1, 1, None) == skg.ERR_INVALID_ARG
    # 512 rows of 2-byte x at this K would pass 2 GiB
    assert lib.skinny_gemm_reserve(4, 10, (1 << 21), 1, None) == skg.ERR_INVALID_ARG


# ------------------------------------------------------------------ planner

BF16 = [p for p in configs.all_points() if p.dtype == "bf16"]


@pytest.mark.parametrize("p", BF16, ids=lambda p: p.key())
def test_default_rule_without_table(lib, p):
    # a made-up 200-CU device never uses the MI355X table: the pages' rule
    # (dot product for M <= 4 or K < 2048, here also up to 16 rows at
    # N <= 512 with x of at most 192 KB), then the whole-row ring from 5 to
    # 32 rows, else the tiled kernel (split-K only where K is not a multiple
    # of 32)
    q = skg.plan_on(p.M, p.N, p.K, 200)
    if p.M > 128:
        want = skg.KIND_TILED  # above 128 rows only the tiled kernel runs
    elif p.M <= 4 or p.K < 2048 or (p.M <= 16 and p.N <= 512 and p.M * p.K <= 98304):
        want = skg.KIND_DOT
    elif p.M <= 16 and p.N > 512 and 2 * -(-p.N // 8) < 200:
        want = skg.KIND_DOT  # between N = 512 and the whole-row ring: 3 or 4 columns
    elif p.M <= 32 and 2 * -(-p.N // 8) >= 200 and p.M * p.K <= 114688:
        want = skg.KIND_ROWS  # the whole-row ring: 8-column groups fill half the CUs, x <= 224 KB
    else:
        want = skg.KIND_TILED if p.K % 32 == 0 else skg.KIND_SPLITK
    assert q.kind == want and q.from_table == 0
    _check_coverage(q, p.M, p.N, p.K)
    if q.kind == skg.KIND_DOT and p.M >= 5 and p.N > 512 and p.K >= 2048:
        # the band below the ring: 4 columns while N / 4 groups cover three
        # quarters of the CUs, else 3
        assert q.cols == (4 if 4 * -(-p.N // 4) >= 600 else 3), q
    elif q.kind == skg.KIND_DOT:
        # the most columns per workgroup that leave two workgroups per CU
        c = next(c for c in (4, 2, 1) if c == 1 or -(-p.N // c) >= 400)
        assert q.cols == c, (q.cols, c)
    if q.kind == skg.KIND_DOT:
        # the dot instruction, and the W-first load order from 8 rows
        assert q.flags == skg.FLAG_DOT2 | (skg.FLAG_DOT_WFIRST if p.M >= 8 else 0)


@pytest.mark.parametrize("p", BF16, ids=lambda p: p.key())
def test_library_plan_is_valid_and_covers(lib, p):
    q = skg.plan(p.M, p.N, p.K)
    again = skg.plan_complete(p.M, p.N, p.K, q)
    for f in ("kind", "threads", "cols", "splits", "depth", "reduce", "k_chunk", "grid"):
        assert getattr(again, f) == getattr(q, f), f
    _check_coverage(q, p.M, p.N, p.K)


def test_default_rule_details(lib):
    # bf16 dot plans: the dot instruction (W first from 8 rows), two vectors
    # per thread above 4 rows, and 4 (else 2) columns while two workgroups
    # per CU remain
    wfirst = skg.FLAG_DOT2 | skg.FLAG_DOT_WFIRST
    q = skg.plan_on(12, 256, 6144, 255)
    assert (q.kind, q.flags, q.depth, q.cols) == (skg.KIND_DOT, wfirst, 2, 1)
    assert q.threads == 384
    assert skg.plan_on(7, 256, 6144, 255).flags == skg.FLAG_DOT2
    assert skg.plan_on(8, 256, 6144, 255).flags == wfirst
    assert skg.plan_on(4, 4096, 7168, 255).flags == skg.FLAG_DOT2
    q = skg.plan_on(2, 4096, 7168, 255)
    assert (q.kind, q.cols) == (skg.KIND_DOT, 4) and q.grid == 1024
    q = skg.plan_on(2, 768, 7168, 255)
    assert (q.kind, q.cols) == (skg.KIND_DOT, 1)  # 2 columns would leave 384 < 510 workgroups
    # past the x bound of the small-N rule: the tiled kernel
    assert skg.plan_on(16, 512, 7168, 255).kind == skg.KIND_TILED
    # bf16 from 5 to 32 rows: the whole-row ring when its 8-column groups
    # fill half the CUs and M * K <= 114688 (x <= 224 KB); columns 8, 12 (up
    # to 16 rows) or 16, the fewest on the busiest CU (tie: 8 up to 8 rows,
    # else the most); half-width stages with two groups per CU or above 16
    # rows.  Off-table shapes at 256 CUs take the rule too.
    def ring(M, N, K, cus):
        q = skg.plan_on(M, N, K, cus)
        assert q.kind == skg.KIND_ROWS and (q.threads, q.depth) == (256, 4) and q.from_table == 0, q
        return q.cols, q.flags
    half = skg.FLAG_ROWS_HALF
    assert ring(8, 4096, 4096, 256) == (8, half)      # tie 8/16, two groups per CU
    assert ring(16, 4096, 4096, 256) == (16, 0)       # tie above 8 rows, one per CU
    assert ring(12, 3072, 5120, 256) == (12, 0)       # 12 columns fill the CUs once
    assert ring(16, 4096, 7168, 256) == (16, 0)       # M * K = 114688: at the bound
    assert ring(24, 2048, 4096, 256) == (8, half)     # above 16 rows: no 12, half-width
    assert ring(8, 4096, 4096, 255) == (8, half)      # 24 columns on the busiest CU, as 12
    assert skg.plan_on(20, 4096, 7168, 256).kind == skg.KIND_TILED  # x 280 KB
    assert skg.plan_on(33, 4096, 2048, 256).kind == skg.KIND_TILED  # past 32 rows
    # below that, from 5 to 16 rows above N = 512: the dot kernel with 4
    # columns while N / 4 groups cover three quarters of the CUs, else 3,
    # and one 16-byte vector of K per thread where the registers allow
    q = skg.plan_on(8, 768, 4096, 256)
    assert (q.kind, q.cols, q.threads, q.flags) == (skg.KIND_DOT, 4, 512, wfirst)
    assert skg.plan_on(6, 640, 3072, 256).flags == skg.FLAG_DOT2
    q = skg.plan_on(10, 704, 6144, 256)
    assert (q.kind, q.cols, q.threads) == (skg.KIND_DOT, 3, 768)
    q = skg.plan_on(12, 768, 7168, 256)
    assert (q.kind, q.cols, q.threads) == (skg.KIND_DOT, 4, 448)  # two vectors: registers
    assert skg.plan_on(24, 768, 4096, 256).kind == skg.KIND_TILED  # past 16 rows
    assert skg.plan_on(12, 512, 7168, 255).kind == skg.KIND_DOT
    # FP8 from 3 to 32 rows: the whole-row ring when the 8-column groups
    # reach a quarter of the CUs (all of them at 3-4 rows, else the dot
    # kernel). Columns: the fewer on the busiest CU, on a tie 8 up to 8 rows
    # with at most two groups per CU, else 16. Half-width stages with two
    # groups per CU or above 8 rows; 3 stages with three groups per CU or
    # two 16-column groups
    def ring(M, N, K, dt=skg.DTYPE_FP8, cus=256):
        q = skg.plan_on(M, N, K, cus, dt)
        assert q.kind == skg.KIND_ROWS and q.threads == 256, q
        return q.cols, q.depth, q.flags, q.grid
    half = skg.FLAG_ROWS_HALF
    assert ring(8, 4096, 4096) == (8, 4, half, 512)           # tie, two per CU
    assert ring(4, 4096, 4096, skg.DTYPE_FP8_MX) == (8, 4, half, 512)
    assert ring(4, 7168, 2048) == (16, 3, half, 448)          # tie, 896 groups of 8
    assert ring(32, 4096, 4096) == (16, 4, half, 256)         # tie above 8 rows
    assert ring(32, 2048, 7168) == (8, 4, half, 256)          # 16 columns idle half
    assert ring(6, 5120, 3072) == (8, 3, half, 640)           # 3 groups per CU
    assert ring(8, 1536, 4096) == (8, 4, 0, 192)              # one group per CU
    assert ring(3, 2048, 7168) == (8, 4, 0, 256)
    assert ring(8, 512, 4096) == (8, 4, 0, 64)                # a quarter of the CUs
    assert ring(24, 8192, 4096) == (16, 3, half, 512)           # tie above 8 rows
    assert ring(24, 8192, 4096, cus=255) == (8, 3, half, 1024)  # 40 columns against 48
    q = skg.plan_on(4, 1024, 4096, 256, skg.DTYPE_FP8)        # 128 groups: dot
    assert (q.kind, q.cols) == (skg.KIND_DOT, 1)
    q = skg.plan_on(2, 4096, 4096, 255, skg.DTYPE_FP8)
    assert (q.kind, q.cols) == (skg.KIND_DOT, 1)
    assert skg.plan_on(33, 4096, 4096, 255, skg.DTYPE_FP8).kind == skg.KIND_TILED
    # below a quarter of the CUs: from 5 rows tiled, split-K for K % 128 != 0
    assert skg.plan_on(12, 256, 4096, 256, skg.DTYPE_FP8).kind == skg.KIND_TILED
    assert skg.plan_on(24, 256, 4112, 256, skg.DTYPE_FP8).kind == skg.KIND_SPLITK
    # the ring takes any K per tensor; MX needs K % 512 == 0, else from 5
    # to 16 rows split-K without a K split where its 16-column groups fill
    # half the CUs
    assert skg.plan_on(16, 4096, 4128, 255, skg.DTYPE_FP8).kind == skg.KIND_ROWS
    q = skg.plan_on(16, 4096, 4128, 255, skg.DTYPE_FP8_MX)
    assert (q.kind, q.splits) == (skg.KIND_SPLITK, 1)


def test_split_count_follows_cu_count(lib):
    # the default rule (no table below 256 CUs) sizes the grid to the device
    # (40 rows: past the whole-row ring's 32)
    for K, kind in ((7168, skg.KIND_TILED), (7176, skg.KIND_SPLITK)):
        small = skg.plan_on(40, 1024, K, 64)
        big = skg.plan_on(40, 1024, K, 200)
        assert small.kind == big.kind == kind and small.from_table == big.from_table == 0
        assert small.splits < big.splits
        assert small.grid >= 48 and big.grid >= 150


def test_table_entries_are_exact_and_valid(lib):
    # every table entry is returned for its exact (M, N, K) at 256 CUs, and
    # its completed plan covers the problem
    for p in BF16:
        if p.group == "larger_m":  # parity points, not swept
            continue
        q = skg.plan(p.M, p.N, p.K)
        assert q.from_table == 1, p.key()
        _check_coverage(q, p.M, p.N, p.K)
    # a shape outside the table falls back to the rule
    assert skg.plan(8, 320, 7168).from_table == 0


@pytest.mark.parametrize("plan,M,N,K", [
    (dict(kind=9, threads=256), 4, 256, 2048),
    (dict(kind=skg.KIND_DOT, threads=100), 4, 256, 2048),
    (dict(kind=skg.KIND_DOT, threads=2048), 4, 256, 2048),
    (dict(kind=skg.KIND_DOT, threads=256, cols=5), 4, 256, 2048),
    (dict(kind=skg.KIND_DOT, threads=64), 4, 256, 7168),        # > 8 vectors a thread
    (dict(kind=skg.KIND_DOT, threads=256), 17, 256, 2048),      # DOT is built for M <= 16
    (dict(kind=skg.KIND_DOT, threads=1024), 16, 256, 7168),     # registers at 1024 threads
    (dict(kind=skg.KIND_SPLITK, threads=256, cols=3, splits=2, depth=2), 4, 256, 2048),
    (dict(kind=skg.KIND_SPLITK, threads=256, cols=1, splits=2, depth=3), 4, 256, 2048),
    (dict(kind=skg.KIND_SPLITK, threads=256, cols=1, splits=0, depth=2), 4, 256, 2048),
    (dict(kind=skg.KIND_SPLITK, threads=256, cols=1, splits=300, depth=2), 4, 256, 2048),
    (dict(kind=skg.KIND_SPLITK, threads=512, cols=4, splits=2, depth=2), 128, 256, 2048),
    (dict(kind=skg.KIND_SPLITK, threads=256, cols=1, splits=2, depth=2, reduce=5), 4, 256, 2048),
])
def test_complete_rejects_invalid_plans(lib, plan, M, N, K):
    p = skg.make_plan(**plan)
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.plan_complete(M, N, K, p)
    assert e.value.status == skg.ERR_INVALID_ARG


def test_launch_size_limits(lib):
    # the output plane is indexed by int: M * N < 2^31, else unsupported
    p = skg.SkgPlan()
    assert lib.skinny_gemm_plan(2, 1 << 30, 64, skg.DTYPE_BF16, ctypes.byref(p)) == \
        skg.ERR_UNSUPPORTED
    # within that domain the automatic planner refuses what no plan can launch
    assert lib.skinny_gemm_plan(1, (1 << 31) - 1, 64, skg.DTYPE_BF16, ctypes.byref(p)) == \
        skg.ERR_UNSUPPORTED
    q = skg.plan(1, 1 << 24, 64)
    assert q.grid * q.threads < (1 << 32)
    # grid * threads is a 32-bit work-item count: 2^26 one-wave workgroups
    # of 64 threads reach 2^32 and are refused; one fewer column fits
    n = 1 << 26
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.plan_complete(1, n, 64, skg.make_plan(skg.KIND_DOT, 64, 1))
    assert e.value.status == skg.ERR_INVALID_ARG
    assert skg.plan_complete(1, n - 1, 64, skg.make_plan(skg.KIND_DOT, 64, 1)).grid == n - 1
    assert skg.plan_complete(1, n, 64, skg.make_plan(skg.KIND_DOT, 64, 2)).grid == n // 2
    with pytest.raises(skg.SkinnyGemmError):
        skg.plan_complete(1, n, 128, skg.make_plan(skg.KIND_DOT, 64, 1), skg.DTYPE_FP8)
    # split plans multiply the column groups by the splits
    with pytest.raises(skg.SkinnyGemmError):
        skg.plan_complete(8, 1 << 24, 2048, skg.make_plan(skg.KIND_SPLITK, 256, 1, 64, 2,
                                                          skg.REDUCE_KERNEL))
    assert skg.plan_complete(8, 1 << 16, 2048, skg.make_plan(skg.KIND_SPLITK, 256, 1, 64, 2,
                                                             skg.REDUCE_KERNEL)).grid == 4096 * 64


def test_complete_drops_empty_splits(lib):
    # K = 2880 has 90 steps of 32; 64 splits of ceil(90/64) = 2 steps leave
    # only 45 non-empty splits
    q = skg.plan_complete(16, 128, 2880, skg.make_plan(skg.KIND_SPLITK, 256, 1, 64, 2, skg.REDUCE_LAST))
    assert q.splits == 45 and q.k_chunk == 64 and q.grid == 8 * 45
    q = skg.plan_complete(16, 128, 2880, skg.make_plan(skg.KIND_SPLITK, 256, 1, 1, 2, skg.REDUCE_LAST))
    assert q.reduce == skg.REDUCE_NONE


# ------------------------------------------------------------------ coverage
# A model of the kernels' index arithmetic: every output written exactly
# once, and every k of every output accumulated exactly once.

def _check_xlds_coverage(p, M, N, K):
    # waves of CW columns over the whole K: lane l takes vectors l + 64 i;
    # x is copied to LDS by waves in 64-chunk runs q0 = 64 w + j T
    T, C, V = p.threads, p.cols, p.depth
    nw = T // 64
    CW = C // nw
    K8 = K // 8
    assert C == CW * nw and CW in (1, 2, 4) and V * 64 == K8 and p.grid == -(-N // C)
    cols = [n for b in range(p.grid) for w in range(nw) for c in range(CW)
            if (n := (b * nw + w) * CW + c) < N]
    assert sorted(cols) == list(range(N))
    assert sorted(l + 64 * i for l in range(64) for i in range(V)) == list(range(K8))
    chunks = sorted(q0 + l for w in range(nw) for q0 in range(64 * w, M * K8, T) for l in range(64))
    assert chunks == list(range(M * K8)) and M * K8 * 16 <= 160 * 1024 - 256


def _check_rows_coverage(p, M, N, K):
    # whole-row MFMA ring: workgroup b owns columns R*b ..; stages of KS K
    # walked in rotated order; a load instruction fills 1 KB: row j*RPL +
    # p/CPR, position p%CPR holding chunk (p%CPR) ^ (LDS row % 16); wave w of
    # NW issues instructions w + NW i of each block and multiplies MFMA steps
    # w, w + NW, ... (32 K each, lane group g = l / 16 reads chunk 4u + g at
    # position (4u + g) ^ (row % 16))
    R, NW, NS = p.cols, p.threads // 64, p.depth
    KS = 256 if p.flags & skg.FLAG_ROWS_HALF else 512
    MP = M if M <= 16 else next(v for v in (24, 32, 48, 64) if v >= M)
    CPR, RPL = KS // 8, 1024 // (2 * KS)
    XR = -(-MP // RPL) * RPL
    assert (R in (8, 16) or (R in (10, 12) and M <= 16)) and NW in (4, 8) and 3 <= NS <= 6
    assert M <= 64 and p.splits == 1 and p.grid == -(-N // R)
    cols = sorted(n for b in range(p.grid) for c in range(R) if (n := b * R + c) < N)
    assert cols == list(range(N))
    wl, xl = R // RPL, XR // RPL
    wpw, xpw = -(-wl // NW), -(-xl // NW)
    stage = (R + XR) * 2 * KS + 1024
    assert NS * stage <= 160 * 1024 - 256 and (NS - 2) * (wpw + xpw) < 64
    assert NW * (-(-MP // 16)) * 16 * 17 * 4 <= NS * stage
    # every (LDS row, chunk) of a stage is filled exactly once, from that row's chunk
    for blk_rows, nl, npw in ((R, wl, wpw), (XR, xl, xpw)):
        filled = {}
        for w in range(NW):
            for i in range(npw):
                j = w + NW * i
                if j >= nl:
                    continue
                for l in range(64):
                    r, pos = j * RPL + l // CPR, l % CPR
                    row = r if blk_rows == R else R + r
                    filled[(r, pos ^ (row & 15))] = filled.get((r, pos ^ (row & 15)), 0) + 1
        assert filled == {(r, c): 1 for r in range(blk_rows) for c in range(CPR)}
    # fragment reads of a step land on the chunk the MFMA step needs, and the
    # 16 rows of one lane group hit 16 distinct 16-byte bank groups
    for u in range(KS // 32):
        for g in range(4):
            kc = 4 * u + g
            banks = {(r * 2 * KS // 16 + (kc ^ (r & 15))) % 16 for r in range(16)}
            assert len(banks) == 16 and all((kc ^ (r & 15)) < CPR for r in range(R + XR))
    nst = -(-K // KS)
    for b in {0, p.grid - 1, p.grid // 2}:
        rot = b % nst
        order = [(st + rot) % nst for st in range(nst)]
        assert sorted(order) == list(range(nst))
        steps = sorted(w + NW * q for w in range(NW) for q in range(KS // 32 // NW))
        assert steps == list(range(KS // 32))
        mult = sorted(KS * pos + 32 * u + 8 * g + e for pos in order for u in steps
                      for g in range(4) for e in range(8))
        assert mult == list(range(KS * nst))  # past K: zeros from the range check


def _check_coverage(p, M, N, K):
    if p.kind == skg.KIND_ROWS:
        _check_rows_coverage(p, M, N, K)
        return
    if p.kind == skg.KIND_DOT and p.flags & skg.FLAG_DOT_XLDS:
        _check_xlds_coverage(p, M, N, K)
        return
    if p.kind == skg.KIND_DOT:
        T, C, V = p.threads, p.cols, p.depth
        K8 = K // 8
        cols = [n for b in range(p.grid) for c in range(C) if (n := b * C + c) < N]
        assert sorted(cols) == list(range(N))
        vecs = sorted(t + i * T for t in range(T) for i in range(V) if t + i * T < K8)
        assert vecs == list(range(K8))
        assert T % 64 == 0 and T <= 1024 and p.grid == -(-N // C)
        return
    if p.kind == skg.KIND_TILED:
        _check_tiled_coverage(p, M, N, K)
        return
    assert p.kind == skg.KIND_SPLITK
    S, NB, D, kc = p.splits, p.cols, p.depth, p.k_chunk
    nw = p.threads // 64
    groups = -(-N // (16 * NB))
    assert p.grid == groups * S and kc % 32 == 0 and (S - 1) * kc < K <= S * kc
    # columns: tile j covers [16*NB*j, 16*NB*(j+1)) clipped to N
    cols = sorted(n for j in range(groups) for c in range(16 * NB) if (n := 16 * NB * j + c) < N)
    assert cols == list(range(N))
    # K: per split, the waves' steps, the two-stage chunk schedule, lane groups
    seen = [0] * K
    for s in range(S):
        kbeg, kend = s * kc, min(K, (s + 1) * kc)
        nsteps = -(-(kend - kbeg) // 32)
        spw = -(-nsteps // nw)
        for w in range(nw):
            first = w * spw
            my = max(0, min(spw, nsteps - first))
            nch = -(-my // D)
            consumed = [0] if nch <= 1 else [c for c0 in range(0, nch, 2) for c in (c0, c0 + 1)]
            for ch in consumed:
                for d in range(D):
                    i = ch * D + d
                    for g in range(4):  # lane groups of 16: k offset 8*g
                        k = kbeg + (first + i) * 32 + 8 * g
                        if i < my and k < kend:
                            for kk in range(k, k + 8):
                                seen[kk] += 1
    assert seen == [1] * K


def _check_tiled_coverage(p, M, N, K):
    S, NB, NS, kc, WM = p.splits, p.cols, p.depth, p.k_chunk, p.waves_m
    U = 4 if p.flags & skg.FLAG_TILED_WIDE else 2
    WN = 4 // WM
    natural = next((v for v in (1, 2, 4, 8) if v >= -(-M // 16)), 8)
    MT = p.m_tiles  # the rows' own power of two, or a smaller one (row blocks)
    assert MT in (1, 2, 4, 8) and MT <= natural and MT % WM == 0 and NB % WN == 0
    MTW, NBW = MT // WM, NB // WN
    assert p.threads == 256 and K % 32 == 0
    groups = -(-N // (16 * NB))
    MB = -(-M // (MT * 16))   # row blocks: above 128 rows, or fewer m-tiles asked for
    assert MB == 1 or S == 1 or p.reduce != skg.REDUCE_LAST
    assert p.grid == MB * groups * S and kc % 32 == 0 and (S - 1) * kc < K <= S * kc
    # the grid's (mb, s, j) decode, and the row blocks of one (s, j) on one
    # XCD (ids 8 apart) whenever the (s, j) pairs come in whole groups of 8
    dec = [_tiled_position(b, MB, S, p.grid // MB) for b in range(p.grid)]
    assert sorted(dec) == sorted((mb, s, j) for mb in range(MB) for s in range(S) for j in range(groups))
    if (p.grid // MB) % 8 == 0:
        xcd = {}
        for b, (mb, s, j) in enumerate(dec):
            xcd.setdefault((s, j), set()).add(b % 8)
        assert all(len(v) == 1 for v in xcd.values())
    rows = sorted(mb * MT * 16 + r for mb in range(MB) for r in range(min(MT * 16, M - mb * MT * 16)))
    assert rows == list(range(M))
    # waves partition the workgroup's (m-tile, column-block) grid
    owned = sorted((wm * MTW + a, wn * NBW + b) for wm in range(WM) for wn in range(WN)
                   for a in range(MTW) for b in range(NBW))
    assert owned == sorted((a, b) for a in range(MT) for b in range(NB))
    # a block: 16 rows x 4U chunks of 16 bytes, chunk c of row r at position
    # r*4U + (c ^ swz(r)); instruction part i of a block fills positions
    # 64i .. 64i+63 (lane p: position 64i + p)
    CPR = 4 * U

    def swz(r):
        return (r // (4 // U)) & (CPR - 1)

    stored = {}
    for part in range(U):
        for lane in range(64):
            lin = part * 64 + lane
            r, c = lin // CPR, (lin % CPR) ^ swz(lin // CPR)
            assert (r, c) not in stored
            stored[(r, c)] = lin
    assert sorted(stored) == [(r, c) for r in range(16) for c in range(CPR)]
    assert all(stored[(r, c)] == r * CPR + (c ^ swz(r)) for (r, c) in stored)
    # fragment reads: step u, lane l wants row l % 16, k 32u + 8(l // 16)..+8,
    # i.e. chunk 4u + l // 16; 16 consecutive lanes hit 16 bank groups
    for u in range(U):
        for g in range(4):
            pos = [stored[(l % 16, 4 * u + l // 16)] for l in range(16 * g, 16 * g + 16)]
            assert len({(q * 16 % 256) // 16 for q in pos}) == 16
    # the instructions of a stage: every (block, part) once, per wave a fixed count
    XPW, WPW = -(-(MT * U) // 4), -(-(NB * U) // 4)
    xs = sorted(w + 4 * i for w in range(4) for i in range(XPW) if w + 4 * i < MT * U)
    ws_ = sorted(w + 4 * i for w in range(4) for i in range(WPW) if w + 4 * i < NB * U)
    assert xs == list(range(MT * U)) and ws_ == list(range(NB * U))
    # the epilogue's fp32 tile [MT*16][NB*16 + 4] fits the ring; its 16-byte
    # groups cover every (row < M, column < ncols) of every column group once
    ring = NS * U * (MT + NB) * 1024 + 1024
    TS = NB * 16 + 4
    assert MT * 16 * TS * 4 <= ring and (TS * 4) % 16 == 0
    assert len({(4 * r * TS * 4) % 256 // 64 for r in range(4)}) == 4  # rows 4 apart: other banks
    Mb = min(M, MT * 16)
    for j in range(groups):
        ncols = min(NB * 16, N - 16 * NB * j)
        cov = sorted((e // (NB * 4), (e % (NB * 4)) * 4 + q) for e in range(Mb * NB * 4)
                     for q in range(4) if (e % (NB * 4)) * 4 + q < ncols)
        assert cov == [(r, c) for r in range(Mb) for c in range(ncols)]
    # the ring: stages 0..NS-2 issued up front, stage st+NS-1 issued after
    # stage st is computed into slot (st+NS-1) % NS; a slot is overwritten
    # only after its stage was computed, and the vmcnt wait leaves exactly
    # the loads of the NS-2 later stages outstanding
    assert (NS - 2) * (XPW + WPW) < 64
    for j in range(groups):  # each column group visits every stage once (rotated)
        for s in range(S):
            nsteps = (min(K, (s + 1) * kc) - s * kc) // 32
            nst = -(-nsteps // U)
            rot = j % nst
            assert sorted((st + rot) % nst for st in range(nst)) == list(range(nst))
    seen = [0] * K
    for s in range(S):
        kbeg, kend = s * kc, min(K, (s + 1) * kc)
        nsteps = (kend - kbeg) // 32
        nst = -(-nsteps // U)
        slot_of = {}
        issued = []
        for st in range(NS - 1):
            slot_of[st % NS] = st
            issued.append(st)
        for st in range(nst):
            assert issued[-1] - st == NS - 2  # stages issued after st
            assert slot_of[st % NS] == st
            for u in range(U):
                step = st * U + u
                if step < nsteps:
                    for kk in range(32):
                        seen[kbeg + step * 32 + kk] += 1
            nxt = st + NS - 1
            prev = slot_of.get(nxt % NS)
            assert prev is None or prev <= st
            assert nxt % NS != st % NS or NS == 1
            slot_of[nxt % NS] = nxt
            issued.append(nxt)
    assert seen == [1] * K


@pytest.mark.parametrize("M,N,K,NB,wm,NS,U,S", [
    (512, 4096, 7168, 4, 2, 2, 4, 1), (200, 576, 2048, 8, 2, 4, 2, 2), (129, 64, 1024, 2, 4, 3, 2, 3),
    (128, 4096, 7168, 8, 2, 4, 2, 8), (128, 4096, 7168, 8, 4, 3, 2, 16), (64, 576, 7168, 4, 0, 6, 2, 12),
    (8, 4096, 7168, 8, 1, 6, 2, 8), (33, 200, 2080, 4, 0, 3, 4, 3), (1, 2112, 7168, 16, 0, 2, 4, 4),
    (5, 100, 2880, 4, 1, 4, 2, 5), (100, 50, 1024, 2, 4, 3, 4, 7), (128, 4096, 7168, 8, 2, 2, 4, 8)])
def test_tiled_plans_cover(lib, M, N, K, NB, wm, NS, U, S):
    red = skg.REDUCE_LAST if M <= 128 else skg.REDUCE_KERNEL  # last arriver: one row block
    p = skg.make_plan(skg.KIND_TILED, 256, NB, S, NS, red, waves_m=wm,
                      flags=skg.FLAG_TILED_WIDE if U == 4 else 0)
    q = skg.plan_complete(M, N, K, p)
    assert q.kind == skg.KIND_TILED and q.waves_m in (1, 2, 4)
    _check_coverage(q, M, N, K)


def test_tiled_rejects_bad_plans(lib):
    for plan in (dict(threads=128, cols=4), dict(threads=256, cols=3), dict(threads=256, cols=4, depth=7),
                 dict(threads=256, cols=4, depth=1), dict(threads=256, cols=4, waves_m=3),
                 dict(threads=256, cols=2, waves_m=1), dict(threads=256, cols=4, flags=1),
                 dict(threads=256, cols=16, depth=8, flags=2)):
        p = skg.make_plan(skg.KIND_TILED, plan["threads"], plan["cols"], 2, plan.get("depth", 4),
                          skg.REDUCE_LAST, waves_m=plan.get("waves_m", 0), flags=plan.get("flags", 0))
        with pytest.raises(skg.SkinnyGemmError):
            skg.plan_complete(128, 4096, 7168, p)
    # whole 32-wide steps only
    with pytest.raises(skg.SkinnyGemmError):
        skg.plan_complete(64, 256, 2056, skg.make_plan(skg.KIND_TILED, 256, 4, 2, 4))


# ------------------------------------------------------------------ x in LDS

XLDS = skg.FLAG_DOT_XLDS | skg.FLAG_DOT2


@pytest.mark.parametrize("M,N,K,T,C", [
    (8, 4096, 7168, 512, 16), (1, 4096, 7168, 512, 16), (11, 2112, 7168, 512, 16),
    (4, 300, 2048, 256, 16), (16, 37, 4096, 64, 1), (2, 1, 8192, 1024, 16),
    (5, 1000, 3072, 128, 2), (3, 7, 6144, 256, 8)])
def test_xlds_plans_cover(lib, M, N, K, T, C):
    q = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_DOT, T, C, flags=XLDS))
    assert (q.depth, q.splits, q.reduce, q.k_chunk) == (K // 512, 1, skg.REDUCE_NONE, K)
    _check_coverage(q, M, N, K)


@pytest.mark.parametrize("M,N,K,T,C,flags,dtype", [
    (8, 4096, 7168, 512, 16, skg.FLAG_DOT_XLDS, skg.DTYPE_BF16),   # needs the dot instruction
    (8, 4096, 2880, 512, 16, XLDS, skg.DTYPE_BF16),                # K not 512 V
    (8, 4096, 5120, 512, 16, XLDS, skg.DTYPE_BF16),                # V = 10 not built
    (12, 4096, 7168, 512, 16, XLDS, skg.DTYPE_BF16),               # x over the LDS bound
    (8, 4096, 7168, 256, 12, XLDS, skg.DTYPE_BF16),                # 3 columns a wave
    (8, 4096, 7168, 512, 12, XLDS, skg.DTYPE_BF16),                # cols not a multiple of waves
    (8, 4096, 7168, 512, 4, XLDS, skg.DTYPE_BF16),                 # fewer cols than waves
    (8, 4096, 7168, 256, 16, XLDS, skg.DTYPE_BF16),                # registers (4 x 14 vectors)
    (8, 4096, 7168, 1024, 32, XLDS, skg.DTYPE_BF16),               # registers at 1024 threads
    (17, 4096, 4096, 256, 4, XLDS, skg.DTYPE_BF16),                # M above the dot kernels
    (8, 4096, 4096, 256, 4, XLDS, skg.DTYPE_FP8),                  # bf16 only
    (8, 4096, 7168, 512, 16, XLDS | skg.FLAG_TILED_WIDE, skg.DTYPE_BF16),
])
def test_xlds_rejects(lib, M, N, K, T, C, flags, dtype):
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_DOT, T, C, flags=flags), dtype)
    assert e.value.status == skg.ERR_INVALID_ARG


def test_xlds_rejects_two_splits(lib):
    with pytest.raises(skg.SkinnyGemmError):
        skg.plan_complete(8, 4096, 7168, skg.make_plan(skg.KIND_DOT, 512, 16, splits=2, flags=XLDS))


# ------------------------------------------------------------------ W-first load order

WFIRST = skg.FLAG_DOT2 | skg.FLAG_DOT_WFIRST
PLAN_FIELDS = ("kind", "threads", "cols", "splits", "depth", "waves_m", "reduce", "k_chunk",
               "m_tiles", "grid")


@pytest.mark.parametrize("M,N,K,T,C", [
    (8, 256, 7168, 448, 1), (16, 384, 7168, 448, 2), (1, 256, 7168, 64, 1), (3, 128, 2880, 192, 1),
    (13, 1000, 4096, 256, 3), (2, 7, 2048, 1024, 4)])
def test_wfirst_plans_match_dot2(lib, M, N, K, T, C):
    # the same geometry as the dot plan without it: only the load order differs
    q = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_DOT, T, C, flags=WFIRST))
    r = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_DOT, T, C, flags=skg.FLAG_DOT2))
    assert q.flags == WFIRST
    assert [getattr(q, f) for f in PLAN_FIELDS] == [getattr(r, f) for f in PLAN_FIELDS]
    _check_coverage(q, M, N, K)


@pytest.mark.parametrize("kind,M,N,K,plan,good,bad,dtype", [
    (skg.KIND_DOT, 8, 256, 7168, dict(threads=448), 0, skg.FLAG_DOT_WFIRST,   # needs dot2
     skg.DTYPE_BF16),
    (skg.KIND_DOT, 8, 4096, 7168, dict(threads=512, cols=16), XLDS,          # not with x in LDS
     XLDS | skg.FLAG_DOT_WFIRST, skg.DTYPE_BF16),
    (skg.KIND_DOT, 8, 256, 4096, dict(threads=256), 0, WFIRST, skg.DTYPE_FP8),  # bf16 only
    (skg.KIND_DOT, 8, 256, 4096, dict(threads=256), 0, WFIRST, skg.DTYPE_FP8_MX),
    (skg.KIND_ROWS, 8, 4096, 7168, dict(threads=256, cols=16, depth=4), 0, skg.FLAG_DOT_WFIRST,
     skg.DTYPE_BF16),
    (skg.KIND_TILED, 64, 4096, 7168, dict(threads=256, cols=4, splits=2, depth=4), 0,
     skg.FLAG_DOT_WFIRST, skg.DTYPE_BF16),
    (skg.KIND_SPLITK, 8, 4096, 7168, dict(threads=256, cols=1, splits=4, depth=2,
                                          reduce=skg.REDUCE_KERNEL), 0, skg.FLAG_DOT_WFIRST,
     skg.DTYPE_BF16),
])
def test_wfirst_rejects(lib, kind, M, N, K, plan, good, bad, dtype):
    # the plan is valid without the flag and invalid with it
    skg.plan_complete(M, N, K, skg.make_plan(kind, flags=good, **plan), dtype)
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.plan_complete(M, N, K, skg.make_plan(kind, flags=bad, **plan), dtype)
    assert e.value.status == skg.ERR_INVALID_ARG


def test_wfirst_rejects_above_16_rows(lib):
    with pytest.raises(skg.SkinnyGemmError):
        skg.plan_complete(17, 256, 7168, skg.make_plan(skg.KIND_DOT, 448, 1, flags=WFIRST))


# ------------------------------------------------------------------ whole-row MFMA ring


HALF = skg.FLAG_ROWS_HALF


@pytest.mark.parametrize("M,N,K,T,R,NS,fl", [
    (8, 4096, 7168, 256, 16, 4, 0), (8, 4096, 7168, 512, 16, 6, 0), (1, 2112, 7168, 256, 8, 3, 0),
    (16, 100, 2880, 512, 8, 5, 0), (3, 7, 4104, 256, 16, 4, 0), (13, 4096, 4096, 512, 16, 3, 0),
    (16, 1, 8, 256, 8, 3, 0), (32, 4096, 7168, 256, 16, 3, 0), (64, 4096, 7168, 256, 16, 3, HALF),
    (17, 300, 2056, 512, 8, 6, HALF), (40, 33, 7168, 256, 8, 4, HALF), (5, 4096, 7168, 512, 16, 5, HALF),
    (8, 2112, 7168, 256, 10, 5, HALF), (16, 2112, 7168, 512, 12, 3, 0), (3, 77, 2880, 256, 10, 4, 0)])
def test_rows_plans_cover(lib, M, N, K, T, R, NS, fl):
    q = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_ROWS, T, R, depth=NS, flags=fl))
    assert (q.splits, q.reduce, q.k_chunk, q.m_tiles) == (1, skg.REDUCE_NONE, K, 1)
    _check_coverage(q, M, N, K)


@pytest.mark.parametrize("plan,M,dtype", [
    (dict(threads=256, cols=16, depth=4), 65, skg.DTYPE_BF16),           # M > 64
    (dict(threads=256, cols=10, depth=4), 17, skg.DTYPE_BF16),           # 10 columns: M <= 16
    (dict(threads=256, cols=9, depth=4), 8, skg.DTYPE_BF16),
    (dict(threads=256, cols=4, depth=4), 8, skg.DTYPE_BF16),
    (dict(threads=256, cols=16, depth=3), 64, skg.DTYPE_BF16),           # LDS: 64 rows of 1 KB
    (dict(threads=256, cols=16, depth=4, flags=16), 8, skg.DTYPE_BF16),  # a dot flag
    (dict(threads=128, cols=16, depth=4), 8, skg.DTYPE_BF16),            # 2 waves
    (dict(threads=1024, cols=16, depth=4), 8, skg.DTYPE_BF16),           # 16 waves
    (dict(threads=256, cols=2, depth=4), 8, skg.DTYPE_BF16),             # 2 columns
    (dict(threads=256, cols=32, depth=4), 8, skg.DTYPE_BF16),
    (dict(threads=256, cols=16, depth=2), 8, skg.DTYPE_BF16),            # ring of 2
    (dict(threads=256, cols=16, depth=7), 8, skg.DTYPE_BF16),
    (dict(threads=256, cols=16, depth=6), 16, skg.DTYPE_BF16),           # LDS: 6 x 33 rows
    (dict(threads=256, cols=16, depth=4, splits=2), 8, skg.DTYPE_BF16),
    (dict(threads=256, cols=16, depth=4, flags=skg.FLAG_DOT2), 8, skg.DTYPE_BF16),
    (dict(threads=256, cols=16, depth=4, flags=skg.FLAG_TILED_WIDE), 8, skg.DTYPE_BF16),
    (dict(threads=256, cols=16, depth=4, waves_m=1), 8, skg.DTYPE_BF16),
    (dict(threads=256, cols=16, depth=4, reduce=skg.REDUCE_LAST), 8, skg.DTYPE_BF16),
    (dict(threads=256, cols=16, depth=4), 40, skg.DTYPE_FP8),            # FP8: M <= 32
])
def test_rows_rejects(lib, plan, M, dtype):
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.plan_complete(M, 4096, 4096, skg.make_plan(skg.KIND_ROWS, **plan), dtype)
    assert e.value.status == skg.ERR_INVALID_ARG


# ------------------------------------------------------------------ tiled row blocks below 129 rows


@pytest.mark.parametrize("dtype,M,N,K,NB,mt,S", [
    (skg.DTYPE_BF16, 128, 4096, 7168, 4, 2, 1), (skg.DTYPE_BF16, 100, 576, 7168, 2, 4, 2),
    (skg.DTYPE_BF16, 32, 2112, 7168, 4, 1, 1), (skg.DTYPE_BF16, 17, 300, 1056, 4, 1, 3),
    (skg.DTYPE_FP8, 128, 4096, 4096, 4, 2, 1), (skg.DTYPE_FP8, 128, 4096, 4096, 2, 4, 1),
    (skg.DTYPE_FP8, 77, 1000, 4096, 4, 1, 2), (skg.DTYPE_FP8_MX, 64, 4096, 4096, 4, 2, 1),
    (skg.DTYPE_BF16, 200, 4096, 7168, 4, 4, 1)])
def test_tiled_row_blocks_below_129_rows(lib, dtype, M, N, K, NB, mt, S):
    q = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_TILED, 256, NB, S, 3, m_tiles=mt), dtype)
    MB = -(-M // (16 * mt))
    assert q.m_tiles == mt and q.grid == MB * -(-N // (16 * NB)) * q.splits
    assert q.splits == 1 or q.reduce == skg.REDUCE_KERNEL  # the last arriver needs one row block
    # (above 128 rows the rows' own power of two is 8)
    if dtype == skg.DTYPE_BF16:
        _check_coverage(q, M, N, K)
    else:
        _check_fp8_tiled_coverage(q, M, N, K)
    # 0 keeps the rows' own power of two; so does asking for exactly that
    nat = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_TILED, 256, NB, S, 3), dtype)
    assert nat.m_tiles == next((v for v in (1, 2, 4, 8) if v >= -(-M // 16)), 8)
    again = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_TILED, 256, NB, S, 3,
                                                     m_tiles=nat.m_tiles), dtype)
    assert (again.m_tiles, again.grid) == (nat.m_tiles, nat.grid)


@pytest.mark.parametrize("dtype", (skg.DTYPE_BF16, skg.DTYPE_FP8))
@pytest.mark.parametrize("M,mt,reduce", [(16, 2, 0), (64, 8, 0), (128, 3, 0), (128, 16, 0),
                                         (128, 2, skg.REDUCE_LAST), (200, 16, 0)])
def test_tiled_row_block_requests_rejected(lib, dtype, M, mt, reduce):
    # more tiles than the rows need (or than 8), not a power of two, a
    # last-arriver reduction over several row blocks
    p = skg.make_plan(skg.KIND_TILED, 256, 4, 2 if reduce else 1, 3, reduce, m_tiles=mt)
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.plan_complete(M, 4096, 4096, p, dtype)
    assert e.value.status == skg.ERR_INVALID_ARG


# ------------------------------------------------------------------ FP8 whole-row ring


@pytest.mark.parametrize("dtype,M,N,K,T,R,NS,fl", [
    (skg.DTYPE_FP8, 16, 4096, 4096, 256, 16, 4, 0), (skg.DTYPE_FP8_MX, 16, 4096, 4096, 256, 16, 4, 0),
    (skg.DTYPE_FP8, 1, 4096, 4096, 512, 16, 6, 0), (skg.DTYPE_FP8_MX, 32, 4096, 4096, 256, 16, 3, 8),
    (skg.DTYPE_FP8, 5, 300, 4112, 256, 8, 5, 8), (skg.DTYPE_FP8, 13, 7, 16, 512, 16, 3, 0),
    (skg.DTYPE_FP8_MX, 9, 1000, 2048, 256, 8, 5, 0)])
def test_fp8_rows_plans_cover(lib, dtype, M, N, K, T, R, NS, fl):
    q = skg.plan_complete(M, N, K, skg.make_plan(skg.KIND_ROWS, T, R, depth=NS, flags=fl), dtype)
    assert (q.splits, q.reduce, q.k_chunk, q.m_tiles) == (1, skg.REDUCE_NONE, K, 1)
    _check_fp8_coverage(q, M, N, K, dtype == skg.DTYPE_FP8_MX)


@pytest.mark.parametrize("dtype,M,K,plan", [
    (skg.DTYPE_FP8, 33, 4096, dict(threads=256, cols=16, depth=4)),             # M > 32
    (skg.DTYPE_FP8_MX, 16, 4128, dict(threads=256, cols=16, depth=4)),          # MX: K % 512
    (skg.DTYPE_FP8, 16, 4096, dict(threads=512, cols=16, depth=4, flags=8)),    # 4 steps, 8 waves
    (skg.DTYPE_FP8, 32, 4096, dict(threads=256, cols=16, depth=4)),             # LDS (MX layout)
    (skg.DTYPE_FP8, 16, 4096, dict(threads=256, cols=16, depth=4, flags=1)),
    (skg.DTYPE_FP8, 16, 4096, dict(threads=256, cols=4, depth=4)),
    (skg.DTYPE_FP8, 16, 4096, dict(threads=256, cols=16, depth=4, splits=2)),
])
def test_fp8_rows_rejects(lib, dtype, M, K, plan):
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.plan_complete(M, 4096, K, skg.make_plan(skg.KIND_ROWS, **plan), dtype)
    assert e.value.status == skg.ERR_INVALID_ARG
