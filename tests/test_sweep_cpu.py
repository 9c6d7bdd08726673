"""CPU tests of the dispatch-table emission from sweep logs (no GPU): the
median rule across logs, the filters for timings of earlier kernels, the
per-mode FP8 entries and the rejection of plans the planner no longer
accepts."""
import json

import pytest

import latency_skinny_gemm_amd as skg
from latency_skinny_gemm_amd import sweep


def _plan(kind, threads, cols=1, splits=1, depth=0, reduce=0, flags=0, waves_m=0):
    return {"kind": kind, "threads": threads, "cols": cols, "splits": splits, "depth": depth,
            "waves_m": waves_m, "reduce": reduce, "flags": flags}


def _write(path, recs):
    with open(path, "w") as fh:
        for r in recs:
            fh.write(json.dumps(r) + "\n")
    return str(path)


def _rows(path):
    out = {}
    for line in open(path):
        if line.startswith("{"):
            key = tuple(x.strip() for x in line[1:].split(",")[:4])
            out[key] = line.split("//")[0].strip()
    return out


@pytest.fixture(scope="module")
def lib():
    try:
        return skg.lib()
    except RuntimeError as e:
        pytest.skip(str(e))


def test_emit_ranks_by_median_and_filters(lib, tmp_path):
    M, N, K = 8, 256, 7168
    a = _plan(1, 448, depth=2, flags=1)   # T = 448, V = 2
    b = _plan(1, 256, depth=4, flags=1)   # T = 256, V = 4
    w1 = _plan(1, 64, depth=14, flags=1)  # one wave
    tiled = _plan(3, 256, cols=4, splits=4, depth=3, reduce=2, flags=2, waves_m=1)
    base = {"M": M, "N": N, "K": K, "slots": 4, "dot_reduce": "scatter"}
    # b wins once by luck; a wins on the median of three logs
    logs = [
        _write(tmp_path / "l1.jsonl", [dict(base, candidates=[[4.0, a], [3.0, b]])]),
        _write(tmp_path / "l2.jsonl", [dict(base, candidates=[[4.1, a], [5.0, b]])]),
        _write(tmp_path / "l3.jsonl", [dict(base, candidates=[[4.2, a], [5.1, b]])]),
        # earlier kernels' timings: a tiled plan without the ring tag, and
        # (at M = 1) a one-wave plan without the direct-store tag, are ignored
        _write(tmp_path / "l4.jsonl", [dict(base, candidates=[[1.0, tiled]]),
                                       dict(base, M=1, candidates=[[1.0, w1], [2.0, a]])]),
    ]
    out = tmp_path / "table.inc"
    sweep.emit_table(logs, out_path=str(out))
    rows = _rows(out)
    assert rows[("SKG_DTYPE_BF16", "7168", "256", "8")] == \
        "{SKG_DTYPE_BF16, 7168, 256, 8, {SKG_KIND_DOT, 448, 1, 1, 2, 0, SKG_REDUCE_NONE, 1}},"
    assert "SKG_KIND_DOT, 448" in rows[("SKG_DTYPE_BF16", "7168", "256", "1")]
    # with the tags the same timings count
    logs.append(_write(tmp_path / "l5.jsonl", [dict(base, tiled="ring2", candidates=[[1.0, tiled]]),
                                               dict(base, M=1, dot_wave1="direct",
                                                    candidates=[[1.0, w1]])]))
    sweep.emit_table(logs, out_path=str(out))
    rows = _rows(out)
    assert "SKG_KIND_TILED, 256, 4, 4, 3, 1" in rows[("SKG_DTYPE_BF16", "7168", "256", "8")]
    assert "SKG_KIND_DOT, 64, 1, 1, 14" in rows[("SKG_DTYPE_BF16", "7168", "256", "1")]
    # dot timings from before the reduce-scatter (no dot_reduce tag) are ignored
    untagged = {k: v for k, v in base.items() if k != "dot_reduce"}
    logs.append(_write(tmp_path / "l6.jsonl", [dict(untagged, M=2, candidates=[[0.5, b], [9.0, tiled]],
                                                    tiled="ring2")]))
    sweep.emit_table(logs, out_path=str(out))
    assert "SKG_KIND_TILED" in _rows(out)[("SKG_DTYPE_BF16", "7168", "256", "2")]


def test_emit_skips_plans_the_planner_rejects(lib, tmp_path):
    M, N, K = 4, 256, 2048
    bad = _plan(1, 256, cols=5, depth=1, flags=1)   # 5 columns: not built
    stale = _plan(1, 256, depth=3, flags=1)         # V is 1 at this K: completes differently
    good = _plan(1, 256, depth=1, flags=1)
    log = _write(tmp_path / "l.jsonl", [{"M": M, "N": N, "K": K, "slots": 4, "dot_reduce": "scatter",
                                         "candidates": [[1.0, bad], [1.5, stale], [2.0, good]]}])
    out = tmp_path / "table.inc"
    sweep.emit_table([log], out_path=str(out))
    assert _rows(out)[("SKG_DTYPE_BF16", "2048", "256", "4")] == \
        "{SKG_DTYPE_BF16, 2048, 256, 4, {SKG_KIND_DOT, 256, 1, 1, 1, 0, SKG_REDUCE_NONE, 1}},"


def test_emit_fp8_entries_per_scale_mode(lib, tmp_path):
    M, N, K = 1, 4096, 4096
    d = _plan(1, 256, depth=1)
    s = _plan(2, 256, cols=1, splits=1, depth=2)
    rec = {"dtype": "fp8", "M": M, "N": N, "K": K, "slots": 4, "mx_scales": "per_slot",
           "dot_reduce": "scatter",
           "candidates": [[9.0, {"tensor": 4.0, "mx": 5.0}, d], [9.0, {"tensor": 4.5, "mx": 4.5}, s]]}
    out = tmp_path / "table.inc"
    sweep.emit_table([_write(tmp_path / "f.jsonl", [rec])], out_path=str(out))
    rows = _rows(out)
    assert "SKG_KIND_DOT" in rows[("SKG_DTYPE_FP8", "4096", "4096", "1")]
    assert "SKG_KIND_SPLITK" in rows[("SKG_DTYPE_FP8_MX", "4096", "4096", "1")]
    # MX timings count only where the scale bytes were cold too
    rec.pop("mx_scales")
    sweep.emit_table([_write(tmp_path / "g.jsonl", [rec])], out_path=str(out))
    assert ("SKG_DTYPE_FP8_MX", "4096", "4096", "1") not in _rows(out)
