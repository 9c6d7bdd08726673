"""A C client of the library (tests/c_client/c_abi_client.c) built with gcc
against include/ and the HIP runtime only: it links on any machine (CPU
test) and, on a GPU, runs the automatic, split-K and tiled plans and checks
every output exactly against a closed form (GPU test)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_client", "c_abi_client.c")
LIBDIR = os.path.join(ROOT, "latency_skinny_gemm_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(out_dir):
    exe = os.path.join(str(out_dir), "c_abi_client")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", LIBDIR, "-lskinny_gemm", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + LIBDIR + ":" + os.path.join(ROCM, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_client_builds_and_links(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libskinny_gemm.so")):
        pytest.skip("library not built")
    _build(tmp_path)


@pytest.mark.gpu
def test_c_client_runs(tmp_path):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = _build(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c-abi client: ok" in r.stdout, r.stdout + r.stderr
