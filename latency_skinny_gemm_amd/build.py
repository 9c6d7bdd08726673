"""Builds libskinny_gemm.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-fp32 instruction selection turned
off (-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass of
hipcc warns that it does not know that feature, which is harmless.
Objects go to _build/ (git-ignored); the library lands beside this file.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libskinny_gemm.so")
FLOORS_LIB = os.path.join(HERE, "libskinny_floors.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
              "-I", "/opt/rocm/include", "-I", INCLUDE, "-I", CSRC]

LIB_HIP = ["api.hip", "kernels_dot.hip", "kernels_splitk.hip", "kernels_tiled.hip",
           "kernels_fp8.hip", "kernels_quant.hip", "kernels_fp8_tiled.hip", "kernels_rows.hip",
           "kernels_fp8_rows.hip"]
LIB_HOST = ["plan.cpp"]
# Per-file flags.  The tiled kernels keep their accumulators in VGPRs: with the
# compiler's default AGPR form, the loop-carried accumulators were copied
# between AGPRs and VGPRs around every MFMA (resource report and assembly).
EXTRA_FLAGS = {"kernels_tiled.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "kernels_fp8_tiled.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "kernels_rows.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "kernels_fp8_rows.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
FLOORS_HIP = ["floors.hip"]


def _compile(src, obj, hip, verbose):
    cmd = ([HIPCC] + HIP_FLAGS if hip else ["g++"] + HOST_FLAGS) + \
        EXTRA_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature: drop that note
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def _link(objs, out, verbose):
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, jobs: int = 8):
    os.makedirs(BUILD, exist_ok=True)
    work = []
    for s in LIB_HIP + FLOORS_HIP:
        work.append((os.path.join(CSRC, s), os.path.join(BUILD, s + ".o"), True))
    for s in LIB_HOST:
        work.append((os.path.join(CSRC, s), os.path.join(BUILD, s + ".o"), False))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda w: _compile(w[0], w[1], w[2], verbose), work))
    _link([os.path.join(BUILD, s + ".o") for s in LIB_HIP + LIB_HOST], LIB, verbose)
    _link([os.path.join(BUILD, s + ".o") for s in FLOORS_HIP], FLOORS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
