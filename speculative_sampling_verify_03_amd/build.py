"""Build libspecverify.so in-tree: HIP sources for gfx950 with hipcc, the host validator
with g++, linked into one shared library next to this file.

    python -m speculative_sampling_verify_03_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

HIP_SOURCES = ["api.hip", "verify_rows.hip", "verify_split.hip", "verify_greedy.hip", "lmhead_gemm.hip", "lmhead_verify.hip", "plug.hip",
               "lookup.hip"]
CXX_SOURCES = ["validate.cpp"]

ARCH = "gfx950"
HIP_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    # packed fp32 instructions are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source additions.  The LM-head GEMM keeps its accumulators in VGPRs: with the
# compiler's default AGPR placement the loop-carried accumulators were shuffled between
# register files every step, which stalls on the matrix-core results.
HIP_FILE_FLAGS = {"lmhead_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source (always) and link LIB_PATH.  Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    incs = [f"-I{INCLUDE}", f"-I{CSRC}"]
    steps = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append([hipcc, *HIP_FLAGS, *HIP_FILE_FLAGS.get(src, []), *incs, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append(["g++", *CXX_FLAGS, *incs, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(steps)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), steps))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
