"""Build libastr.so in-tree for gfx950.

    python -m paged_gqa_attention_rope_amd.build [-v]

HIP sources are compiled by hipcc for gfx950 only, with the packed-fp32
instructions disabled (-Xclang -target-feature -Xclang -packed-fp32-ops); the
host-only page-table builder is compiled by g++.  Objects go to _build/ and
the library is renamed into place atomically.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libastr.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GXX = os.environ.get("CXX", "g++")

HIP_SOURCES = ["rope.hip", "decode.hip", "prefill.hip", "ceiling.hip"]
# per-source extra flags: the attention kernels never rely on NaN propagation
# (masking uses -inf, which stays honoured), and without it every fmaxf of a
# matrix-core result is preceded by a NaN-quieting canonicalisation
EXTRA = {"prefill.hip": ["-fno-honor-nans"], "decode.hip": ["-fno-honor-nans"]}
HIP_HOST_SOURCES = ["abi.cpp"]
HOST_SOURCES = ["pagepool.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
HIP_FLAGS = COMMON + [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
                      "-packed-fp32-ops", "-munsafe-fp-atomics"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([GXX, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
