"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_461_amd.build        # or: from paged_kv_cache_461_amd import build; build.build()

Each .hip source under csrc/ is compiled to an object in csrc/_build/ with hipcc, each .cpp
source (host-only code) with g++, in parallel; the objects are linked into
paged_kv_cache_461_amd/libpagedattn.so.  Packed fp32 instructions are disabled for all device
code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "libpagedattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


# Per-file additions.  The prefill kernel never produces NaN scores (masked keys are -inf, keys
# of invalid blocks are zeroed before use), so its max reductions need no IEEE NaN quieting.
FILE_FLAGS = {
    "prefill.hip": ["-Xarch_device", "-fno-honor-nans", "-Xarch_device", "-mno-amdgpu-ieee",
                    "-Wno-nan-infinity-disabled"],
}


CXX = os.environ.get("CXX_HOST", "g++")
HOST_CFLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        cmd = [CXX, *HOST_CFLAGS, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
