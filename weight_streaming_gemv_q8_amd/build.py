"""Build libwsgemv.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``) and without
fast-math, so fp32 division is IEEE (the Q8_0 quantizer relies on it).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwsgemv.so")
OBJ_DIR = os.path.join(PKG, "_build")
# the diagnostic build: the same library with per-workgroup timestamps in the
# int8 GEMV (csrc/timeline.hpp, read by timeline.py)
TIMELINE_LIB = os.path.join(PKG, "libwsgemv_timeline.so")
TIMELINE_OBJ_DIR = os.path.join(PKG, "_build_timeline")

SOURCES = ["api.cpp", "quant.hip", "norm.hip", "gemv.hip", "stream.hip", "decode.hip", "probe.hip", "plan.cpp"]

HIP_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, verbose: bool, timeline: bool = False) -> str:
    obj = os.path.join(TIMELINE_OBJ_DIR if timeline else OBJ_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = ["-DWSG_TIMELINE"] if timeline else []
    cmd = ["hipcc", *HIP_FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Builds libwsgemv.so (or, with timeline=True, the diagnostic
    libwsgemv_timeline.so) and returns its path."""
    lib = TIMELINE_LIB if timeline else LIB
    os.makedirs(TIMELINE_OBJ_DIR if timeline else OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, timeline), SOURCES))
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, timeline="--timeline" in sys.argv)
