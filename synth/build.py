"""Build the host (gcc) and device (hipcc, gfx950) generator libraries in-tree."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))

HIP_FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17",
             "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_host(verbose: bool = False) -> str:
    out = os.path.join(_HERE, "libsynth.so")
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", out + ".tmp", os.path.join(_HERE, "synth.c"), "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_device(verbose: bool = False) -> str:
    out = os.path.join(_HERE, "libsynth_dev.so")
    cmd = ["hipcc", *HIP_FLAGS, "-o", out + ".tmp", os.path.join(_HERE, "synth_dev.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> None:
    build_host(verbose)
    build_device(verbose)


if __name__ == "__main__":
    build(verbose=True)
