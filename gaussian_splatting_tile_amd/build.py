"""Build libgs.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m gaussian_splatting_tile_amd.build

Compiles every csrc/*.hip into one shared library next to this file.
Floating-point flags matter for parity: no contraction, IEEE-correct fp32
division and square root, denormals kept. Packed-FP32 instructions are
disabled (-packed-fp32-ops).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgs.so")
ARCH = os.environ.get("GS_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-ffp-contract=off", "-fno-fast-math",
            "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def sources() -> list:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + compile_flags() + ["-shared", "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def asm(source: str, out: str) -> None:
    """Write the gfx950 assembly of one source (for inspection)."""
    cmd = [hipcc()] + compile_flags() + ["--cuda-device-only", "-S", "-o", out, source]
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
