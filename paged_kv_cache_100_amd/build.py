"""Build libpagedkv.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m paged_kv_cache_100_amd.build [--save-temps DIR]

Compiles ``csrc/pagedkv.hip`` with hipcc into ``paged_kv_cache_100_amd/
libpagedkv.so``.  Packed-FP32 instructions are disabled for device code.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "pagedkv.hip")
LIB = os.path.join(PKG, "libpagedkv.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build libpagedkv.so)")
    return path


def command(out: str = LIB, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-result",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # Matrix-instruction accumulators in ordinary vector registers: the
            # online softmax rescales the output accumulators with vector
            # multiplies, and accumulation registers would need a copy of them
            # kept in vector registers on every chunk.
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
            *extra, "-o", out, SRC]


def build(save_temps: str | None = None, verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    extra = []
    cwd = None
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        extra = ["--save-temps"]
        cwd = save_temps
    cmd = command(tmp, extra)
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None)
    a = ap.parse_args()
    print(build(a.save_temps, verbose=True))
