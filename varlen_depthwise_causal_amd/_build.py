"""Ahead-of-time build of libvdc.so for gfx950 with hipcc (no JIT)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libvdc.so")

ARCH = "gfx950"
# Packed FP32 instructions stay off: plain float code is scheduled on the
# scalar-per-lane FP32 pipes.  FMA contraction is off too: every FMA in the
# kernels is written out, so the evaluation order is exactly the source's.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-ffp-contract=off"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libvdc.so")
    return path


def build(verbose: bool = False) -> str:
    """Compile csrc/*.hip + csrc/*.cpp into libvdc.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src, extra in (("vdc_kernels.hip", DEVICE_FLAGS), ("vdc_api.cpp", [])):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
