"""Builds tests/_build/c_abi_check from tests/c_abi_check.c: a plain C program
that drives libvdc.so through include/vdc.h and checks it against the FP64
oracle (test infrastructure; it links the oracle's library)."""
from __future__ import annotations

import os
import shutil
import subprocess

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
SOURCE = os.path.join(TESTS, "c_abi_check.c")
BINARY = os.path.join(TESTS, "_build", "c_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    """Compile and link against the in-tree libvdc.so and liboracle.so (both
    must be built first); the run path is relative to the binary, so the
    tree can move."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(os.path.dirname(BINARY), exist_ok=True)
    tmp = BINARY + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-O2", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-I" + os.path.join(ROOT, "include"), "-o", tmp, SOURCE,
           "-L" + os.path.join(ROOT, "varlen_depthwise_causal_amd"), "-lvdc",
           "-L" + os.path.join(ROOT, "oracle"), "-loracle",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../varlen_depthwise_causal_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, BINARY)
    return BINARY


if __name__ == "__main__":
    print(build())
