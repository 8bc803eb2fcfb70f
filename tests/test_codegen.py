"""Checks of the gfx950 code the kernels compile to (CPU only: hipcc
cross-compiles).

* No machine instruction of the final code reads a register the register
  allocator marked undefined.  The ROCm LLVM in use once dropped the
  sub-register liveness of a loaded row that was overwritten in place with
  its packed result, leaving a read of a clobbered register: a silent wrong
  value that only a parity run shows.  This scan catches that class of
  miscompile at build time.
* No kernel spills to scratch memory (a performance guard: the kernels are
  sized to live in registers at one wave per SIMD).
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from varlen_depthwise_causal_amd import _build

KERNELS = os.path.join(_build.CSRC, "vdc_kernels.hip")


def _compile(extra):
    cmd = [_build.hipcc(), *_build.COMMON, *_build.DEVICE_FLAGS, "--cuda-device-only", "-S",
           "-o", os.devnull, KERNELS, *extra]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return res.stderr


@pytest.fixture(scope="module")
def final_mir():
    try:
        _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    return _compile(["-mllvm", "-print-after=postmisched"])


def _functions(mir):
    name, body = None, []
    for line in mir.splitlines():
        m = re.match(r"# Machine code for function (\S+):", line)
        if m:
            if name:
                yield name, body
            name, body = m.group(1), []
        elif name:
            body.append(line)
    if name:
        yield name, body


def test_every_kernel_is_scanned(final_mir):
    names = [n for n, _ in _functions(final_mir)]
    assert any("fwd_kernel" in n for n in names)
    assert sum("bwd_main_kernel" in n for n in names) == 12
    assert sum("bwd_reduce_kernel" in n for n in names) == 2


def test_no_read_of_undefined_registers(final_mir):
    bad = []
    for name, body in _functions(final_mir):
        for line in body:
            if "IMPLICIT_DEF" in line or " KILL" in line:
                continue
            # operands after the '=' (or the whole line for stores)
            rhs = line.split("=", 1)[1] if "=" in line else line
            if re.search(r"undef \$[va]gpr", rhs):
                bad.append("%s: %s" % (name, line.strip()[:160]))
    assert not bad, "reads of registers the allocator left undefined:\n" + "\n".join(bad[:20])


def test_no_scratch_spills():
    try:
        _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = _compile(["-Rpass-analysis=kernel-resource-usage"])
    names = re.findall(r"Function Name: (\S+)", out)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out)]
    assert names and len(names) == len(scratch)
    spilled = [(n, s) for n, s in zip(names, scratch) if s]
    assert not spilled, spilled
