"""The C ABI used from a plain C program (tests/c_abi_check.c): device
memory and a stream from the HIP runtime, no Python in the loop, results
checked against the FP64 oracle inside the program."""
import os
import subprocess

import pytest

import c_abi_build


def _binary():
    if not os.path.exists(c_abi_build.BINARY):
        from varlen_depthwise_causal_amd import _build
        import oracle
        if not os.path.exists(_build.LIBRARY):
            _build.build()
        if not os.path.exists(oracle.LIBRARY):
            oracle.build()
        c_abi_build.build()
    return c_abi_build.BINARY


def test_c_program_links_and_reports_no_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the GPU test runs the program")
    r = subprocess.run([_binary()], capture_output=True, text=True, timeout=60)
    assert r.returncode == 77, (r.returncode, r.stdout, r.stderr)
    assert "no GPU" in r.stderr


@pytest.mark.gpu
def test_c_program_against_oracle():
    exe = c_abi_build.BINARY
    assert os.path.exists(exe), "tests/_build/c_abi_check is not built: run __graft_entry__.build()"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
