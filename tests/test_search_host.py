"""The kernels' search over cu_seqlens, run on the CPU (tests/search_check.cpp
with an emulated wave ballot over the bracket arithmetic of
varlen_depthwise_causal_amd/csrc/vdc_search.h): probes stay inside
[0, num_docs + 1) up to 2^31 - 1 entries, the search ends, and it finds the
first entry at or above the value for well-formed cu_seqlens."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_search_bracket_on_cpu(tmp_path):
    exe = str(tmp_path / "search_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "varlen_depthwise_causal_amd", "csrc"),
                    os.path.join(ROOT, "tests", "search_check.cpp"), "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "search_check: ok" in out.stdout
