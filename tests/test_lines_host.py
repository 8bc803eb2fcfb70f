"""The forward's choice of streaming stores on rows that are not a multiple
of 128 bytes, run on the CPU (tests/lines_check.cpp over
varlen_depthwise_causal_amd/csrc/vdc_lines.h): a lane's store streams only
where its wave, within the lane's band, writes every byte of the cache line
for that row, and the choice repeats every 8 rows."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_whole_lines_on_cpu(tmp_path):
    exe = str(tmp_path / "lines_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "varlen_depthwise_causal_amd", "csrc"),
                    os.path.join(ROOT, "tests", "lines_check.cpp"), "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "lines_check: ok" in out.stdout
