"""Host-only checks of bench.py's bookkeeping (no GPU needed).

The byte counts are checked against the element counts of the pages' data
layouts (row-major [S, C] BF16 activations, [C, 4] weight, [C] bias, int32
cu_seqlens of num_docs + 1 entries); the counter file's digest rule, and the
refusal of more than one GPU, are checked on temporary files.
"""
import json
import os
import subprocess
import sys
import types

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _wl(S, C, w_dtype, b_dtype, docs):
    return types.SimpleNamespace(S=S, C=C, w_dtype=w_dtype, b_dtype=b_dtype,
                                 b=None if b_dtype is None else np.zeros(C),
                                 cu=np.zeros(docs + 1, dtype=np.int32))


def test_algorithmic_bytes_headline():
    wl = _wl(65536, 4096, "f32", "f32", 22)
    act = 65536 * 4096 * 2
    params = 4096 * 16 + 4096 * 4 + 23 * 4
    assert bench.algorithmic_bytes(wl, "fwd") == 2 * act + params
    # x and dy read, dx written; FP32 dweight [C, 4] and dbias [C] written.
    assert bench.algorithmic_bytes(wl, "bwd") == 3 * act + params + 4096 * 16 + 4096 * 4


def test_algorithmic_bytes_bf16_params_no_bias():
    wl = _wl(1000, 64, "bf16", None, 8)
    assert bench.algorithmic_bytes(wl, "fwd") == 4 * 1000 * 64 + 64 * 8 + 9 * 4
    assert bench.algorithmic_bytes(wl, "bwd") == 6 * 1000 * 64 + 64 * 8 + 9 * 4 + 64 * 16


def test_sources_digest_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int a) { return a + 1; }  // one\n/* block */\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    d0 = bench.sources_digest()
    src.write_text("// another comment\nint f(int a) {\n  return a + 1;\n}\n")
    assert bench.sources_digest() == d0
    src.write_text("int f(int a) { return a + 2; }\n")
    assert bench.sources_digest() != d0


def test_counted_traffic_follows_digest_and_policy(tmp_path, monkeypatch):
    counters = tmp_path / "counters.md"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(counters))
    assert bench.counted_traffic("bf16") is None            # no file
    rec = {"sources": bench.sources_digest(), "policy": "bf16",
           "bytes_per_launch": {"fwd_kernel": 1, "bwd_main_kernel": 2, "bwd_reduce_kernel": 3}}
    counters.write_text("# summary\n\ntraffic-json: %s\n" % json.dumps(rec))
    assert bench.counted_traffic("bf16") == rec
    assert bench.counted_traffic("fp32") is None             # other policy
    rec["sources"] = "0" * 16
    counters.write_text("traffic-json: %s\n" % json.dumps(rec))
    assert bench.counted_traffic("bf16") is None             # other sources


def test_committed_counters_parse():
    """The committed summary holds one well-formed traffic record per
    policy, all taken on the same kernel sources."""
    lines = [l for l in open(bench.COUNTERS_FILE).read().splitlines() if l.startswith("traffic-json: ")]
    recs = [json.loads(l[len("traffic-json: "):]) for l in lines]
    assert sorted(r["policy"] for r in recs) == ["bf16", "fp32"]
    assert len({r["sources"] for r in recs}) == 1
    for rec in recs:
        assert set(rec["bytes_per_launch"]) == {"fwd_kernel", "bwd_main_kernel", "bwd_reduce_kernel"}


@pytest.mark.parametrize("argv, env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, env=e, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
