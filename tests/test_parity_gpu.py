"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle.

Small cases are compared element by element on every output; the full-size
workloads run at their real shapes (the launch configuration the benchmark
times) and are compared on whole 8-channel groups of sampled columns for
every token, plus bitwise reproducibility of the whole gradients.
"""
import numpy as np
import pytest

import gpu_cases as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
def test_tiny_all_elements(torch_cuda, policy):
    G.say("CASE tiny", policy)
    wl = G.named("tiny")
    dev = G.to_device(wl)
    y, dx, dw, db = G.run_gpu(dev, policy)
    G.compare(wl, policy, y, dx, dw, db, label="tiny")


SMALL = [
    # (label, seed, S, C, lengths or None (one doc), w_dtype, b_dtype, sat)
    ("c8_ragged", 5, 777, 8, [0, 3, 1, 0, 40, 2, 300, 431, 0], "f32", "f32", None),
    ("c24_single", 6, 2049, 24, None, "f32", None, None),
    ("c520_stress", 7, 3001, 520, "randint", "f32", "f32", (0.01, 60.0)),
    ("c1024_bf16params", 8, 1500, 1024, [700, 0, 1, 2, 3, 794], "bf16", "bf16", None),
    ("c64_len1", 9, 300, 64, [1] * 300, "f32", "f32", None),
    ("c64_empty_ends", 10, 500, 64, [0, 0, 250, 0, 250, 0, 0], "bf16", None, None),
    ("c4096_rows", 11, 700, 4096, [350, 350], "f32", "f32", None),
    ("c520_deep", 12, 1200, 520, [1200], "f32", "f32", (0.05, 60.0)),
    # one wave per band row (C/4 = 64) and a start every ~13 rows: nearly
    # every group of every wave takes the masked path
    ("c256_dense", 13, 2000, 256, "randint", "f32", "f32", None),
    # fewer tokens than the halo and than one row group: every band's tail,
    # the look-ahead rows and the skipped first dx rows fall outside [0, S)
    ("s1_c8", 15, 1, 8, [1], "f32", "f32", None),
    ("s2_c64", 16, 2, 64, [0, 1, 1], "bf16", "f32", None),
    ("s5_c136", 17, 5, 136, [2, 0, 3], "f32", None, None),
    # backward lanes in column blocks (four bands per workgroup): 2048
    # channels, bands of 48 rows, 105 bands (the last group of four holds
    # one), a start every ~13 rows
    ("c2048_groups", 18, 5000, 2048, "randint", "f32", "f32", None),
]


_small = G.small_case


def _random_shapes(n, seed=2024):
    """Seeded shapes: C any multiple of 8 up to 1032 (waves straddle bands at
    many ratios), S from 1 to 3000, documents of random lengths with empty
    and length-1 documents mixed in, bias or none, FP32 or BF16 parameters."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        C = 8 * int(rng.integers(1, 130))
        S = int(rng.integers(1, 3001))
        lengths, left = [], S
        while left > 0:
            kind = rng.random()
            n_t = 0 if kind < 0.1 else (1 if kind < 0.2 else int(rng.integers(1, max(2, S // 3))))
            n_t = min(n_t, left)
            lengths.append(n_t)
            left -= n_t
        if rng.random() < 0.3:
            lengths.append(0)
        w_dt = "bf16" if rng.random() < 0.3 else "f32"
        b_dt = None if rng.random() < 0.25 else ("bf16" if rng.random() < 0.3 else "f32")
        sat = (0.02, 60.0) if rng.random() < 0.2 else None
        out.append(("rand%02d_s%d_c%d" % (i, S, C), 100 + i, S, C, lengths, w_dt, b_dt, sat))
    return out


RANDOM = _random_shapes(48)


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_all_elements(torch_cuda, case, policy):
    label = case[0]
    G.say("CASE", label, policy)
    wl = _small(*case[1:])
    dev = G.to_device(wl)
    y, dx, dw, db = G.run_gpu(dev, policy)
    G.compare(wl, policy, y, dx, dw, db, label=label)


FULL = [("uniform", "bf16"), ("headline", "bf16"), ("long", "fp32"),
        ("stress", "bf16"), ("stress", "fp32")]


def _medium_shapes(n, seed=77):
    """Seeded mid-size shapes (up to 6.4e7 elements) spread over the launch
    planner: C any multiple of 8 up to 6400, S up to 250000, so band sizes,
    band counts, straddling waves and padded grids vary.  Documents: one,
    many short ones (U{0..30}), or random lengths up to S / 4."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        C = 8 * int(rng.integers(1, 801))
        S = int(rng.integers(2000, max(2001, min(250000, 64_000_000 // C))))
        kind = i % 3
        if kind == 0:
            lengths = [S]
        else:
            hi = 31 if kind == 1 else max(2, S // 4)
            lengths, left = [], S
            while left > 0:
                n_t = min(int(rng.integers(0, hi)), left)
                lengths.append(n_t)
                left -= n_t
        w_dt = "bf16" if rng.random() < 0.3 else "f32"
        b_dt = None if rng.random() < 0.25 else ("bf16" if rng.random() < 0.3 else "f32")
        out.append(("mid%02d_s%d_c%d" % (i, S, C), 300 + i, S, C, lengths, w_dt, b_dt, None))
    return out


MEDIUM = _medium_shapes(12)


@pytest.mark.parametrize("case", MEDIUM, ids=[c[0] for c in MEDIUM])
def test_medium_shapes_sampled(torch_cuda, case):
    """Whole 8-channel groups of sampled columns, every token, both policies."""
    label = case[0]
    wl = _small(*case[1:])
    dev = G.to_device(wl)
    cols = G.sample_columns(wl.C, groups=8, seed=case[1])
    for policy in ("bf16", "fp32"):
        G.say("CASE", label, policy)
        y, dx, dw, db = G.run_gpu(dev, policy)
        G.compare(wl, policy, y, dx, dw, db, cols, label=label)


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_shapes_all_elements(torch_cuda, case):
    label = case[0]
    policy = "fp32" if case[1] % 2 else "bf16"
    G.say("CASE", label, policy)
    wl = _small(*case[1:])
    dev = G.to_device(wl)
    y, dx, dw, db = G.run_gpu(dev, policy)
    G.compare(wl, policy, y, dx, dw, db, label=label)


@pytest.mark.parametrize("name,policy", FULL, ids=["%s-%s" % f for f in FULL])
def test_full_size_sampled(torch_cuda, name, policy):
    torch = torch_cuda
    G.say("CASE full", name, policy)
    wl = G.named(name)
    dev = G.to_device(wl)
    y, dx, dw, db = G.run_gpu(dev, policy)
    cols = G.sample_columns(wl.C, groups=8, seed=1)
    G.compare(wl, policy, y, dx, dw, db, cols, label=name)
    # A second run gives bitwise the same outputs.
    y2, dx2, dw2, db2 = G.run_gpu(dev, policy)
    assert torch.equal(y, y2) and torch.equal(dx, dx2) and torch.equal(dw, dw2)
    if db is not None:
        assert torch.equal(db, db2)
    del dev, y, dx, dw, db, y2, dx2, dw2, db2
    torch.cuda.empty_cache()


# Every element of generic (seeded random) full-size inputs, in the launch
# configuration the benchmark times: (workload, policy, column block).
FULL_ALL = [("headline", "bf16", 256), ("headline", "fp32", 256),
            ("stress", "bf16", 32), ("stress", "fp32", 32),
            ("long", "fp32", 256), ("uniform", "bf16", 128)]


@pytest.mark.parametrize("name,policy,block", FULL_ALL, ids=["%s-%s" % f[:2] for f in FULL_ALL])
def test_full_size_all_elements(torch_cuda, name, policy, block):
    """All S x C elements of y and dx, and all of dweight / dbias, against
    the oracle under the same rules as the small cases (the oracle runs on
    blocks of columns on host threads)."""
    torch = torch_cuda
    G.say("CASE full, every element", name, policy)
    wl = G.named(name)
    dev = G.to_device(wl)
    y, dx, dw, db = G.run_gpu(dev, policy)
    G.compare_all(wl, policy, y, dx, dw, db, label=name + " all", block=block, workers=16)
    del dev, y, dx, dw, db
    torch.cuda.empty_cache()


def test_zero_tokens_launch_nothing(torch_cuda):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE S=0")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((64, 4), device="cuda")
    b = torch.randn((64,), device="cuda")
    for cu in ([0], [0, 0, 0]):
        cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
        n0 = vdc.conv1d_launch_count()
        y = vdc.conv1d_fwd(x, w, cu_t, bias=b)
        dw = torch.full((64, 4), 7.0, device="cuda")
        db = torch.full((64,), 7.0, device="cuda")
        dx, dw, db = vdc.conv1d_bwd(x, w, cu_t, x, bias=b, dweight=dw, dbias=db)
        torch.cuda.synchronize()
        assert vdc.conv1d_launch_count() == n0
        assert y.shape == (0, 64) and dx.shape == (0, 64)
        assert torch.all(dw == 0) and torch.all(db == 0)


def test_bitwise_across_workspaces_and_streams(torch_cuda):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE determinism")
    wl = _small(13, 20000, 520, "randint", "f32", "f32", (0.01, 60.0))
    dev = G.to_device(wl)
    need = vdc.workspace_bytes("bwd", wl.S, wl.C)
    for policy in ("bf16", "fp32"):
        runs = []
        for i in range(3):
            ws = torch.randint(0, 256, (need + 4096,), dtype=torch.uint8, device="cuda")
            s = torch.cuda.Stream() if i == 2 else torch.cuda.current_stream()
            with torch.cuda.stream(s):
                r = vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"], bias=dev["b"],
                                   silu_grad_preactivation=policy, workspace=ws)
            torch.cuda.synchronize()
            runs.append(r)
        for r in runs[1:]:
            for a, b in zip(runs[0], r):
                assert torch.equal(a, b), policy


def test_empty_documents_change_nothing(torch_cuda):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE empty docs")
    wl = _small(14, 4000, 136, [1000, 37, 5, 1958, 1000], "f32", "f32", None)
    dev = G.to_device(wl)
    cu2 = torch.tensor([0, 0, 1000, 1000, 1037, 1042, 1042, 1042, 3000, 4000, 4000],
                       dtype=torch.int32, device="cuda")
    for policy in ("bf16", "fp32"):
        a = (vdc.conv1d_fwd(dev["x"], dev["w"], dev["cu"], bias=dev["b"]),) + tuple(
            vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"], bias=dev["b"],
                           silu_grad_preactivation=policy))
        b = (vdc.conv1d_fwd(dev["x"], dev["w"], cu2, bias=dev["b"]),) + tuple(
            vdc.conv1d_bwd(dev["x"], dev["w"], cu2, dev["dy"], bias=dev["b"],
                           silu_grad_preactivation=policy))
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u, v), policy


def test_outputs_fully_written(torch_cuda):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE poisoned outputs")
    wl = _small(15, 3333, 200, [1111, 0, 2222], "bf16", "f32", None)
    dev = G.to_device(wl)
    y = torch.full_like(dev["x"], float("nan"))
    dx = torch.full_like(dev["x"], float("nan"))
    dw = torch.full((200, 4), float("nan"), device="cuda")
    db = torch.full((200,), float("nan"), device="cuda")
    vdc.conv1d_fwd(dev["x"], dev["w"], dev["cu"], bias=dev["b"], out=y)
    vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"], bias=dev["b"], dx=dx,
                   dweight=dw, dbias=db)
    torch.cuda.synchronize()
    for t in (y, dx, dw, db):
        assert not torch.isnan(t).any()


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
def test_bf16_gradient_outputs(torch_cuda, policy):
    """BF16 dweight / dbias: each within one BF16 ulp of the oracle, plus the
    FP32-level reduction error, and rel-L2 within the policy bound + 2^-8."""
    import oracle
    import tolerance as tol
    G.say("CASE bf16 grads", policy)
    wl = _small(16, 5000, 256, [2500, 2500], "bf16", "bf16", None)
    dev = G.to_device(wl)
    _, _, dw, db = G.run_gpu(dev, policy, grad_dtype="bf16")
    x64 = oracle.decode_bf16(wl.x)
    g = oracle.backward(x64, oracle.decode_param(wl.w, "bf16"), oracle.decode_param(wl.b, "bf16"),
                        wl.cu, oracle.decode_bf16(wl.dy), policy)
    for got, ref in ((dw.float().cpu().numpy().astype(np.float64), g["dw"]),
                     (db.float().cpu().numpy().astype(np.float64), g["db"])):
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.abs(got - ref)
        assert np.all(err <= tol.ulp_bf16(ref) + 4 * tol.BOUND[policy] * rms)
        assert tol.rel_l2(got, ref) <= tol.BOUND[policy] + 2.0 ** -8
