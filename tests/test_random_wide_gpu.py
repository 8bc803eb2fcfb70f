"""Seeded random shapes over the whole planner, every element against the
oracle under both policies: C up to 6400 with a third of the shapes at
multiples of 256 from 1024 (column-block lanes of the backward when bands
are short) and a third below 1024 at any multiple of 8 (rows not a
multiple of 128 bytes: the forward's split stores, per-workgroup partial
rows), S up to 40000 with S*C <= 3e6, dense, single and random documents,
empty documents inserted, FP32 or BF16 parameters, bias or none, saturated
inputs.  VDC_RANDOM_WIDE_CASES sets the number of shapes (default 60)."""
import os

import numpy as np
import pytest

import gpu_cases as G

pytestmark = pytest.mark.gpu


def _shapes(n, seed=7):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = rng.random()
        if kind < 0.35:
            C = 256 * int(rng.integers(4, 26))
        elif kind < 0.7:
            C = 8 * int(rng.integers(1, 128))
        else:
            C = 8 * int(rng.integers(128, 801))
        S = int(rng.integers(1, max(2, min(40000, 3_000_000 // C))))
        mode = rng.random()
        lengths, left = [], S
        while left > 0:
            if mode < 0.3:
                n_t = int(rng.integers(0, 26))
            elif mode < 0.5:
                n_t = left
            else:
                k = rng.random()
                n_t = 0 if k < 0.1 else (1 if k < 0.2 else int(rng.integers(1, max(2, S // 3))))
            n_t = min(n_t, left)
            lengths.append(n_t)
            left -= n_t
        if rng.random() < 0.2:
            lengths.insert(int(rng.integers(0, len(lengths) + 1)), 0)
        w_dt = "bf16" if rng.random() < 0.3 else "f32"
        b_dt = None if rng.random() < 0.25 else ("bf16" if rng.random() < 0.3 else "f32")
        sat = (0.02, 60.0) if rng.random() < 0.15 else None
        out.append(("wide%03d_s%d_c%d" % (i, S, C), 7000 + i, S, C, lengths, w_dt, b_dt, sat))
    return out


WIDE = _shapes(int(os.environ.get("VDC_RANDOM_WIDE_CASES", "60")))


@pytest.fixture(scope="module")
def torch_cuda():
    torch = G.torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
@pytest.mark.parametrize("case", WIDE, ids=[c[0] for c in WIDE])
def test_random_wide_all_elements(torch_cuda, case, policy):
    label, seed, S, C, lengths, w_dt, b_dt, sat = case
    G.say("CASE", label, policy)
    wl = G.small_case(seed, S, C, lengths, w_dt, b_dt, sat)
    dev = G.to_device(wl)
    y, dx, dw, db = G.run_gpu(dev, policy)
    G.compare(wl, policy, y, dx, dw, db, label=label)
