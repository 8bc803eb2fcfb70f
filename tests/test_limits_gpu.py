"""The path at the edges of its size range: a two-stage reduce (more than
2048 partial rows), the largest channel count (a band's rows capped so one
wave's span fits 32-bit offsets) and the largest token count S = 2^31 - 1
(row indices near the top of int32; ~140 GB of device memory).

Inputs too large for the oracle are built on the device by repeating a
seeded block of rows (or of columns), so every output the test compares can
be computed by the oracle from the block alone.  Token-sliced comparisons
keep only rows whose window lies inside the slice; the weight and bias
gradients at S = 2^31 - 1 are compared with a sum over tiles of the block:
a tile with no document start in or just before it contributes the same
terms wherever it lies.
"""
import numpy as np
import pytest

import gpu_cases as G
import oracle
import tolerance as tol
from varlen_depthwise_causal_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
def test_two_stage_reduce_all_elements(torch_cuda, policy):
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE two-stage reduce", policy)
    S, C = 1 << 21, 8
    rng = np.random.default_rng(40)
    lengths = [0, 3, 1, 0, 5000] + list(rng.integers(1, 40000, size=60))
    lengths.append(S - sum(lengths))
    assert lengths[-1] > 0
    plan = vdc.conv1d_plan("bwd", S, C, policy)
    assert plan["bands"] > 2048 and plan["red_stage1"] == -(-plan["bands"] // 2048)
    wl = W.random_case(40, S, C, lengths, w_dtype="f32", b_dtype="f32")
    dev = G.to_device(wl)
    y, dx, dw, db = G.run_gpu(dev, policy)
    G.compare(wl, policy, y, dx, dw, db, label="two-stage %d partial rows" % plan["bands"])
    _, dx2, dw2, db2 = G.run_gpu(dev, policy)
    assert torch_cuda.equal(dx, dx2) and torch_cuda.equal(dw, dw2) and torch_cuda.equal(db, db2)


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
def test_max_channels(torch_cuda, policy):
    """C = 2^20 (rows of 2 MiB): the planner caps T so one wave's rows span
    less than 2^31 bytes; compared on sampled columns, every token."""
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE C=2^20", policy)
    S, C, CB = 600, 1 << 20, 4096
    lengths = [0, 250, 0, 350]
    for d in ("fwd", "bwd"):
        p = vdc.conv1d_plan(d, S, C, policy)
        span = (-(-64 // (C // p["vec"])) + 1) * p["rows"] + 8
        assert p["rows"] < S and p["bands"] >= 2 and span * C * 2 < 2 ** 31
    blk = W.random_case(42, S, CB, lengths, w_dtype="f32", b_dtype="f32")
    wrng = np.random.default_rng(43)
    w = wrng.uniform(-0.5, 0.5, size=(C, 4)).astype(np.float32)
    b = wrng.normal(0.0, 0.1, size=(C,)).astype(np.float32)
    dev_blk = G.to_device(blk)
    x = dev_blk["x"].repeat(1, C // CB)
    dy = dev_blk["dy"].repeat(1, C // CB)
    w_t, b_t = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    y = vdc.conv1d_fwd(x, w_t, dev_blk["cu"], bias=b_t)
    dw = torch.empty((C, 4), device="cuda")
    db = torch.empty((C,), device="cuda")
    dx, dw, db = vdc.conv1d_bwd(x, w_t, dev_blk["cu"], dy, bias=b_t,
                                silu_grad_preactivation=policy, dweight=dw, dbias=db)
    torch.cuda.synchronize()
    cols = G.sample_columns(C, groups=16, seed=44)
    cols_t = torch.from_numpy(cols.astype(np.int64)).cuda()
    loc = W.Workload("c2^20 sample", S, len(cols), blk.x[:, cols % CB], blk.dy[:, cols % CB],
                     w[cols], "f32", b[cols], "f32", blk.cu, (policy,))
    G.compare(loc, policy, y.index_select(1, cols_t), dx.index_select(1, cols_t),
              dw.index_select(0, cols_t), db.index_select(0, cols_t), label="C=2^20")
    del x, dy, y, dx
    torch.cuda.empty_cache()


def _rows_of(xb, rows):
    return xb[np.asarray(rows) % xb.shape[0]]


def _local_cu(starts, a, b):
    inner = sorted(int(s) - a for s in starts if a < s < b)
    return np.asarray([0] + inner + [b - a], dtype=np.int32)


def _tile_terms(blk, w64, b64, starts, a, b, policy):
    """dweight / dbias terms of rows [a, b) (FP64), with their in-document
    history: rows a-3 .. a-1 ride along and their own terms are removed."""
    h = max(a - 3, 0)
    x64 = oracle.decode_bf16(_rows_of(blk.x, range(h, b)))
    dy64 = oracle.decode_bf16(_rows_of(blk.dy, range(h, b)))
    cu = _local_cu(starts, h, b)
    g = oracle.backward(x64, w64, b64, cu, dy64, policy, want=("dw", "db"))
    if a == h:
        return g["dw"], g["db"]
    k = a - h
    cu_h = np.asarray([c for c in cu if c < k] + [k], dtype=np.int32)
    gh = oracle.backward(x64[:k], w64, b64, cu_h, dy64[:k], policy, want=("dw", "db"))
    return g["dw"] - gh["dw"], g["db"] - gh["db"]


def test_max_tokens(torch_cuda):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    S, C, TILE = (1 << 31) - 1, 8, 1 << 16
    free, _ = torch.cuda.mem_get_info()
    need = 4 * S * C * 2 + vdc.workspace_bytes("bwd", S, C) + (4 << 30)
    if free < need:
        pytest.skip("needs %.0f GB of device memory, %.0f GB free" % (need / 1e9, free / 1e9))
    G.say("CASE S=2^31-1 C=8")
    for d in ("fwd", "bwd"):
        p = vdc.conv1d_plan(d, S, C)
        assert p["bands"] * p["rows"] >= S
    assert vdc.conv1d_plan("bwd", S, C)["red_stage1"] > 0
    blk = W.random_case(45, TILE, C, [TILE], w_dtype="f32", b_dtype="f32")
    dev_blk = G.to_device(blk)
    x = torch.empty((S, C), dtype=torch.bfloat16, device="cuda")
    dy = torch.empty_like(x)
    step = 1 << 26
    for a in range(0, S, step):
        n = min(step, S - a)
        reps = -(-n // TILE)
        x[a:a + n] = dev_blk["x"].repeat(reps, 1)[:n]
        dy[a:a + n] = dev_blk["dy"].repeat(reps, 1)[:n]
    starts = [0, 1000, 1 << 30, (1 << 30) + 5, S - 100]
    cu = torch.tensor(starts + [S], dtype=torch.int32, device="cuda")
    w64 = oracle.decode_param(blk.w, "f32")
    b64 = oracle.decode_param(blk.b, "f32")
    y = vdc.conv1d_fwd(x, dev_blk["w"], cu, bias=dev_blk["b"])
    slices = [(0, 4096), ((1 << 30) - 2048, (1 << 30) + 2048), ((1 << 30) + 70000, (1 << 30) + 74096),
              (S - 4096, S)]
    for policy in ("bf16", "fp32"):
        dw = torch.empty((C, 4), device="cuda")
        db = torch.empty((C,), device="cuda")
        dx, dw, db = vdc.conv1d_bwd(x, dev_blk["w"], cu, dy, bias=dev_blk["b"],
                                    silu_grad_preactivation=policy, dweight=dw, dbias=db)
        torch.cuda.synchronize()
        for a, b in slices:
            x64 = oracle.decode_bf16(_rows_of(blk.x, range(a, b)))
            dy64 = oracle.decode_bf16(_rows_of(blk.dy, range(a, b)))
            cu_l = _local_cu(starts, a, b)
            f = oracle.forward(x64, w64, b64, cu_l)
            g = oracle.backward(x64, w64, b64, cu_l, dy64, policy)
            # rows whose window (x rows t-3 .. t, dpre rows t .. t+3) lies in
            # the slice, unless the slice starts the data or ends it
            ok_y = slice(0 if a == 0 else 3, b - a)
            ok_dx = slice(0 if a == 0 else 3, b - a if b == S else b - a - 3)
            y_h = oracle.decode_bf16(G.bf16_bits(y[a:b]))
            dx_h = oracle.decode_bf16(G.bf16_bits(dx[a:b]))
            tol.check_ulp("S=2^31-1 y [%d, %d)" % (a, b), y_h[ok_y], f["y"][ok_y],
                          tol.allowance_y(f["p"], f["pabs"], f["y"])[ok_y])
            a_dpre = tol.allowance_dpre(f["p"], f["pabs"], dy64, g["dpre"], policy)
            a_dx = tol.allowance_dx(w64, cu_l, a_dpre, g["dpre"])
            tol.check_ulp("S=2^31-1 dx %s [%d, %d)" % (policy, a, b), dx_h[ok_dx], g["dx"][ok_dx],
                          a_dx[ok_dx])
        # gradients: tiles 0, 2^14 and the last one hold the document starts;
        # every other tile (all complete, none within 2 rows of a start)
        # contributes what tile 1 does.
        ntiles = -(-S // TILE)
        special = sorted({s // TILE for s in starts} | {ntiles - 1})
        for s in starts:
            assert s % TILE < TILE - 2 or s // TILE + 1 in special
        dw_ref = np.zeros((C, 4))
        db_ref = np.zeros(C)
        for i in special:
            tw, tb = _tile_terms(blk, w64, b64, starts, i * TILE, min((i + 1) * TILE, S), policy)
            dw_ref += tw
            db_ref += tb
        assert 1 not in special
        pw, pb = _tile_terms(blk, w64, b64, starts, TILE, 2 * TILE, policy)
        dw_ref += (ntiles - len(special)) * pw
        db_ref += (ntiles - len(special)) * pb
        dw_h = dw.cpu().numpy().astype(np.float64)
        db_h = db.cpu().numpy().astype(np.float64)
        # under "bf16" each tile's rare BF16 boundary flips may move the sums
        # (the same bound as elsewhere, summed over tiles)
        lim_w = lim_b = tol.BOUND[policy]
        if policy == "bf16":
            x_t = oracle.decode_bf16(blk.x)
            f_t = oracle.forward(x_t, w64, b64, blk.cu)
            flip = tol.bf16_flip(f_t["p"], f_t["pabs"], oracle.decode_bf16(blk.dy))
            fw, fb = tol.flip_bound_grads(flip, x_t, blk.cu)
            lim_w += ntiles * np.linalg.norm(fw) / np.linalg.norm(dw_ref)
            lim_b += ntiles * np.linalg.norm(fb) / np.linalg.norm(db_ref)
        G.say("S=2^31-1", policy, "dw rel-L2", tol.rel_l2(dw_h, dw_ref), "db rel-L2",
              tol.rel_l2(db_h, db_ref))
        assert tol.rel_l2(dw_h, dw_ref) <= lim_w
        assert tol.rel_l2(db_h, db_ref) <= lim_b
        del dx
    del x, dy, y
    torch.cuda.empty_cache()
