"""Shared machinery of the GPU parity tests: run the library on a workload
through the Python binding (C ABI) and compare with the FP64 oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
import tolerance as tol
from varlen_depthwise_causal_amd import workloads as W


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_device(wl, device="cuda:0"):
    torch = torch_mod()

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    def param(a, dt):
        if a is None:
            return None
        return bf16(a) if dt == "bf16" else torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return {"x": bf16(wl.x), "dy": bf16(wl.dy), "w": param(wl.w, wl.w_dtype),
            "b": param(wl.b, wl.b_dtype), "cu": torch.from_numpy(wl.cu).to(device)}


def bf16_bits(t):
    """Device bf16 tensor -> host uint16 bit patterns."""
    torch = torch_mod()
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)


def small_case(seed, S, C, lengths, w_dtype, b_dtype, sat):
    """A seeded case of the given shape; lengths "randint" draws U{0..25}
    document lengths (the Stress recipe) with a remainder document."""
    if lengths == "randint":
        rng = np.random.default_rng(seed)
        lengths = list(rng.integers(0, 26, size=S // 14))
        lengths.append(S - sum(lengths))
    return W.random_case(seed, S, C, lengths, w_dtype=w_dtype, b_dtype=b_dtype,
                         w_scale=1.0 if sat else 0.5, b_scale=0.5 if sat else 0.1, sat=sat)


@functools.lru_cache(maxsize=4)
def named(name):
    return W.make(name, workers=16)


def run_gpu(dev, policy, *, grad_dtype="f32"):
    """Forward + backward on device tensors; gradients in FP32 buffers by default."""
    torch = torch_mod()
    import varlen_depthwise_causal_amd as vdc
    y = vdc.conv1d_fwd(dev["x"], dev["w"], dev["cu"], bias=dev["b"])
    C = dev["x"].shape[-1]
    gdt = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    dw = torch.empty((C, 4), dtype=gdt, device=dev["x"].device)
    db = torch.empty((C,), dtype=gdt, device=dev["x"].device) if dev["b"] is not None else None
    res = vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"], bias=dev["b"],
                         silu_grad_preactivation=policy, dweight=dw, dbias=db)
    torch.cuda.synchronize()
    return y, res[0], res[1], (res[2] if len(res) > 2 else None)


def sample_columns(C, groups=8, seed=0):
    """Whole 8-channel groups: the first, the last and random ones in between."""
    nv = C // 8
    rng = np.random.default_rng(seed)
    pick = {0, nv - 1}
    if nv > 2:
        pick.update(int(v) for v in rng.choice(np.arange(1, nv - 1), size=min(groups - 2, nv - 2),
                                               replace=False))
    return np.concatenate([np.arange(8 * v, 8 * v + 8) for v in sorted(pick)])


def _check_columns(wl, policy, y_bits, dx_bits, cols, label):
    """Oracle and per-element rules on columns `cols`: y and dx under the
    one-ulp rule (asserted here), and the pieces of the gradient checks
    (the oracle's dw / db on these columns and, under "bf16", the flip
    bounds).  y_bits / dx_bits hold the GPU results of exactly `cols`."""
    y_h = oracle.decode_bf16(y_bits)
    dx_h = oracle.decode_bf16(dx_bits)
    x64 = oracle.decode_bf16(wl.x[:, cols])
    dy64 = oracle.decode_bf16(wl.dy[:, cols])
    w64 = oracle.decode_param(wl.w, wl.w_dtype)[cols]
    b64 = oracle.decode_param(wl.b, wl.b_dtype)[cols] if wl.b is not None else None
    f = oracle.forward(x64, w64, b64, wl.cu)
    g = oracle.backward(x64, w64, b64, wl.cu, dy64, policy)
    rep = {}
    rep["y"] = tol.check_ulp(label + " y", y_h, f["y"], tol.allowance_y(f["p"], f["pabs"], f["y"]))
    a_dpre = tol.allowance_dpre(f["p"], f["pabs"], dy64, g["dpre"], policy)
    rep["dx"] = tol.check_ulp(label + " dx (%s)" % policy, dx_h, g["dx"],
                              tol.allowance_dx(w64, wl.cu, a_dpre, g["dpre"]))
    if policy == "bf16":
        flip = tol.bf16_flip(f["p"], f["pabs"], dy64)
        fw, fb = tol.flip_bound_grads(flip, x64, wl.cu)
        rep["flip_elems"] = int(np.count_nonzero(flip))
    else:
        fw, fb = np.zeros_like(g["dw"]), np.zeros_like(g["db"])
    return rep, g["dw"], g["db"], fw, fb


def _check_gradients(label, policy, dw_h, db_h, dw64, db64, fw, fb, rep):
    bound = tol.BOUND[policy]
    rep["dw_rel_l2"] = tol.rel_l2(dw_h, dw64)
    lim = bound + np.linalg.norm(fw) / max(np.linalg.norm(dw64), 1e-300)
    assert rep["dw_rel_l2"] <= lim, "%s dweight rel-L2 %.3e > %.3e" % (label, rep["dw_rel_l2"], lim)
    if db_h is not None:
        rep["db_rel_l2"] = tol.rel_l2(db_h, db64)
        lim = bound + np.linalg.norm(fb) / max(np.linalg.norm(db64), 1e-300)
        assert rep["db_rel_l2"] <= lim, "%s dbias rel-L2 %.3e > %.3e" % (label, rep["db_rel_l2"], lim)


def compare(wl, policy, y, dx, dw, db, cols=None, *, label=""):
    """Check GPU outputs (device tensors) on columns `cols` (all if None) against the oracle."""
    torch = torch_mod()
    if cols is None:
        cols = np.arange(wl.C)
    cols_t = torch.from_numpy(cols.astype(np.int64)).to(y.device)
    y_bits = bf16_bits(y.index_select(1, cols_t))
    dx_bits = bf16_bits(dx.index_select(1, cols_t))
    dw_h = dw.float().cpu().numpy().astype(np.float64)[cols]
    db_h = db.float().cpu().numpy().astype(np.float64)[cols] if db is not None else None
    rep, dw64, db64, fw, fb = _check_columns(wl, policy, y_bits, dx_bits, cols, label)
    rep = {"label": label, "policy": policy, **rep}
    _check_gradients(label, policy, dw_h, db_h, dw64, db64, fw, fb, rep)
    say("PARITY", rep)
    return rep


def compare_all(wl, policy, y, dx, dw, db, *, label="", block=256, workers=16):
    """Every element of every column, as compare() does, for full-size
    workloads: the columns are checked in blocks of `block` (channels are
    independent, so the oracle on a block is the oracle on those columns),
    `workers` blocks at a time on host threads (the oracle's C code and
    numpy's array operations release the interpreter lock).  The gradients'
    rel-L2 and flip bounds are assembled over all columns."""
    from concurrent.futures import ThreadPoolExecutor
    y_bits, dx_bits = bf16_bits(y), bf16_bits(dx)
    dw_h = dw.float().cpu().numpy().astype(np.float64)
    db_h = db.float().cpu().numpy().astype(np.float64) if db is not None else None
    blocks = [np.arange(c0, min(c0 + block, wl.C)) for c0 in range(0, wl.C, block)]
    done = [0]

    def one(cols):
        r = _check_columns(wl, policy, np.ascontiguousarray(y_bits[:, cols]),
                           np.ascontiguousarray(dx_bits[:, cols]), cols,
                           "%s cols %d..%d" % (label, cols[0], cols[-1]))
        done[0] += 1
        say("  block %d/%d (cols %d..%d): y %d beyond 1 ulp, dx %d beyond 1 ulp"
            % (done[0], len(blocks), cols[0], cols[-1], r[0]["y"]["beyond_1ulp"],
               r[0]["dx"]["beyond_1ulp"]))
        return r

    with ThreadPoolExecutor(min(workers, len(blocks))) as pool:
        parts = list(pool.map(one, blocks))
    rep = {"label": label, "policy": policy}
    for key in ("y", "dx"):
        rs = [p[0][key] for p in parts]
        rep[key] = {"n": sum(r["n"] for r in rs), "violations": sum(r["violations"] for r in rs),
                    "beyond_1ulp": sum(r["beyond_1ulp"] for r in rs),
                    "max_ulps": max(r["max_ulps"] for r in rs)}
    if policy == "bf16":
        rep["flip_elems"] = sum(p[0]["flip_elems"] for p in parts)
    dw64 = np.concatenate([p[1] for p in parts])
    db64 = np.concatenate([p[2] for p in parts])
    fw = np.concatenate([p[3] for p in parts])
    fb = np.concatenate([p[4] for p in parts])
    _check_gradients(label, policy, dw_h, db_h, dw64, db64, fw, fb, rep)
    say("PARITY", rep)
    return rep
