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


def compare(wl, policy, y, dx, dw, db, cols=None, *, label=""):
    """Check GPU outputs (device tensors) on columns `cols` (all if None) against the oracle."""
    torch = torch_mod()
    if cols is None:
        cols = np.arange(wl.C)
    cols_t = torch.from_numpy(cols.astype(np.int64)).to(y.device)
    y_h = oracle.decode_bf16(bf16_bits(y.index_select(1, cols_t)))
    dx_h = oracle.decode_bf16(bf16_bits(dx.index_select(1, cols_t)))
    dw_h = dw.float().cpu().numpy().astype(np.float64)[cols]
    db_h = db.float().cpu().numpy().astype(np.float64)[cols] if db is not None else None

    x64 = oracle.decode_bf16(wl.x[:, cols])
    dy64 = oracle.decode_bf16(wl.dy[:, cols])
    w64 = oracle.decode_param(wl.w, wl.w_dtype)[cols]
    b64 = oracle.decode_param(wl.b, wl.b_dtype)[cols] if wl.b is not None else None
    f = oracle.forward(x64, w64, b64, wl.cu)
    g = oracle.backward(x64, w64, b64, wl.cu, dy64, policy)

    rep = {"label": label, "policy": policy}
    rep["y"] = tol.check_ulp(label + " y", y_h, f["y"], tol.allowance_y(f["p"], f["pabs"], f["y"]))
    a_dpre = tol.allowance_dpre(f["p"], f["pabs"], dy64, g["dpre"], policy)
    rep["dx"] = tol.check_ulp(label + " dx (%s)" % policy, dx_h, g["dx"],
                              tol.allowance_dx(w64, wl.cu, a_dpre, g["dpre"]))
    bound = tol.BOUND[policy]
    if policy == "bf16":
        flip = tol.bf16_flip(f["p"], f["pabs"], dy64)
        fw, fb = tol.flip_bound_grads(flip, x64, wl.cu)
        rep["flip_elems"] = int(np.count_nonzero(flip))
    else:
        fw, fb = np.zeros_like(g["dw"]), np.zeros_like(g["db"])
    rep["dw_rel_l2"] = tol.rel_l2(dw_h, g["dw"])
    lim = bound + np.linalg.norm(fw) / max(np.linalg.norm(g["dw"]), 1e-300)
    assert rep["dw_rel_l2"] <= lim, "%s dweight rel-L2 %.3e > %.3e" % (label, rep["dw_rel_l2"], lim)
    if db_h is not None:
        rep["db_rel_l2"] = tol.rel_l2(db_h, g["db"])
        lim = bound + np.linalg.norm(fb) / max(np.linalg.norm(g["db"]), 1e-300)
        assert rep["db_rel_l2"] <= lim, "%s dbias rel-L2 %.3e > %.3e" % (label, rep["db_rel_l2"], lim)
    say("PARITY", rep)
    return rep
