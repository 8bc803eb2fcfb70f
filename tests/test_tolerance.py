"""The acceptance rules themselves (CPU only): exact roundings of the oracle
pass them, results two ulps off fail them, and the allowance only matters
where the taps cancel."""
import numpy as np

import oracle
import tolerance as tol
from varlen_depthwise_causal_amd import workloads as W


def _case():
    wl = W.random_case(3, 3000, 64, [0, 5, 1, 2000, 994], sat=(0.01, 60.0), w_scale=1.0, b_scale=0.5)
    x = oracle.decode_bf16(wl.x)
    dy = oracle.decode_bf16(wl.dy)
    w = oracle.decode_f32(wl.w)
    b = oracle.decode_f32(wl.b)
    return wl, x, dy, w, b


def test_ulp_bf16():
    v = np.array([1.0, 1.5, 2.0 - 1e-12, 2.0, -3.0, 0.0, 1e-45])
    assert list(tol.ulp_bf16(v)) == [2 ** -7, 2 ** -7, 2 ** -7, 2 ** -6, 2 ** -6, 2 ** -133, 2 ** -133]


def test_rounded_oracle_passes_and_shifted_fails():
    wl, x, dy, w, b = _case()
    f = oracle.forward(x, w, b, wl.cu)
    y_r = oracle.decode_bf16(oracle.bf16_rne(f["y"]))
    a_y = tol.allowance_y(f["p"], f["pabs"], f["y"])
    rep = tol.check_ulp("y", y_r, f["y"], a_y)
    assert rep["beyond_1ulp"] == 0
    # the allowance exceeds half an ulp only where the taps nearly cancel
    assert np.mean(a_y > 0.5 * tol.ulp_bf16(f["y"])) < 1e-2
    off = y_r + 2.5 * tol.ulp_bf16(f["y"])
    try:
        tol.check_ulp("y", off, f["y"], a_y)
    except AssertionError:
        pass
    else:
        raise AssertionError("2.5 ulp error accepted")
    for policy in ("bf16", "fp32"):
        g = oracle.backward(x, w, b, wl.cu, dy, policy)
        a_dpre = tol.allowance_dpre(f["p"], f["pabs"], dy, g["dpre"], policy)
        a_dx = tol.allowance_dx(w, wl.cu, a_dpre, g["dpre"])
        dx_r = oracle.decode_bf16(oracle.bf16_rne(g["dx"]))
        tol.check_ulp("dx", dx_r, g["dx"], a_dx)
        assert np.mean(a_dx > 0.5 * tol.ulp_bf16(g["dx"])) < 2e-2


def test_rel_l2():
    r = np.array([3.0, 4.0])
    assert tol.rel_l2(r, r) == 0.0
    assert abs(tol.rel_l2(r + np.array([0.0, 5e-5]), r) - 1e-5) < 1e-12


def test_silu_derivative_bounds():
    z = np.linspace(-60, 60, 1200001)
    g = tol.silu_grad64(z)
    assert abs(tol.silu_grad2_64(tol.Z_CRIT)) < 1e-12
    assert np.max(g) <= tol.silu_grad64(tol.Z_CRIT) + 1e-12
    assert np.min(g) >= tol.silu_grad64(-tol.Z_CRIT) - 1e-12
    g2 = tol.silu_grad2_64(z)
    g3 = np.gradient(g2, z)
    assert np.max(np.abs(g3)) < 1.0
