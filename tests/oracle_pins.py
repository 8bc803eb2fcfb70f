"""Pins of the FP64 oracle to things other than itself.

Each ``pin_*`` function takes a loaded ``oracle.Oracle`` and raises
``AssertionError`` on a mismatch.  ``tests/test_oracle.py`` runs them on the
real oracle; ``tests/test_oracle_mutants.py`` runs them on copies of the
oracle with a planted mistake and requires that every mistake is caught.

What each pin compares against:

* worked examples under ``tests/golden/`` (hand-derived, exact arithmetic);
* torch float64 autograd of ``F.conv1d(groups=C)`` over each document with
  3 tokens of zero left padding, followed by ``F.silu`` (a library routine);
* central finite differences of the forward;
* closed forms (identity tap, shift taps, every document of length 1);
* invariants (document split locality, document permutation, empty
  documents, S = 0, the two SiLU' policies coinciding when every
  preactivation is BF16-representable);
* exhaustive / brute-force checks of the BF16 decode and rounding.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers --

def read_golden(name):
    vals = {"p": {}, "dx": {}}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            if key in ("p", "dx"):
                vals[key][int(rest[0])] = float(rest[1])
            elif key in ("S", "C"):
                vals[key] = int(rest[0])
            elif key == "cu_seqlens":
                vals[key] = np.array([int(v) for v in rest], np.int32)
            else:
                vals[key] = np.array([float(v) for v in rest], np.float64)
    return vals


def _rng(seed):
    return np.random.default_rng(seed)


def _random_problem(seed, lengths, C, bias=True, scale=1.0):
    rng = _rng(seed)
    S = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = rng.standard_normal((S, C)) * scale
    w = rng.uniform(-0.5, 0.5, (C, 4))
    b = rng.normal(0, 0.3, C) if bias else None
    dy = rng.standard_normal((S, C))
    return x, w, b, cu, dy


def torch_reference(orc, x, w, b, cu, dy, policy):
    """Forward and backward through torch float64 autograd, per document.

    Under the "bf16" policy the derivative of SiLU is taken (by autograd) at
    the BF16 rounding of torch's preactivation, rounded by ``orc.bf16_rne``
    (which the BF16 pins check exhaustively).
    """
    import torch
    import torch.nn.functional as F

    S, C = x.shape
    X = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    W = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    B = torch.tensor(b, dtype=torch.float64, requires_grad=True) if b is not None else None
    parts = []
    for d in range(len(cu) - 1):
        s, e = int(cu[d]), int(cu[d + 1])
        if s == e:
            continue
        seg = F.pad(X[s:e].T.unsqueeze(0), (3, 0))          # [1, C, 3 + L]
        p = F.conv1d(seg, W.unsqueeze(1), groups=C)         # [1, C, L]
        p = p[0].T
        if B is not None:
            p = p + B
        parts.append(p)
    P = torch.cat(parts) if parts else torch.zeros((0, C), dtype=torch.float64)
    Y = F.silu(P)
    DY = torch.tensor(dy, dtype=torch.float64)
    if policy == "fp32":
        Z = P
    else:
        zbits = orc.bf16_rne(P.detach().numpy())
        Z = torch.tensor(orc.decode_bf16(zbits), dtype=torch.float64)
    Z = Z.detach().requires_grad_(True)
    (dpre,) = torch.autograd.grad(F.silu(Z), Z, grad_outputs=DY)
    params = [X, W] + ([B] if B is not None else [])
    grads = torch.autograd.grad(P, params, grad_outputs=dpre, allow_unused=True)
    out = {"p": P.detach().numpy(), "y": Y.detach().numpy(), "dpre": dpre.numpy(),
           "dx": grads[0].numpy(), "dw": grads[1].numpy()}
    out["db"] = grads[2].numpy() if B is not None else dpre.sum(0).numpy()
    return out


def _close(a, b, scale, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.abs(a - b)
    lim = tol * np.maximum(np.asarray(scale, np.float64), 1e-300)
    bad = err > lim
    assert not bad.any(), "%s: %d mismatches, worst %.3e (limit %.3e)" % (
        what, int(bad.sum()), float(err.max()), float(np.max(lim)))


# ------------------------------------------------------------------ BF16 --

def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def pin_decode_bf16_exhaustive(orc):
    """Every finite BF16 pattern decodes to torch's own BF16 -> float64 value."""
    import torch
    bits = _all_finite_bf16()
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.decode_bf16(bits)
    assert np.array_equal(got, ref), "bf16 decode differs from torch"
    assert np.array_equal(np.signbit(got), np.signbit(ref)), "bf16 decode sign of zero"


def pin_decode_f32(orc):
    rng = _rng(11)
    v = (rng.standard_normal(4096) * np.exp(rng.uniform(-80, 80, 4096))).astype(np.float32)
    v[:4] = [0.0, -0.0, 1e-45, -3.4e38]
    assert np.array_equal(orc.decode_f32(v), v.astype(np.float64))


def pin_bf16_rne_fixed_points(orc):
    """Every finite BF16 value rounds to itself."""
    bits = _all_finite_bf16()
    vals = orc.decode_bf16(bits)
    got = orc.bf16_rne(vals)
    same = (got == bits) | ((vals == 0) & ((got & 0x7FFF) == 0))
    assert same.all(), "bf16 fixed points not preserved"


def pin_bf16_rne_ties_and_brackets(orc):
    """Midpoints go to the even neighbour; other values to the nearer one.

    The nearer neighbour is decided in exact rational arithmetic.
    """
    pos = np.arange(0x0000, 0x7F80, dtype=np.uint16)       # +0 .. largest finite
    lo_vals = orc.decode_bf16(pos[:-1])
    hi_vals = orc.decode_bf16(pos[1:])
    mids = (lo_vals + hi_vals) / 2.0                       # exact in binary64
    got = orc.bf16_rne(mids)
    want = np.where((pos[:-1] & 1) == 0, pos[:-1], pos[1:])
    assert np.array_equal(got, want), "ties not to even"
    assert np.array_equal(orc.bf16_rne(-mids), want | 0x8000), "negative ties"
    rng = _rng(12)
    idx = rng.integers(0, pos.size - 1, 3000)
    frac = rng.uniform(0, 1, idx.size)
    v = lo_vals[idx] + frac * (hi_vals[idx] - lo_vals[idx])
    got = orc.bf16_rne(v)
    for i in range(idx.size):
        a, b, vi = Fraction(float(lo_vals[idx[i]])), Fraction(float(hi_vals[idx[i]])), Fraction(float(v[i]))
        if vi - a < b - vi:
            want_i = pos[idx[i]]
        elif vi - a > b - vi:
            want_i = pos[idx[i] + 1]
        else:
            want_i = pos[idx[i]] if pos[idx[i]] % 2 == 0 else pos[idx[i] + 1]
        assert got[i] == want_i, "value %r rounded to %#x, want %#x" % (float(v[i]), got[i], want_i)


def pin_bf16_rne_vs_torch_f32(orc):
    """Single rounding of binary32 inputs agrees with torch's float32 -> bfloat16."""
    import torch
    rng = _rng(13)
    u = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_rne(f.astype(np.float64))
    assert np.array_equal(got, ref), "disagrees with torch on %d values" % int((got != ref).sum())


# ------------------------------------------------------------------ SiLU --

def pin_silu_scalars(orc):
    """SiLU and its derivative against mpmath at 50 digits."""
    import mpmath
    mpmath.mp.dps = 50
    for z in [-800.0, -300.0, -100.0, -88.0, -20.0, -1.2784645, -1.0, -0.25, 0.0,
              1e-8, 0.5, 1.0, 3.0, 20.0, 88.0, 300.0]:
        zm = mpmath.mpf(z)
        s = 1 / (1 + mpmath.e ** (-zm))
        want_y = float(zm * s)
        want_g = float(s + zm * s * (1 - s))
        got_y, got_g = orc.silu(z), orc.silu_grad(z)
        assert abs(got_y - want_y) <= 4e-16 * abs(want_y) + 1e-300, ("silu", z, got_y, want_y)
        assert abs(got_g - want_g) <= 1e-15 * max(abs(want_g), 1e-300) + 1e-16 * (abs(z) * abs(float(s))), \
            ("silu'", z, got_g, want_g)


# --------------------------------------------------------- worked examples --

def pin_worked_forward(orc):
    g = read_golden("worked_forward.txt")
    x = g["x"].reshape(g["S"], g["C"])
    out = orc.forward(x, g["weight"].reshape(g["C"], 4), g.get("bias"), g["cu_seqlens"])
    for t, want in g["p"].items():
        assert out["p"][t, 0] == want, ("p", t, out["p"][t, 0], want)


def _check_worked_backward(orc, name):
    g = read_golden(name)
    S, C = g["S"], g["C"]
    for policy in ("bf16", "fp32"):
        out = orc.backward(g["x"].reshape(S, C), g["weight"].reshape(C, 4), g.get("bias"),
                           g["cu_seqlens"], g["dy"].reshape(S, C), policy)
        for t, want in g["dx"].items():
            assert out["dx"][t, 0] == want, (name, policy, "dx", t, out["dx"][t, 0], want)
        assert np.array_equal(out["dw"].ravel(), g["dweight"]), (name, policy, out["dw"], g["dweight"])
        assert out["db"][0] == g["dbias"][0], (name, policy, out["db"], g["dbias"])


def pin_worked_backward_dx(orc):
    _check_worked_backward(orc, "worked_backward_dx.txt")


def pin_worked_backward_dw(orc):
    _check_worked_backward(orc, "worked_backward_dw.txt")


# ------------------------------------------------- library cross-checks --

_LENGTHS = [0, 1, 2, 3, 5, 0, 9, 17]


def _cross_check(orc, policy, bias):
    x, w, b, cu, dy = _random_problem(21 + bias, _LENGTHS, 8, bias=bias)
    ref = torch_reference(orc, x, w, b, cu, dy, policy)
    f = orc.forward(x, w, b, cu)
    scale = f["pabs"]
    _close(f["p"], ref["p"], scale, 1e-14, "p vs torch conv1d")
    ref_abs = torch_reference(orc, np.abs(x), np.abs(w), None if b is None else np.abs(b),
                              cu, dy, policy)
    _close(f["pabs"], ref_abs["p"], scale, 1e-14, "pabs vs torch conv1d of |x|, |w|, |b|")
    _close(f["y"], ref["y"], scale + np.abs(ref["y"]), 1e-14, "y vs torch silu")
    g = orc.backward(x, w, b, cu, dy, policy)
    dscale = np.abs(dy) * 1.2
    _close(g["dpre"], ref["dpre"], dscale, 1e-13, "dpre vs torch (%s)" % policy)
    _close(g["dx"], ref["dx"], 1.0, 1e-13, "dx vs torch (%s)" % policy)
    _close(g["dw"], ref["dw"], 1.0 + np.abs(ref["dw"]), 1e-13, "dw vs torch (%s)" % policy)
    _close(g["db"], ref["db"], 1.0 + np.abs(ref["db"]), 1e-13, "db vs torch (%s)" % policy)


def pin_torch_fp32_bias(orc):
    _cross_check(orc, "fp32", True)


def pin_torch_fp32_nobias(orc):
    _cross_check(orc, "fp32", False)


def pin_torch_bf16_bias(orc):
    _cross_check(orc, "bf16", True)


def pin_torch_bf16_nobias(orc):
    _cross_check(orc, "bf16", False)


# ---------------------------------------------------- finite differences --

def pin_finite_differences_fp32(orc):
    """Central differences of L = sum dy * SiLU(p) match the "fp32" gradients."""
    lengths = [0, 1, 2, 3, 5, 8]
    x, w, b, cu, dy = _random_problem(31, lengths, 3)
    h = 1e-6

    def loss(xx, ww, bb):
        return float(np.sum(dy * orc.forward(xx, ww, bb, cu, want=("y",))["y"]))

    g = orc.backward(x, w, b, cu, dy, "fp32")
    for (t, c) in [(i, j) for i in range(x.shape[0]) for j in range(x.shape[1])]:
        xp, xm = x.copy(), x.copy()
        xp[t, c] += h
        xm[t, c] -= h
        fd = (loss(xp, w, b) - loss(xm, w, b)) / (2 * h)
        assert abs(fd - g["dx"][t, c]) <= 1e-7 * max(1.0, abs(fd)), ("dx", t, c, fd, g["dx"][t, c])
    for c in range(w.shape[0]):
        for k in range(4):
            wp, wm = w.copy(), w.copy()
            wp[c, k] += h
            wm[c, k] -= h
            fd = (loss(x, wp, b) - loss(x, wm, b)) / (2 * h)
            assert abs(fd - g["dw"][c, k]) <= 1e-7 * max(1.0, abs(fd)), ("dw", c, k, fd, g["dw"][c, k])
        bp, bm = b.copy(), b.copy()
        bp[c] += h
        bm[c] -= h
        fd = (loss(x, w, bp) - loss(x, w, bm)) / (2 * h)
        assert abs(fd - g["db"][c]) <= 1e-7 * max(1.0, abs(fd)), ("db", c, fd, g["db"][c])


# ------------------------------------------------ closed forms, invariants --

def pin_identity_tap(orc):
    """weight = e3, no bias: y = SiLU(x) (torch), and both policies coincide."""
    import torch
    import torch.nn.functional as F
    rng = _rng(41)
    lengths = [4, 0, 7, 1, 12]
    S, C = sum(lengths), 8
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = orc.decode_bf16(orc.bf16_rne(rng.standard_normal((S, C)) * 3))
    w = np.zeros((C, 4))
    w[:, 3] = 1.0
    f = orc.forward(x, w, None, cu)
    assert np.array_equal(f["p"], x)
    ref = F.silu(torch.tensor(x, dtype=torch.float64)).numpy()
    _close(f["y"], ref, np.abs(ref) + 1e-300, 1e-15, "y = silu(x)")
    dy = rng.standard_normal((S, C))
    a = orc.backward(x, w, None, cu, dy, "bf16")
    bb = orc.backward(x, w, None, cu, dy, "fp32")
    for k in ("dpre", "dx", "dw", "db"):
        assert np.array_equal(a[k], bb[k]), k
    assert np.array_equal(a["dx"], a["dpre"])          # dx = 1 * dpre at the same token


def pin_shift_taps(orc):
    """weight = e_k: p[t] = x[t-(3-k)] inside the document, 0 in its first 3-k tokens."""
    rng = _rng(42)
    lengths = [2, 5, 0, 1, 9]
    S, C = sum(lengths), 8
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = rng.standard_normal((S, C))
    for k in range(4):
        w = np.zeros((C, 4))
        w[:, k] = 1.0
        p = orc.forward(x, w, None, cu, want=("p",))["p"]
        lag = 3 - k
        for d in range(len(lengths)):
            s, e = cu[d], cu[d + 1]
            for t in range(s, e):
                want = x[t - lag] if t - lag >= s else np.zeros(C)
                assert np.array_equal(p[t], want), (k, t)


def pin_all_length_one(orc):
    """Every document one token long: only the current tap survives."""
    rng = _rng(43)
    S, C = 13, 8
    cu = np.arange(S + 1, dtype=np.int32)
    x = rng.standard_normal((S, C))
    w = rng.uniform(-0.5, 0.5, (C, 4))
    b = rng.normal(0, 0.3, C)
    dy = rng.standard_normal((S, C))
    f = orc.forward(x, w, b, cu)
    assert np.array_equal(f["p"], w[:, 3] * x + b)
    g = orc.backward(x, w, b, cu, dy, "fp32")
    assert np.array_equal(g["dx"], w[:, 3] * g["dpre"])
    assert np.all(g["dw"][:, :3] == 0.0)
    _close(g["dw"][:, 3], np.sum(g["dpre"] * x, 0), 1.0, 1e-15, "dw3")


def pin_split_locality(orc):
    """Splitting a document at j changes y only at tokens j, j+1, j+2."""
    x, w, b, cu, dy = _random_problem(44, [40], 8)
    whole = orc.forward(x, w, b, cu)["y"]
    j = 17
    split = orc.forward(x, w, b, np.array([0, j, 40], np.int32))["y"]
    changed = np.any(whole != split, axis=1)
    assert list(np.nonzero(changed)[0]) == [j, j + 1, j + 2]


def pin_doc_permutation(orc):
    """Permuting documents permutes the per-token outputs; dw, db are unchanged."""
    lengths = [3, 0, 11, 1, 6, 2]
    x, w, b, cu, dy = _random_problem(45, lengths, 8)
    order = [4, 2, 0, 5, 1, 3]
    rows = np.concatenate([np.arange(cu[d], cu[d + 1]) for d in order]).astype(int)
    cu2 = np.concatenate([[0], np.cumsum([lengths[d] for d in order])]).astype(np.int32)
    for policy in ("bf16", "fp32"):
        a = orc.backward(x, w, b, cu, dy, policy)
        c = orc.backward(x[rows], w, b, cu2, dy[rows], policy)
        assert np.array_equal(a["dx"][rows], c["dx"])
        assert np.array_equal(a["dpre"][rows], c["dpre"])
        _close(a["dw"], c["dw"], 1.0, 1e-14, "dw under permutation")
        _close(a["db"], c["db"], 1.0, 1e-14, "db under permutation")
    fa = orc.forward(x, w, b, cu)["y"]
    fc = orc.forward(x[rows], w, b, cu2)["y"]
    assert np.array_equal(fa[rows], fc)


def pin_empty_documents(orc):
    """Repeating cu_seqlens values (empty documents) changes nothing, bitwise."""
    lengths = [5, 9, 3]
    x, w, b, cu, dy = _random_problem(46, lengths, 8)
    cu2 = np.array([0, 0, 5, 5, 5, 14, 17, 17], np.int32)
    for policy in ("bf16", "fp32"):
        a = orc.backward(x, w, b, cu, dy, policy)
        c = orc.backward(x, w, b, cu2, dy, policy)
        for k in a:
            assert np.array_equal(a[k], c[k]), k
    assert np.array_equal(orc.forward(x, w, b, cu)["y"], orc.forward(x, w, b, cu2)["y"])


def pin_zero_tokens(orc):
    """S == 0: empty outputs and exactly zero gradients."""
    x = np.zeros((0, 8))
    w = np.ones((8, 4))
    b = np.ones(8)
    for cu in (np.array([0], np.int32), np.array([0, 0, 0], np.int32)):
        f = orc.forward(x, w, b, cu)
        assert f["y"].shape == (0, 8)
        g = orc.backward(x, w, b, cu, x, "bf16")
        assert np.all(g["dw"] == 0) and np.all(g["db"] == 0) and g["dx"].shape == (0, 8)


def pin_policies_coincide_on_bf16_preactivations(orc):
    """If every preactivation is a BF16 value, the two policies are identical."""
    rng = _rng(47)
    lengths = [6, 0, 10, 3]
    S, C = sum(lengths), 8
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = rng.integers(-3, 4, (S, C)).astype(np.float64)
    w = rng.choice([0.0, 0.25, -0.25, 0.5, -0.5], (C, 4))
    dy = rng.standard_normal((S, C))
    p = orc.forward(x, w, None, cu, want=("p",))["p"]
    assert np.array_equal(orc.decode_bf16(orc.bf16_rne(p)), p)
    a = orc.backward(x, w, None, cu, dy, "bf16")
    c = orc.backward(x, w, None, cu, dy, "fp32")
    for k in a:
        assert np.array_equal(a[k], c[k]), k


def pin_policies_differ_otherwise(orc):
    """With generic inputs "bf16" evaluates SiLU' at the rounded value: dpre differs."""
    x, w, b, cu, dy = _random_problem(48, [30], 8)
    a = orc.backward(x, w, b, cu, dy, "bf16")
    c = orc.backward(x, w, b, cu, dy, "fp32")
    assert not np.array_equal(a["dpre"], c["dpre"])
    rel = np.abs(a["dpre"] - c["dpre"]) / np.maximum(np.abs(c["dpre"]), 1e-30)
    assert np.median(rel) < 1e-2


def pin_malformed_cu_rejected(orc):
    from oracle import OracleError
    x = np.zeros((4, 8))
    w = np.zeros((8, 4))
    for cu in ([0, 3], [1, 4], [0, 3, 2, 4], []):
        try:
            orc.forward(x, w, None, np.array(cu, np.int32))
        except OracleError:
            continue
        raise AssertionError("accepted malformed cu_seqlens %r" % (cu,))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def first_failure(orc):
    """Name and message of the first pin that fails, or None."""
    for fn in ALL_PINS:
        try:
            fn(orc)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            return "%s: %s: %s" % (fn.__name__, type(exc).__name__, str(exc)[:200])
    return None


def run_all(orc):
    """Run every pin; returns {name: None | failure message}."""
    res = {}
    for fn in ALL_PINS:
        try:
            fn(orc)
            res[fn.__name__] = None
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            res[fn.__name__] = "%s: %s" % (type(exc).__name__, exc)
    return res
