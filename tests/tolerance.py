"""Acceptance rules for GPU results against the FP64 oracle.

The bounds come from the documentation of
flashinfer.cake_causal_conv1d_train.cake_causal_conv1d_train_backward
(Parameters, silu_grad_preactivation): dweight within about 3e-5 (rel-L2)
of the exact FP64 gradient under "bf16", about 2e-7 under "fp32", and dx
within one BF16 ulp of exact under both; y is held to the same one-ulp rule.

Readings (each one is also listed in the design notes):

* "exact FP64 gradient" under "bf16" is the FP64 gradient of the same
  policy, i.e. SiLU' evaluated at the BF16 rounding of the FP64
  preactivation (the oracle's "bf16" policy).
* "within one BF16 ulp" is read as |out - v64| <= ulp(v64) + A (see
  check_ulp for the case A is not small against |v64|), where A
  bounds the error any binary32 evaluation of the prescribed formula can
  make before the final rounding (standard forward-error bounds, u = 2^-24):
    dp  = 6 u sum|terms of p|                       preactivation error
    A_y = max|SiLU'| on [p-dp, p+dp] * dp + (1.25|p| + 8) u |y|
    A_g = (1.25|z| + 9) u sigma(z) (1 + |z|)        error of SiLU'(z) itself
    D   = (|SiLU''(p)| + dp) dp   ("fp32"; |SiLU'''| < 1)
        = max |SiLU'(b) - SiLU'(z64)| over the BF16 values b that
          p64 +- dp rounds to ("bf16": the rounded argument may move)
    A_dpre = |dy| (D + A_g) + u |dpre|
    A_dx = sum_k |w_k| A_dpre[t+3-k] + 5 u sum_k |w_k dpre64[t+3-k]|
  Where nothing cancels, A is far below half an ulp and the rule is the
  plain one-ulp rule.  Two things cancel.  The first is the taps of p or of
  dx.  The second, under "fp32", is SiLU' near its zero, z ~ -1.278: there
  s (1 + z (1 - s)) in binary32 has a large relative error, which A_g
  covers.
* rel-L2 = ||g - r||_2 / ||r||_2 over the entries compared, in FP64.  Under
  "bf16" the check is ||g - r|| <= bound ||r|| + ||F||, where F is the most
  the rare BF16 boundary flips of the preactivation (see bf16_flip) can move
  the gradients; at the workloads' sizes ||F|| is far below bound ||r||, on
  tiny problems one flip can exceed the bound on its own.
"""
from __future__ import annotations

import numpy as np

import oracle

U32 = 2.0 ** -24
BOUND = {"bf16": 3e-5, "fp32": 2e-7}


def ulp_bf16(v):
    """Spacing of BF16 numbers at |v|: 2^(floor(log2|v|) - 7), at least 2^-133."""
    a = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(a)                      # a = m 2^e, m in [0.5, 1)
    u = np.ldexp(1.0, e - 8)
    return np.where(a > 0, np.maximum(u, 2.0 ** -133), 2.0 ** -133)


def _sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu_grad64(z):
    s = _sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def silu_grad2_64(z):
    s = _sigmoid(z)
    return s * (1.0 - s) * (2.0 + z * (1.0 - 2.0 * s))


def _critical_point():
    """The positive root of SiLU'' (where SiLU' peaks), by Newton's method on
    z tanh(z/2) = 2."""
    z = 2.4
    for _ in range(50):
        t = np.tanh(z / 2)
        z -= (z * t - 2.0) / (t + z * 0.5 * (1 - t * t))
    return z


Z_CRIT = _critical_point()


def max_abs_silu_grad(lo, hi):
    """max |SiLU'| over [lo, hi]: at an end point or at a critical point inside."""
    m = np.maximum(np.abs(silu_grad64(lo)), np.abs(silu_grad64(hi)))
    for zc in (Z_CRIT, -Z_CRIT):
        m = np.where((lo <= zc) & (hi >= zc), np.maximum(m, abs(silu_grad64(zc))), m)
    return m


def allowance_y(p64, pabs, y64):
    dp = 6.0 * U32 * pabs
    slope = max_abs_silu_grad(p64 - dp, p64 + dp)
    return slope * dp + (1.25 * np.abs(p64) + 8.0) * U32 * np.abs(y64)


def bf16_flip(p64, pabs, dy64):
    """|dy| * max |SiLU'(b) - SiLU'(bf16(p64))| over the BF16 values b that
    p64 +- dp rounds to: the most the "bf16" policy's dpre can move when the
    binary32 preactivation lands on the other side of a BF16 rounding
    boundary.  Zero for nearly every element."""
    dp = 6.0 * U32 * pabs
    z = oracle.decode_bf16(oracle.bf16_rne(p64))
    lo = oracle.decode_bf16(oracle.bf16_rne(p64 - dp))
    hi = oracle.decode_bf16(oracle.bf16_rne(p64 + dp))
    g0 = silu_grad64(z)
    return np.abs(dy64) * np.maximum(np.abs(silu_grad64(lo) - g0), np.abs(silu_grad64(hi) - g0))


def flip_bound_grads(flip, x64, cu):
    """Largest change of dweight [C,4] and dbias [C] the flips can cause:
    sum_t flip[t] |x[t-3+k]| over taps inside t's document, and sum_t flip[t]."""
    S, C = flip.shape
    start = np.empty(S, np.int64)
    for d in range(len(cu) - 1):
        start[cu[d]:cu[d + 1]] = cu[d]
    t = np.arange(S)
    fw = np.zeros((C, 4))
    for k in range(4):
        src = t - 3 + k
        ok = src >= start
        srcc = np.where(ok, src, 0)
        fw[:, k] = np.sum(np.where(ok[:, None], flip * np.abs(x64[srcc]), 0.0), axis=0)
    return fw, flip.sum(axis=0)


def allowance_dpre(p64, pabs, dy64, dpre64, policy):
    dp = 6.0 * U32 * pabs
    if policy == "bf16":
        z = oracle.decode_bf16(oracle.bf16_rne(p64))
        lo = oracle.decode_bf16(oracle.bf16_rne(p64 - dp))
        hi = oracle.decode_bf16(oracle.bf16_rne(p64 + dp))
        g0 = silu_grad64(z)
        move = np.maximum(np.abs(silu_grad64(lo) - g0), np.abs(silu_grad64(hi) - g0))
    else:
        z = p64
        move = (np.abs(silu_grad2_64(p64)) + dp) * dp      # |SiLU'''| < 1
    ag = (1.25 * np.abs(z) + 9.0) * U32 * _sigmoid(z) * (1.0 + np.abs(z))
    return np.abs(dy64) * (move + ag) + U32 * np.abs(dpre64)


def allowance_dx(w64, cu, a_dpre, dpre64):
    """sum over the taps of t's document of |w_k| a_dpre[t+3-k] + 5u |w_k dpre[t+3-k]|."""
    S, C = a_dpre.shape
    end = np.empty(S, np.int64)
    for d in range(len(cu) - 1):
        end[cu[d]:cu[d + 1]] = cu[d + 1]
    out = np.zeros((S, C))
    mag = np.zeros((S, C))
    t = np.arange(S)
    for k in range(4):
        src = t + 3 - k
        ok = src < end
        srcc = np.where(ok, src, 0)
        wa = np.abs(w64[:, k])[None, :]
        out += np.where(ok[:, None], wa * a_dpre[srcc], 0.0)
        mag += np.where(ok[:, None], wa * np.abs(dpre64[srcc]), 0.0)
    return out + 5.0 * U32 * mag


def check_ulp(name, got, v64, allow):
    """Assert |got - v64| <= max(ulp(v64), ulp(|v64| + allow) / 2) + allow.

    got is the BF16 rounding of a binary32 value within `allow` of v64, so
    its own rounding adds at most half an ulp at |v64| + allow; where allow
    is small against |v64| this is the plain one-ulp rule."""
    err = np.abs(np.asarray(got, np.float64) - v64)
    u = np.maximum(ulp_bf16(v64), 0.5 * ulp_bf16(np.abs(v64) + allow))
    bad = err > u + allow
    beyond_plain = int(np.count_nonzero(err > ulp_bf16(v64)))
    rep = {"n": int(err.size), "violations": int(np.count_nonzero(bad)),
           "beyond_1ulp": beyond_plain,
           "max_ulps": float(np.max(err / u)) if err.size else 0.0}
    if bad.any():
        i = np.argmax(np.where(bad, err - u - allow, -np.inf))
        idx = np.unravel_index(i, err.shape)
        raise AssertionError("%s: %d of %d outside ulp + allowance; worst at %s: got %r want %r "
                             "(ulp %g, allowance %g)" % (name, rep["violations"], err.size, idx,
                                                         float(np.asarray(got).flat[i]),
                                                         float(v64.flat[i]), float(u.flat[i]),
                                                         float(np.asarray(allow).flat[i])))
    return rep


def rel_l2(g, r):
    g = np.asarray(g, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    n = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / n) if n > 0 else float(np.linalg.norm(g))
