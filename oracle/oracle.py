"""ctypes front end of the FP64 CPU oracle in ``vdc_oracle.c``.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg call it; the HIP library never does.

The oracle follows the documentation pages of
``flashinfer.cake_causal_conv1d_train``:

* ``cake_causal_conv1d_train_forward`` (Parameters, Returns) for the forward,
* ``cake_causal_conv1d_train_backward`` (Description, Parameters, Returns)
  for the backward.

Arrays are numpy.  BF16 data travels as ``uint16`` bit patterns; FP32 as
``float32``.  Everything the oracle computes is IEEE double.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

POLICY_BF16 = 0
POLICY_FP32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "vdc_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lock = threading.Lock()
_default = None


class OracleError(RuntimeError):
    pass


def compile_library(src: str, out: str) -> str:
    """gcc -O2, no fast-math, no FMA contraction: plain IEEE double code."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile ``vdc_oracle.c`` into ``liboracle.so`` (always rebuilds)."""
    global _default
    with _lock:
        _default = None
        return compile_library(SOURCE, LIBRARY)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.orc_decode_bf16.argtypes = [vp, vp, i64]
        lib.orc_decode_bf16.restype = None
        lib.orc_decode_f32.argtypes = [vp, vp, i64]
        lib.orc_decode_f32.restype = None
        lib.orc_bf16_rne_array.argtypes = [vp, vp, i64]
        lib.orc_bf16_rne_array.restype = None
        lib.orc_forward.argtypes = [i64, i64, vp, vp, vp, vp, i64, vp, vp, vp]
        lib.orc_forward.restype = ctypes.c_int
        lib.orc_backward.argtypes = [i64, i64, vp, vp, vp, vp, i64, vp,
                                     ctypes.c_int, vp, vp, vp, vp]
        lib.orc_backward.restype = ctypes.c_int
        lib.orc_silu.argtypes = [ctypes.c_double]
        lib.orc_silu.restype = ctypes.c_double
        lib.orc_silu_grad.argtypes = [ctypes.c_double]
        lib.orc_silu_grad.restype = ctypes.c_double
        self.lib = lib
        self.path = path

    # -- scalar and element-wise helpers ---------------------------------
    def decode_bf16(self, bits) -> np.ndarray:
        """BF16 bit patterns (uint16) -> exact float64 values."""
        bits = _c(bits, np.uint16)
        out = np.empty(bits.shape, np.float64)
        self.lib.orc_decode_bf16(_ptr(bits), _ptr(out), bits.size)
        return out

    def decode_f32(self, vals) -> np.ndarray:
        """float32 values -> exact float64 values."""
        vals = _c(vals, np.float32)
        out = np.empty(vals.shape, np.float64)
        self.lib.orc_decode_f32(_ptr(vals), _ptr(out), vals.size)
        return out

    def bf16_rne(self, vals) -> np.ndarray:
        """float64 -> nearest BF16 (ties to even), returned as uint16 bits."""
        vals = _c(vals, np.float64)
        out = np.empty(vals.shape, np.uint16)
        self.lib.orc_bf16_rne_array(_ptr(vals), _ptr(out), vals.size)
        return out

    def silu(self, z: float) -> float:
        return self.lib.orc_silu(float(z))

    def silu_grad(self, z: float) -> float:
        return self.lib.orc_silu_grad(float(z))

    # -- the method ---------------------------------------------------------
    @staticmethod
    def _prep(x, w, b, cu):
        x = _c(x, np.float64)
        if x.ndim != 2:
            raise OracleError("x must be [S, C]")
        S, C = x.shape
        w = _c(w, np.float64).reshape(C, 4)
        if b is not None:
            b = _c(b, np.float64).reshape(C)
        cu = _c(cu, np.int32).reshape(-1)
        return x, w, b, cu, S, C

    def forward(self, x, w, b, cu, *, want=("p", "pabs", "y")):
        """FP64 forward on decoded inputs.

        x: float64 [S, C]; w: float64 [C, 4]; b: float64 [C] or None;
        cu: int32 [D+1].  Returns a dict with the requested arrays among
        ``p`` (preactivation), ``pabs`` (sum of |terms|) and ``y``
        (unrounded SiLU(p)), each float64 [S, C].
        """
        x, w, b, cu, S, C = self._prep(x, w, b, cu)
        out = {k: np.empty((S, C), np.float64) for k in want}
        rc = self.lib.orc_forward(S, C, _ptr(x), _ptr(w), _ptr(b), _ptr(cu),
                                  cu.size - 1, _ptr(out.get("p")),
                                  _ptr(out.get("pabs")), _ptr(out.get("y")))
        if rc:
            raise OracleError("orc_forward failed with status %d" % rc)
        return out

    def backward(self, x, w, b, cu, dy, policy, *, want=("dpre", "dx", "dw", "db")):
        """FP64 backward on decoded inputs.

        policy: POLICY_BF16 / POLICY_FP32 or "bf16" / "fp32".  Returns a dict
        with the requested arrays among ``dpre`` and ``dx`` (float64 [S, C],
        dx unrounded), ``dw`` (float64 [C, 4]) and ``db`` (float64 [C]).
        """
        if isinstance(policy, str):
            policy = {"bf16": POLICY_BF16, "fp32": POLICY_FP32}[policy]
        x, w, b, cu, S, C = self._prep(x, w, b, cu)
        dy = _c(dy, np.float64).reshape(S, C)
        shapes = {"dpre": (S, C), "dx": (S, C), "dw": (C, 4), "db": (C,)}
        out = {k: np.empty(shapes[k], np.float64) for k in want}
        rc = self.lib.orc_backward(S, C, _ptr(x), _ptr(w), _ptr(b), _ptr(cu),
                                   cu.size - 1, _ptr(dy), int(policy),
                                   _ptr(out.get("dpre")), _ptr(out.get("dx")),
                                   _ptr(out.get("dw")), _ptr(out.get("db")))
        if rc:
            raise OracleError("orc_backward failed with status %d" % rc)
        return out


def default() -> Oracle:
    """The oracle built from ``vdc_oracle.c`` (compiled on first use if absent)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIBRARY):
                compile_library(SOURCE, LIBRARY)
            _default = Oracle(LIBRARY)
        return _default


def decode_bf16(bits):
    return default().decode_bf16(bits)


def decode_f32(vals):
    return default().decode_f32(vals)


def bf16_rne(vals):
    return default().bf16_rne(vals)


def silu(z):
    return default().silu(z)


def silu_grad(z):
    return default().silu_grad(z)


def forward(x, w, b, cu, **kw):
    return default().forward(x, w, b, cu, **kw)


def backward(x, w, b, cu, dy, policy, **kw):
    return default().backward(x, w, b, cu, dy, policy, **kw)


def decode_param(arr, dtype: str):
    """Weight / bias array in its storage dtype ("f32" or "bf16" bits) -> float64."""
    if arr is None:
        return None
    return decode_bf16(arr) if dtype == "bf16" else decode_f32(arr)
