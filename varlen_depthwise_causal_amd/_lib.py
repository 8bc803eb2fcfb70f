"""ctypes loader for libvdc.so (the C ABI declared in include/vdc.h)."""
from __future__ import annotations

import ctypes
import os
import threading

from ._build import LIBRARY

VDC_F32, VDC_BF16 = 0, 1
VDC_SILU_GRAD_BF16, VDC_SILU_GRAD_FP32 = 0, 1
VDC_FWD, VDC_BWD = 0, 1
(VDC_OK, VDC_EINVAL, VDC_EDTYPE, VDC_EALIGN, VDC_EWORKSPACE, VDC_ENOBIAS, VDC_EHIP,
 VDC_ESCRATCH) = range(8)
STATUS = {VDC_OK: "VDC_OK", VDC_EINVAL: "VDC_EINVAL", VDC_EDTYPE: "VDC_EDTYPE",
          VDC_EALIGN: "VDC_EALIGN", VDC_EWORKSPACE: "VDC_EWORKSPACE",
          VDC_ENOBIAS: "VDC_ENOBIAS", VDC_EHIP: "VDC_EHIP", VDC_ESCRATCH: "VDC_ESCRATCH"}

_lock = threading.Lock()
_lib = None


class VdcError(RuntimeError):
    """A non-zero vdc_status from the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, STATUS.get(status, status),
                                          load().conv1d_status_string(status).decode()))


def load(path: str | None = None):
    """Load libvdc.so; raises if it has not been built (no fallback exists)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        lib_path = path or LIBRARY
        if not os.path.exists(lib_path):
            raise ImportError(
                "libvdc.so is not built (%s); run varlen_depthwise_causal_amd._build.build() "
                "or __graft_entry__.build()" % lib_path)
        lib = ctypes.CDLL(lib_path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.workspace_bytes.argtypes = [i32, i64, i64]
        lib.workspace_bytes.restype = ctypes.c_size_t
        lib.conv1d_fwd.argtypes = [vp, vp, i32, vp, i32, vp, i64, i64, i64, vp, vp,
                                   ctypes.c_size_t, vp]
        lib.conv1d_fwd.restype = i32
        lib.conv1d_bwd.argtypes = [vp, vp, i32, vp, i32, vp, i64, vp, i64, i64, i32,
                                   vp, vp, i32, vp, i32, vp, ctypes.c_size_t, vp]
        lib.conv1d_bwd.restype = i32
        lib.conv1d_bwd_noalloc.argtypes = [vp, vp, i32, vp, i32, vp, i64, vp, i64, i64, i32,
                                           vp, vp, i32, vp, i32, vp]
        lib.conv1d_bwd_noalloc.restype = i32
        lib.conv1d_noalloc_scratch_bytes.argtypes = []
        lib.conv1d_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.conv1d_status_string.argtypes = [i32]
        lib.conv1d_status_string.restype = ctypes.c_char_p
        lib.conv1d_plan.argtypes = [i32, i64, i64, i32, ctypes.POINTER(i64)]
        lib.conv1d_plan.restype = i32
        lib.conv1d_launch_count.argtypes = []
        lib.conv1d_launch_count.restype = ctypes.c_uint64
        if path is None:
            _lib = lib
        return lib
