"""Packed variable-length width-4 depthwise causal conv1d + SiLU for MI355X.

Python binding of libvdc.so (C ABI in include/vdc.h).  This module only
marshals arguments: every step of the computation runs in the library's HIP
kernels, and PyTorch provides device memory and the current stream.  If the
library is not built, the calls raise; there is no fallback.

The API mirrors the documentation pages of flashinfer.cake_causal_conv1d_train
(cake_causal_conv1d_train_forward / _backward, Parameters and Returns): x and
dy are BF16 [S, C] or [1, S, C]; weight FP32 or BF16 [C, 4]; bias FP32 or BF16
[C]; cu_seqlens int32 [num_docs + 1] on the device.
"""
from __future__ import annotations

import ctypes

from ._lib import (  # noqa: F401
    VDC_BF16,
    VDC_BWD,
    VDC_ENOBIAS,
    VDC_F32,
    VDC_FWD,
    VDC_SILU_GRAD_BF16,
    VDC_SILU_GRAD_FP32,
    VdcError,
    load,
)

__all__ = ["conv1d_fwd", "conv1d_bwd", "conv1d_bwd_noalloc", "workspace_bytes",
           "noalloc_scratch_bytes", "conv1d_plan", "conv1d_launch_count", "VdcError"]

_POLICIES = {"bf16": VDC_SILU_GRAD_BF16, "fp32": VDC_SILU_GRAD_FP32}


def _torch():
    import torch
    return torch


def _dtype_code(t, what):
    torch = _torch()
    if t.dtype == torch.float32:
        return VDC_F32
    if t.dtype == torch.bfloat16:
        return VDC_BF16
    raise TypeError("%s must be float32 or bfloat16, got %s" % (what, t.dtype))


def _check_dev(t, what, device):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % what)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (what, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)


def _activation(x, what):
    torch = _torch()
    if x.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16" % what)
    if x.dim() == 3 and x.shape[0] == 1:
        S, C = int(x.shape[1]), int(x.shape[2])
    elif x.dim() == 2:
        S, C = int(x.shape[0]), int(x.shape[1])
    else:
        raise ValueError("%s must be [S, C] or [1, S, C], got %s" % (what, tuple(x.shape)))
    return S, C


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _params(x, weight, cu_seqlens, bias):
    S, C = _activation(x, "x")
    dev = x.device
    _check_dev(x, "x", dev)
    _check_dev(weight, "weight", dev)
    _check_dev(cu_seqlens, "cu_seqlens", dev)
    if tuple(weight.shape) != (C, 4):
        raise ValueError("weight must be [C, 4] = [%d, 4] (width 4 only), got %s"
                         % (C, tuple(weight.shape)))
    w_code = _dtype_code(weight, "weight")
    torch = _torch()
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a non-empty 1-D int32 tensor")
    b_code = 0
    if bias is not None:
        _check_dev(bias, "bias", dev)
        if tuple(bias.shape) != (C,):
            raise ValueError("bias must be [C]")
        b_code = _dtype_code(bias, "bias")
    return S, C, dev, w_code, b_code


def workspace_bytes(direction: str, S: int, C: int) -> int:
    """Workspace bytes of ``direction`` ("fwd" / "bwd") at (S, C)."""
    d = {"fwd": VDC_FWD, "bwd": VDC_BWD}[direction]
    return int(load().workspace_bytes(d, int(S), int(C)))


def conv1d_plan(direction: str, S: int, C: int, policy: str = "bf16") -> dict:
    """The launch plan the library picks for these sizes (introspection)."""
    d = {"fwd": VDC_FWD, "bwd": VDC_BWD}[direction]
    out = (ctypes.c_int64 * 11)()
    rc = load().conv1d_plan(d, int(S), int(C), _POLICIES[policy], out)
    if rc:
        raise VdcError(rc, "conv1d_plan")
    keys = ("rows", "bands", "lanes", "blocks", "threads", "acc_bytes", "red_blocks", "red_chunks",
            "vec", "red_stage1", "prows")
    return dict(zip(keys, (int(v) for v in out)))


def noalloc_scratch_bytes() -> int:
    """Bytes of the device array conv1d_bwd_noalloc uses as its workspace."""
    return int(load().conv1d_noalloc_scratch_bytes())


def conv1d_launch_count() -> int:
    return int(load().conv1d_launch_count())


def conv1d_fwd(x, weight, cu_seqlens, *, bias=None, out=None, workspace=None):
    """y = bf16(silu(depthwise causal conv(x))) per document; returns y (x's shape)."""
    S, C, dev, w_code, b_code = _params(x, weight, cu_seqlens, bias)
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_dev(out, "out", dev)
        if out.dtype != torch.bfloat16 or out.shape != x.shape:
            raise ValueError("out must be bfloat16 of x's shape")
    ws_ptr, ws_n = None, 0
    if workspace is not None:
        _check_dev(workspace, "workspace", dev)
        ws_ptr, ws_n = _ptr(workspace), workspace.numel() * workspace.element_size()
    rc = load().conv1d_fwd(_ptr(x), _ptr(weight), w_code, _ptr(bias), b_code,
                           _ptr(cu_seqlens), cu_seqlens.numel() - 1, S, C,
                           _ptr(out), ws_ptr, ws_n, _stream(dev))
    if rc:
        raise VdcError(rc, "conv1d_fwd")
    return out


def _bwd_outputs(x, weight, cu_seqlens, dy, bias, silu_grad_preactivation, dx, dweight, dbias,
                 allocate):
    """Checked arguments of a backward call; missing outputs are allocated
    only when `allocate` (otherwise they are required)."""
    S, C, dev, w_code, b_code = _params(x, weight, cu_seqlens, bias)
    torch = _torch()
    if dy.dtype != torch.bfloat16 or dy.shape != x.shape:
        raise ValueError("dy must be bfloat16 of x's shape")
    _check_dev(dy, "dy", dev)
    if silu_grad_preactivation not in _POLICIES:
        raise ValueError("silu_grad_preactivation must be 'bf16' or 'fp32'")
    policy = _POLICIES[silu_grad_preactivation]
    if not allocate and (dx is None or dweight is None or (bias is not None and dbias is None)):
        raise ValueError("conv1d_bwd_noalloc allocates nothing: pass dx, dweight "
                         "(and dbias with a bias)")
    if dx is None:
        dx = torch.empty_like(x)
    else:
        _check_dev(dx, "dx", dev)
        if dx.dtype != torch.bfloat16 or dx.shape != x.shape:
            raise ValueError("dx must be bfloat16 of x's shape")
    if dweight is None:
        dweight = torch.empty((C, 4), dtype=weight.dtype, device=dev)
    else:
        _check_dev(dweight, "dweight", dev)
        if tuple(dweight.shape) != (C, 4):
            raise ValueError("dweight must be [C, 4]")
    dw_code = _dtype_code(dweight, "dweight")
    db_code = 0
    if dbias is not None and bias is None:
        raise VdcError(VDC_ENOBIAS, "conv1d_bwd")
    if bias is not None:
        if dbias is None:
            dbias = torch.empty((C,), dtype=bias.dtype, device=dev)
        else:
            _check_dev(dbias, "dbias", dev)
            if tuple(dbias.shape) != (C,):
                raise ValueError("dbias must be [C]")
        db_code = _dtype_code(dbias, "dbias")
    return S, C, dev, w_code, b_code, policy, dx, dweight, dw_code, dbias, db_code


def conv1d_bwd(x, weight, cu_seqlens, dy, *, bias=None, silu_grad_preactivation="bf16",
               workspace=None, dx=None, dweight=None, dbias=None):
    """Returns (dx, dweight) or (dx, dweight, dbias) when a bias is given.

    dweight / dbias default to the parameters' dtypes; pass preallocated
    float32 buffers to receive FP32 gradients for BF16 parameters.
    """
    torch = _torch()
    (S, C, dev, w_code, b_code, policy, dx, dweight, dw_code, dbias,
     db_code) = _bwd_outputs(x, weight, cu_seqlens, dy, bias, silu_grad_preactivation, dx,
                             dweight, dbias, allocate=True)
    need = workspace_bytes("bwd", S, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _check_dev(workspace, "workspace", dev)
    ws_n = workspace.numel() * workspace.element_size()
    rc = load().conv1d_bwd(_ptr(x), _ptr(weight), w_code, _ptr(bias), b_code,
                           _ptr(cu_seqlens), cu_seqlens.numel() - 1, _ptr(dy), S, C, policy,
                           _ptr(dx), _ptr(dweight), dw_code, _ptr(dbias), db_code,
                           _ptr(workspace), ws_n, _stream(dev))
    if rc:
        raise VdcError(rc, "conv1d_bwd")
    return (dx, dweight) if bias is None else (dx, dweight, dbias)


def conv1d_bwd_noalloc(x, weight, cu_seqlens, dy, *, dx, dweight, bias=None, dbias=None,
                       silu_grad_preactivation="bf16"):
    """conv1d_bwd with the library's own device array as its workspace: no
    allocation anywhere (the outputs are required).  Calls on one GPU share
    the array, so calls that may overlap in time race.  Returns the same
    tuple as conv1d_bwd."""
    (S, C, dev, w_code, b_code, policy, dx, dweight, dw_code, dbias,
     db_code) = _bwd_outputs(x, weight, cu_seqlens, dy, bias, silu_grad_preactivation, dx,
                             dweight, dbias, allocate=False)
    rc = load().conv1d_bwd_noalloc(_ptr(x), _ptr(weight), w_code, _ptr(bias), b_code,
                                   _ptr(cu_seqlens), cu_seqlens.numel() - 1, _ptr(dy), S, C,
                                   policy, _ptr(dx), _ptr(dweight), dw_code, _ptr(dbias),
                                   db_code, _stream(dev))
    if rc:
        raise VdcError(rc, "conv1d_bwd_noalloc")
    return (dx, dweight) if bias is None else (dx, dweight, dbias)
