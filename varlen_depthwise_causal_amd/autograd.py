"""Autograd wrapper of the packed varlen width-4 depthwise causal conv1d +
SiLU (documentation page CakeCausalConv1dFunction, class description).

Only (x, weight, cu_seqlens, bias) are saved: the backward recomputes the
preactivation from x inside the backward kernel, so no activation other than
the inputs is kept alive between the passes.  The kernels read the output
gradient as dense row-major BF16, so a gradient of any other dtype or
strides is converted (a copy) before the call.  The weight and bias
gradients are returned in the dtypes of the parameters they belong to.
Every step runs in libvdc.so's kernels through conv1d_fwd / conv1d_bwd.
"""
from __future__ import annotations

import torch

from . import conv1d_bwd, conv1d_fwd

__all__ = ["CausalConv1dFunction", "causal_conv1d_silu"]


class CausalConv1dFunction(torch.autograd.Function):
    """y = bf16(silu(depthwise causal conv(x) + bias)) per document, with the
    backward of conv1d_bwd under the chosen SiLU' policy."""

    @staticmethod
    def forward(ctx, x, weight, cu_seqlens, bias=None, silu_grad_preactivation="bf16"):
        if silu_grad_preactivation not in ("bf16", "fp32"):
            raise ValueError("silu_grad_preactivation must be 'bf16' or 'fp32'")
        y = conv1d_fwd(x, weight, cu_seqlens, bias=bias)
        ctx.save_for_backward(x, weight, cu_seqlens, bias)
        ctx.policy = silu_grad_preactivation
        return y

    @staticmethod
    def backward(ctx, grad_y):
        x, weight, cu_seqlens, bias = ctx.saved_tensors
        dy = grad_y
        if dy.dtype != torch.bfloat16 or not dy.is_contiguous():
            dy = dy.to(torch.bfloat16).contiguous()
        grads = conv1d_bwd(x, weight, cu_seqlens, dy, bias=bias,
                           silu_grad_preactivation=ctx.policy)
        dx, dweight = grads[0], grads[1]
        dbias = grads[2] if bias is not None else None
        need = ctx.needs_input_grad
        return (dx if need[0] else None, dweight if need[1] else None, None,
                dbias if (bias is not None and need[3]) else None, None)


def causal_conv1d_silu(x, weight, cu_seqlens, bias=None, silu_grad_preactivation="bf16"):
    """Differentiable forward: returns y (x's shape, BF16)."""
    return CausalConv1dFunction.apply(x, weight, cu_seqlens, bias, silu_grad_preactivation)
