"""Host-side behaviour of the autograd wrapper (no GPU needed): it refuses
host tensors and unknown policies before anything reaches the library."""
import pytest
import torch

from varlen_depthwise_causal_amd.autograd import CausalConv1dFunction, causal_conv1d_silu


def _args():
    x = torch.zeros((16, 8), dtype=torch.bfloat16, requires_grad=True)
    w = torch.zeros((8, 4), requires_grad=True)
    cu = torch.tensor([0, 16], dtype=torch.int32)
    return x, w, cu


def test_refuses_host_tensors():
    x, w, cu = _args()
    with pytest.raises(ValueError, match="device tensor"):
        causal_conv1d_silu(x, w, cu)


def test_refuses_unknown_policy():
    x, w, cu = _args()
    with pytest.raises(ValueError, match="silu_grad_preactivation"):
        CausalConv1dFunction.apply(x, w, cu, None, "fp16")
