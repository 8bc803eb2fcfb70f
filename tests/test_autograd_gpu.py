"""The autograd wrapper (documentation page CakeCausalConv1dFunction): the
same bits as the direct calls, gradients in the parameters' dtypes, any
incoming gradient layout, [1, S, C] activations, and oracle parity through
autograd."""
import pytest

import gpu_cases as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _leaf(t, grad=True):
    return None if t is None else t.detach().clone().requires_grad_(grad)


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
def test_autograd_matches_direct_calls(torch_cuda, policy):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    from varlen_depthwise_causal_amd.autograd import causal_conv1d_silu
    G.say("CASE autograd direct", policy)
    wl = G.small_case(21, 3001, 520, "randint", "f32", "f32", (0.01, 60.0))
    dev = G.to_device(wl)
    x, w, b = _leaf(dev["x"]), _leaf(dev["w"]), _leaf(dev["b"])
    y = causal_conv1d_silu(x, w, dev["cu"], b, policy)
    y.backward(dev["dy"])
    y_ref = vdc.conv1d_fwd(dev["x"], dev["w"], dev["cu"], bias=dev["b"])
    dx_ref, dw_ref, db_ref = vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"],
                                            bias=dev["b"], silu_grad_preactivation=policy)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(x.grad, dx_ref) and torch.equal(w.grad, dw_ref) and torch.equal(b.grad, db_ref)
    assert w.grad.dtype == torch.float32 and b.grad.dtype == torch.float32
    G.compare(wl, policy, y.detach(), x.grad, w.grad, b.grad, label="autograd c520")


def test_autograd_bf16_params_and_3d(torch_cuda):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    from varlen_depthwise_causal_amd.autograd import CausalConv1dFunction
    G.say("CASE autograd bf16 params, [1, S, C]")
    wl = G.small_case(22, 1500, 1024, [700, 0, 1, 2, 3, 794], "bf16", "bf16", None)
    dev = G.to_device(wl)
    x3 = _leaf(dev["x"].unsqueeze(0))
    w, b = _leaf(dev["w"]), _leaf(dev["b"])
    y = CausalConv1dFunction.apply(x3, w, dev["cu"], b, "bf16")
    assert y.shape == x3.shape and y.dtype == torch.bfloat16
    y.backward(dev["dy"].unsqueeze(0))
    assert x3.grad.shape == x3.shape
    assert w.grad.dtype == torch.bfloat16 and b.grad.dtype == torch.bfloat16
    dx_ref, dw_ref, db_ref = vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"], bias=dev["b"])
    torch.cuda.synchronize()
    assert torch.equal(x3.grad[0], dx_ref) and torch.equal(w.grad, dw_ref)
    assert torch.equal(b.grad, db_ref)


def test_autograd_materializes_incoming_gradient(torch_cuda):
    """A non-contiguous BF16 gradient and an FP32 one give the bits of the
    contiguous BF16 gradient with the same values."""
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    from varlen_depthwise_causal_amd.autograd import causal_conv1d_silu
    G.say("CASE autograd incoming gradient layouts")
    wl = G.small_case(23, 777, 64, [0, 3, 1, 0, 40, 2, 300, 431, 0], "f32", None, None)
    dev = G.to_device(wl)
    dx_ref, dw_ref = vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"])
    # the same values, laid out column-major: a non-contiguous [S, C] view
    dy_nc = dev["dy"].t().contiguous().t()
    assert not dy_nc.is_contiguous()
    # the FP32 gradient holds BF16 values, so its BF16 rounding is exact
    for label, g in (("non-contiguous bf16", dy_nc), ("fp32", dev["dy"].float())):
        x, w = _leaf(dev["x"]), _leaf(dev["w"])
        y = causal_conv1d_silu(x, w, dev["cu"])
        torch.autograd.backward(y, grad_tensors=g)
        torch.cuda.synchronize()
        assert torch.equal(x.grad, dx_ref), label
        assert torch.equal(w.grad, dw_ref), label


def test_autograd_only_weight_requires_grad(torch_cuda):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    from varlen_depthwise_causal_amd.autograd import causal_conv1d_silu
    G.say("CASE autograd weight only")
    wl = G.small_case(24, 2049, 24, None, "f32", None, None)
    dev = G.to_device(wl)
    w = _leaf(dev["w"])
    y = causal_conv1d_silu(dev["x"], w, dev["cu"], None, "fp32")
    y.backward(dev["dy"])
    _, dw_ref = vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"],
                               silu_grad_preactivation="fp32")
    torch.cuda.synchronize()
    assert torch.equal(w.grad, dw_ref)
