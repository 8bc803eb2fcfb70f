"""Placement invariance: the kernels' choices that depend on where a tensor
sits in memory (the forward's streaming stores of the cache lines a wave
writes alone, on rows that are not a multiple of 128 bytes) must not change
a single bit.  x, dy, y and dx are placed at 16-byte offsets of larger
buffers (every offset modulo 128 that the C ABI allows is reached across the
cases) and the outputs are compared bitwise with those of freshly allocated
tensors."""
import numpy as np
import pytest

import gpu_cases as G

pytestmark = pytest.mark.gpu

# (label, seed, S, C, lengths): rows of 1040, 2000, 8208 and 16 bytes.
CASES = [
    ("c520_dense", 41, 3001, 520, "randint"),
    ("c1000_dense", 42, 2000, 1000, "randint"),
    ("c4104_two_docs", 43, 1500, 4104, [700, 800]),
    ("c8_ragged", 44, 777, 8, [0, 3, 1, 0, 40, 2, 300, 431, 0]),
]
# byte offsets of x, dy, y, dx in their buffers (multiples of 16)
OFFSETS = [(16, 48, 80, 112), (112, 96, 16, 64), (32, 0, 48, 96)]


@pytest.fixture(scope="module")
def torch_cuda():
    torch = G.torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _placed(torch, src, offset):
    """A contiguous copy of src at `offset` bytes into a larger buffer."""
    n = src.numel()
    buf = torch.zeros(n + 64, dtype=src.dtype, device=src.device)
    view = buf[offset // 2: offset // 2 + n].view(src.shape)
    view.copy_(src)
    assert view.data_ptr() % 128 == (buf.data_ptr() + offset) % 128
    return buf, view


def _bits(t):
    torch = G.torch_mod()
    return t.detach().to("cpu").contiguous().view(torch.int16 if t.element_size() == 2
                                                  else torch.int32).numpy()


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_outputs_do_not_depend_on_placement(torch_cuda, case, policy):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    label, seed, S, C, lengths = case
    G.say("CASE placement", label, policy)
    wl = G.small_case(seed, S, C, lengths, "f32", "f32", None)
    dev = G.to_device(wl)
    y0 = vdc.conv1d_fwd(dev["x"], dev["w"], dev["cu"], bias=dev["b"])
    dx0, dw0, db0 = vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"], bias=dev["b"],
                                   silu_grad_preactivation=policy)
    torch.cuda.synchronize()
    ref = [_bits(t) for t in (y0, dx0, dw0, db0)]
    for ox, ody, oy, odx in OFFSETS:
        keep = []
        bx, x = _placed(torch, dev["x"], ox)
        bdy, dy = _placed(torch, dev["dy"], ody)
        by, y = _placed(torch, torch.full_like(dev["x"], 7.0), oy)
        bdx, dx = _placed(torch, torch.full_like(dev["x"], 7.0), odx)
        keep += [bx, bdy, by, bdx]
        vdc.conv1d_fwd(x, dev["w"], dev["cu"], bias=dev["b"], out=y)
        _, dw, db = vdc.conv1d_bwd(x, dev["w"], dev["cu"], dy, bias=dev["b"],
                                   silu_grad_preactivation=policy, dx=dx)
        torch.cuda.synchronize()
        got = [_bits(t) for t in (y, dx, dw, db)]
        for name, a, b in zip(("y", "dx", "dweight", "dbias"), ref, got):
            assert np.array_equal(a, b), "%s: %s differs at offsets %s" % (
                label, name, (ox, ody, oy, odx))
        del keep
