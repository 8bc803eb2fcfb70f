"""The no-allocation backward entry point, conv1d_bwd_noalloc (for callers
that cannot allocate device memory), called through the C ABI and compared
with conv1d_bwd given its own workspace.

Both run the same kernels and launch plan, so dx, dweight and dbias must be
bitwise equal.  Two calls run in a row on one stream, the second with a
smaller input, so the second reads the library's array after the first left
its larger contents there; the conv1d_bwd side gets a workspace filled with
garbage.  The second (small) case is also held to the oracle.
"""
import numpy as np
import pytest

import gpu_cases as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _both(torch, dev, policy, C, grad_dtype):
    import varlen_depthwise_causal_amd as vdc
    d = dev["x"].device
    gdt = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    outs = []
    for noalloc in (True, False):
        dx = torch.full_like(dev["x"], float("nan"))
        dw = torch.full((C, 4), float("nan"), dtype=gdt, device=d)
        db = torch.full((C,), float("nan"), dtype=gdt, device=d) if dev["b"] is not None else None
        if noalloc:
            vdc.conv1d_bwd_noalloc(dev["x"], dev["w"], dev["cu"], dev["dy"], bias=dev["b"],
                                   silu_grad_preactivation=policy, dx=dx, dweight=dw, dbias=db)
        else:
            S = dev["x"].shape[0]
            ws = torch.randint(0, 256, (vdc.workspace_bytes("bwd", S, C),), dtype=torch.uint8,
                               device=d)
            vdc.conv1d_bwd(dev["x"], dev["w"], dev["cu"], dev["dy"], bias=dev["b"],
                           silu_grad_preactivation=policy, workspace=ws, dx=dx, dweight=dw,
                           dbias=db)
        outs.append((dx, dw, db))
    torch.cuda.synchronize()
    return outs


def _bits(t):
    return None if t is None else t.detach().cpu().contiguous().view(-1).view(
        {2: __import__("torch").int16, 4: __import__("torch").int32}[t.element_size()]).numpy()


# (label, seed, S, C, lengths, w_dtype, b_dtype, sat): a large call, then a
# smaller one of another width.
PAIRS = [
    (("stress_like", 31, 60000, 520, "randint", "f32", "f32", (0.01, 60.0)),
     ("small_c264", 32, 3001, 264, [0, 1, 2, 1000, 0, 1998], "f32", "f32", None)),
    (("headline_width", 33, 20000, 4096, [5000, 0, 15000], "f32", "f32", None),
     ("small_c64_nobias", 34, 999, 64, [500, 499], "bf16", None, None)),
]


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
@pytest.mark.parametrize("pair", PAIRS, ids=[p[0][0] + "_then_" + p[1][0] for p in PAIRS])
def test_noalloc_matches_conv1d_bwd(torch_cuda, pair, policy):
    torch = torch_cuda
    for k, case in enumerate(pair):
        label, seed, S, C = case[:4]
        G.say("CASE noalloc", label, "S=%d C=%d" % (S, C), policy, "call", k + 1)
        wl = G.small_case(*case[1:])
        dev = G.to_device(wl)
        (dx0, dw0, db0), (dx1, dw1, db1) = _both(torch, dev, policy, C, "f32")
        assert np.array_equal(_bits(dx0), _bits(dx1)), "%s: dx differs" % label
        assert np.array_equal(_bits(dw0), _bits(dw1)), "%s: dweight differs" % label
        if db0 is not None:
            assert np.array_equal(_bits(db0), _bits(db1)), "%s: dbias differs" % label
        if k == 1:
            y = __import__("varlen_depthwise_causal_amd").conv1d_fwd(dev["x"], dev["w"], dev["cu"],
                                                                    bias=dev["b"])
            torch.cuda.synchronize()
            G.compare(wl, policy, y, dx0, dw0, db0, label="noalloc " + label)


def test_noalloc_bf16_gradients_and_zero_tokens(torch_cuda):
    """BF16 gradient outputs, then S = 0 (zero gradients, no main kernel)."""
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE noalloc bf16 gradients")
    wl = G.small_case(35, 4000, 136, "randint", "bf16", "bf16", None)
    dev = G.to_device(wl)
    (dx0, dw0, db0), (dx1, dw1, db1) = _both(torch, dev, "fp32", 136, "bf16")
    assert np.array_equal(_bits(dx0), _bits(dx1))
    assert np.array_equal(_bits(dw0), _bits(dw1))
    assert np.array_equal(_bits(db0), _bits(db1))
    G.say("CASE noalloc S=0")
    d = dev["x"].device
    x0 = torch.empty((0, 136), dtype=torch.bfloat16, device=d)
    cu0 = torch.zeros((1,), dtype=torch.int32, device=d)
    dw = torch.full((136, 4), 7.0, dtype=torch.float32, device=d)
    db = torch.full((136,), 7.0, dtype=torch.float32, device=d)
    n0 = vdc.conv1d_launch_count()
    vdc.conv1d_bwd_noalloc(x0, dev["w"], cu0, x0, bias=dev["b"], dx=torch.empty_like(x0),
                           dweight=dw, dbias=db)
    torch.cuda.synchronize()
    assert vdc.conv1d_launch_count() == n0
    assert not dw.any() and not db.any()


def test_noalloc_refuses_oversized_problem(torch_cuda):
    """A problem whose workspace exceeds the array is refused before any
    launch, with its outputs untouched."""
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    S, C = 1 << 24, 8          # 69906 partial rows of 8 channels: 22 MB of workspace
    assert vdc.workspace_bytes("bwd", S, C) > vdc.noalloc_scratch_bytes()
    d = torch.device("cuda:0")
    x = torch.zeros((S, C), dtype=torch.bfloat16, device=d)
    w = torch.zeros((C, 4), dtype=torch.float32, device=d)
    cu = torch.tensor([0, S], dtype=torch.int32, device=d)
    dx = torch.full_like(x, 3.0)
    dw = torch.full((C, 4), 3.0, dtype=torch.float32, device=d)
    n0 = vdc.conv1d_launch_count()
    with pytest.raises(vdc.VdcError) as e:
        vdc.conv1d_bwd_noalloc(x, w, cu, x.clone(), dx=dx, dweight=dw)
    assert "VDC_ESCRATCH" in str(e.value)
    torch.cuda.synchronize()
    assert vdc.conv1d_launch_count() == n0
    assert bool((dw == 3.0).all()) and bool((dx == 3.0).all())


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
def test_noalloc_graph_replays_match_eager(torch_cuda, policy):
    """The callers it is for: conv1d_bwd_noalloc captured into a HIP graph
    (torch.cuda.CUDAGraph; nothing allocated during capture), replayed on new
    inputs copied into the captured buffers, with eager calls of both entry
    points between replays: every replay gives conv1d_bwd's bits."""
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE noalloc graph", policy)
    sets = [G.to_device(G.small_case(s, 6001, 520, "randint", "f32", "f32", (0.01, 60.0)))
            for s in (41, 42, 43)]
    static = {k: v.clone() for k, v in sets[0].items()}
    S, C = static["x"].shape
    dx = torch.empty_like(static["x"])
    dw = torch.empty((C, 4), device="cuda")
    db = torch.empty((C,), device="cuda")

    def step():
        vdc.conv1d_bwd_noalloc(static["x"], static["w"], static["cu"], static["dy"],
                               bias=static["b"], silu_grad_preactivation=policy, dx=dx,
                               dweight=dw, dbias=db)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # first call on the device outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep, inp in enumerate(sets + sets[:1]):
        for k in static:
            static[k].copy_(inp[k])
        for t in (dx, dw, db):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (dx, dw, db)]
        ref = vdc.conv1d_bwd(inp["x"], inp["w"], inp["cu"], inp["dy"], bias=inp["b"],
                             silu_grad_preactivation=policy,
                             dweight=torch.empty((C, 4), device="cuda"),
                             dbias=torch.empty((C,), device="cuda"))
        # an eager no-allocation call between replays reuses the array
        vdc.conv1d_bwd_noalloc(inp["x"], inp["w"], inp["cu"], inp["dy"], bias=inp["b"],
                               silu_grad_preactivation=policy, dx=torch.empty_like(dx),
                               dweight=torch.empty_like(dw), dbias=torch.empty_like(db))
        torch.cuda.synchronize()
        for name, a, b in zip(("dx", "dw", "db"), got, ref):
            assert torch.equal(a, b), "replay %d: %s differs from conv1d_bwd" % (rep, name)
