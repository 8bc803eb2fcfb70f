"""Capture of a whole training step (forward, backward main + reduce) in a
HIP graph through torch.cuda.CUDAGraph: every replay, with new inputs copied
into the captured buffers and eager work between replays, gives the bits of
the eager calls.  Covers a caller-owned workspace, the default workspace
(allocated inside the capture from the graph's pool) and S == 0, whose
zero gradients come from a kernel, not a memset node, under capture."""
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


def _inputs(seeds):
    return [G.to_device(G.small_case(s, 4001, 264, "randint", "f32", "f32", (0.01, 60.0)))
            for s in seeds]


@pytest.mark.parametrize("policy", ["bf16", "fp32"])
@pytest.mark.parametrize("own_workspace", [True, False], ids=["caller_ws", "default_ws"])
def test_graph_replays_match_eager(torch_cuda, policy, own_workspace):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE graph", policy, "caller workspace" if own_workspace else "default workspace")
    sets = _inputs([31, 32, 33, 34])
    static = {k: v.clone() for k, v in sets[0].items()}
    S, C = static["x"].shape
    y = torch.empty_like(static["x"])
    dx = torch.empty_like(static["x"])
    dw = torch.empty((C, 4), device="cuda")
    db = torch.empty((C,), device="cuda")
    ws = (torch.empty(vdc.workspace_bytes("bwd", S, C), dtype=torch.uint8, device="cuda")
          if own_workspace else None)

    def step():
        vdc.conv1d_fwd(static["x"], static["w"], static["cu"], bias=static["b"], out=y)
        vdc.conv1d_bwd(static["x"], static["w"], static["cu"], static["dy"], bias=static["b"],
                       silu_grad_preactivation=policy, workspace=ws, dx=dx, dweight=dw, dbias=db)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep, inp in enumerate(sets + sets[:1]):
        for k in static:
            static[k].copy_(inp[k])
        for t in (y, dx, dw, db):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (y, dx, dw, db)]
        # eager work between replays, into separate buffers
        y_e = vdc.conv1d_fwd(inp["x"], inp["w"], inp["cu"], bias=inp["b"])
        dx_e, dw_e, db_e = vdc.conv1d_bwd(inp["x"], inp["w"], inp["cu"], inp["dy"], bias=inp["b"],
                                          silu_grad_preactivation=policy,
                                          dweight=torch.empty((C, 4), device="cuda"),
                                          dbias=torch.empty((C,), device="cuda"))
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "dx", "dw", "db"), got, (y_e, dx_e, dw_e, db_e)):
            assert torch.equal(a, b), "replay %d: %s differs from eager" % (rep, name)


def test_graph_zero_tokens(torch_cuda):
    torch = torch_cuda
    import varlen_depthwise_causal_amd as vdc
    G.say("CASE graph S=0")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((64, 4), device="cuda")
    b = torch.randn((64,), device="cuda")
    cu = torch.zeros((3,), dtype=torch.int32, device="cuda")
    dw = torch.empty((64, 4), device="cuda")
    db = torch.empty((64,), device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    n0 = vdc.conv1d_launch_count()
    with torch.cuda.graph(graph):
        vdc.conv1d_fwd(x, w, cu, bias=b)
        vdc.conv1d_bwd(x, w, cu, x, bias=b, dweight=dw, dbias=db)
    assert vdc.conv1d_launch_count() == n0 + 1  # the zero-fill reduce, no memset node
    for _ in range(3):
        dw.fill_(7.0)
        db.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.all(dw == 0) and torch.all(db == 0)
