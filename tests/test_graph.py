"""The stage, the forward and the RMSNorm backward inside a HIP graph
("DSv4.1 mHC projection/RMS backward", "Prepared class API": prepared
execution supports graph capture, the buffers
staying alive for every replay).  mhcpb_execute only launches kernels (no
allocation, no memset, no synchronisation), so it can be captured; every
replay must give the eager result bit for bit, with eager work (refilling the
outputs with NaN) and synchronisations between the replays."""
import pytest
import torch

import workloads
from rms_backward_amd import mhcpb_execute
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("addend", [False, True])
def test_graph_replays_match_eager(addend):
    wl = workloads.custom(2049, 4, 1280, seed=9, addend=addend)
    inp = workloads.make(wl, "cuda")
    dx0, dw0, _, plan = gh.run(inp)
    dx0, dw0 = dx0.clone(), dw0.clone()
    dx, dw, ws = gh.alloc_outputs(wl.T, wl.K, plan, "cuda")
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        mhcpb_execute(plan.handle, inp["x"], inp["w"], inp["grad_proj"], inp["grad_r"], inp["r"],
                      dx, dw, inp.get("addend"), ws, ws.numel(), side.cuda_stream)
    for replay in range(4):
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32)), f"replay {replay}"
        assert torch.equal(dx.view(torch.int16), dx0.view(torch.int16)), f"replay {replay}"
    del graph


def test_forward_graph_replays_match_eager():
    """The forward entry point captured the same way."""
    from rms_backward_amd import mhcpb_forward
    wl = workloads.custom(1000, 4, 1030, seed=4)
    inp = workloads.forward_inputs(wl, "cuda")
    proj0, r0, plan = gh.run_forward(inp["x"], inp["w"])
    proj0, r0 = proj0.clone(), r0.clone()
    proj = torch.empty_like(proj0)
    r = torch.empty_like(r0)
    ws = plan.alloc_forward_workspace("cuda")
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        mhcpb_forward(plan.handle, inp["x"], inp["w"], 1e-6, proj, r, ws, ws.numel(),
                      side.cuda_stream)
    for replay in range(4):
        proj.fill_(float("nan"))
        r.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(proj.view(torch.int32), proj0.view(torch.int32)), f"replay {replay}"
        assert torch.equal(r.view(torch.int32), r0.view(torch.int32)), f"replay {replay}"
    del graph


@pytest.mark.parametrize("residual", [False, True])
def test_rmsnorm_graph_replays_match_eager(residual):
    """The RMSNorm backward captured the same way (both of its kernels)."""
    import rms_backward_amd as m
    wl = workloads.rms_custom(3000, 5120, seed=6, residual=residual)
    inp = workloads.rms_inputs(wl, "cuda")
    dx0, dw0 = gh.run_rmsnorm(inp)
    dx0, dw0 = dx0.clone(), dw0.clone()
    dx = torch.empty_like(dx0)
    dw = torch.empty_like(dw0)
    ws = torch.empty(m.mhcpb_rmsnorm_backward_workspace_bytes(wl.T, wl.H), dtype=torch.uint8,
                     device="cuda")
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        m.mhcpb_rmsnorm_backward(wl.T, wl.H, inp["g"], inp["x"], inp["w"], m.MHCPB_DTYPE_BF16,
                                 inp["rstd"], inp["res"], dx, dw, ws, ws.numel(),
                                 side.cuda_stream)
    for replay in range(4):
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32)), f"replay {replay}"
        assert torch.equal(dx.view(torch.int16), dx0.view(torch.int16)), f"replay {replay}"
    del graph
