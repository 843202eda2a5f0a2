"""The stage inside a HIP graph ("DSv4.1 mHC projection/RMS backward",
"Prepared class API": prepared execution supports graph capture, the buffers
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
