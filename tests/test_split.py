"""The split backward ("FP8 weight cache, split backward, fused mHC stream
gradient" on the prime-kernels page: the data gradient first, the weight
gradients after).  mhcpb_execute_dx and mhcpb_execute_dw each run the same
arithmetic as the fused mhcpb_execute for their output, so dX and dW must be
the fused call's bits exactly (and hence within the oracle bounds the fused
call is tested to); outputs a form does not produce are left untouched."""
import pytest
import torch

import workloads
from rms_backward_amd import mhcpb_execute_dw, mhcpb_execute_dx
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

SHAPES = [
    # T, hidden, addend
    (1, 2, False),
    (17, 66, True),
    (513, 130, False),
    (2049, 34, True),
    (4096, 5120, False),
    (4095, 5120, True),
    (16384, 5120, False),
]


@pytest.mark.parametrize("T,hidden,addend", SHAPES)
def test_split_forms_give_the_fused_bits(T, hidden, addend):
    wl = workloads.custom(T, 4, hidden, seed=T + 3 * hidden, addend=addend, rescale_rows=True)
    print(f"T={T} hidden={hidden} addend={addend}", flush=True)
    inp = workloads.make(wl, "cuda")
    dx0, dw0, _, plan = gh.run(inp)
    dx0, dw0 = dx0.clone(), dw0.clone()
    dx, dw, ws = gh.alloc_outputs(wl.T, wl.K, plan, "cuda")
    dx_sentinel = dx.clone()
    stream = torch.cuda.current_stream().cuda_stream
    mhcpb_execute_dw(plan.handle, inp["x"], inp["grad_proj"], dw, ws, ws.numel(), stream)
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32))
    assert torch.equal(dx.view(torch.int16), dx_sentinel.view(torch.int16)), "dX touched"
    dw_sentinel = dw.clone().fill_(float("nan"))
    dw.copy_(dw_sentinel)
    mhcpb_execute_dx(plan.handle, inp["x"], inp["w"], inp["grad_proj"], inp["grad_r"], inp["r"],
                     dx, inp.get("addend"), stream)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx0.view(torch.int16))
    assert torch.equal(dw.view(torch.int32), dw_sentinel.view(torch.int32)), "dW touched"
