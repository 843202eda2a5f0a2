"""The entry point for callers that cannot allocate (mhcpb_execute_noalloc):
its static per-GPU workspace gives the same dX and dW bits as mhcpb_execute
with a caller workspace, on two calls in a row (the second smaller, so stale
contents of the shared workspace would show), and plans whose workspace
exceeds the static one are rejected before any launch."""
import pytest
import torch

import workloads
from rms_backward_amd import (MHCPB_ERROR_WORKSPACE, mhcpb_execute_noalloc,
                              mhcpb_plan_create, mhcpb_plan_destroy, mhcpb_workspace_bytes)
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

STATIC_BYTES = 64 << 20


def _noalloc(plan, inp, dx, dw):
    stream = torch.cuda.current_stream().cuda_stream
    mhcpb_execute_noalloc(plan.handle, inp["x"], inp["w"], inp["grad_proj"], inp["grad_r"],
                          inp["r"], dx, dw, inp.get("addend"), stream)
    torch.cuda.synchronize()


@pytest.mark.parametrize("first,second", [
    ((4096, 5120, False), (1100, 96, True)),
    ((16384, 5120, True), (300, 50, False)),
])
def test_noalloc_matches_execute_on_two_calls(first, second):
    for T, hidden, addend in (first, second):
        print(f"T={T} hidden={hidden} addend={addend}", flush=True)
        wl = workloads.custom(T, 4, hidden, seed=T + hidden, addend=addend, rescale_rows=True)
        inp = workloads.make(wl, "cuda")
        dx0, dw0, _, plan = gh.run(inp)
        dx0, dw0 = dx0.clone(), dw0.clone()
        assert plan.workspace_bytes <= STATIC_BYTES
        dx = torch.full_like(dx0, float("nan"))
        dw = torch.full_like(dw0, float("nan"))
        _noalloc(plan, inp, dx, dw)
        assert torch.equal(dx.view(torch.int16), dx0.view(torch.int16))
        assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32))


def test_noalloc_rejects_workspace_beyond_static():
    # T = 16385 at K = 20480 needs 33 slabs... the split count caps at 32, so
    # a wider row is what exceeds the static workspace: 32 x 24 x K x 4 bytes.
    hidden = 6144  # K = 24576: 32 x 24 x 24576 x 4 = 75,497,472 bytes
    T = 32 * 512
    plan = mhcpb_plan_create(T, 4, hidden)
    try:
        assert mhcpb_workspace_bytes(plan) > STATIC_BYTES
        st = mhcpb_execute_noalloc(plan, 16, 16, 16, 16, 16, 32, 48, None, 0, check=False)
        assert st == MHCPB_ERROR_WORKSPACE
    finally:
        mhcpb_plan_destroy(plan)
