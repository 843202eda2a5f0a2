"""The kernels' bounded LDS counter waits: when one gives up (a broken
invariant; forced here by a bound of zero polls, which the library takes
from MHCPB_WAIT_POLLS when a plan is created), every result the workgroup
writes from then on is NaN, so that no caller can take stale operands for a
result.  With the bound at zero the projection's producer wave gives up at
its first step and the forward's waves at their first unit, so every dX, dW,
logit and r is NaN; a plan made without the override then gives the normal
results again.  Every kernel still runs to its end (the give-up changes data,
never addresses)."""
import os

import pytest
import torch

import workloads
from rms_backward_amd.wrapper import Plan
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

ENV = "MHCPB_WAIT_POLLS"


def _plan(T, hidden, polls):
    old = os.environ.get(ENV)
    if polls is None:
        os.environ.pop(ENV, None)
    else:
        os.environ[ENV] = str(polls)
    try:
        return Plan(T, 4, hidden)
    finally:
        if old is None:
            os.environ.pop(ENV, None)
        else:
            os.environ[ENV] = old


@pytest.mark.parametrize("T,hidden,addend", [(300, 64, False), (4096, 5120, True)])
def test_backward_give_up_makes_every_output_nan(T, hidden, addend):
    wl = workloads.custom(T, 4, hidden, seed=7, addend=addend)
    inp = workloads.make(wl, "cuda")
    dx0, dw0, _, _ = gh.run(inp, plan=_plan(T, hidden, None))
    dx0, dw0 = dx0.clone(), dw0.clone()
    assert bool(torch.isfinite(dx0.float()).all()) and bool(torch.isfinite(dw0).all())
    dx, dw, _, _ = gh.run(inp, plan=_plan(T, hidden, 0))
    assert bool(torch.isnan(dx.float()).all()), "a dX value escaped the give-up"
    assert bool(torch.isnan(dw).all()), "a dW value escaped the give-up"
    dx2, dw2, _, _ = gh.run(inp, plan=_plan(T, hidden, None))
    assert torch.equal(dx2.view(torch.int16), dx0.view(torch.int16))
    assert torch.equal(dw2.view(torch.int32), dw0.view(torch.int32))


def test_forward_give_up_makes_every_output_nan():
    wl = workloads.custom(1000, 4, 1030, seed=4)
    inp = workloads.forward_inputs(wl, "cuda")
    proj0, r0, _ = gh.run_forward(inp["x"], inp["w"], plan=_plan(1000, 1030, None))
    proj0, r0 = proj0.clone(), r0.clone()
    proj, r, _ = gh.run_forward(inp["x"], inp["w"], plan=_plan(1000, 1030, 0))
    assert bool(torch.isnan(proj[:, :24]).all()) and bool(torch.isnan(r).all())
    proj2, r2, _ = gh.run_forward(inp["x"], inp["w"], plan=_plan(1000, 1030, None))
    assert torch.equal(proj2.view(torch.int32), proj0.view(torch.int32))
    assert torch.equal(r2.view(torch.int32), r0.view(torch.int32))
