"""The split backward ("FP8 weight cache, split backward, fused mHC stream
gradient" on the prime-kernels page: the data gradient first, the weight
gradients after).  mhcpb_execute_dx writes dX alone and mhcpb_execute_dw dW
alone; each is compared with the FP64 oracle under the stage's bounds (every
element at the small shapes, sampled rows of dX and columns of dW at the
full-size ones), outputs a form does not produce are left untouched, and each
output carries the fused call's bits (the same arithmetic runs in both)."""
import numpy as np
import pytest
import torch

import workloads
from rms_backward_amd import mhcpb_execute_dw, mhcpb_execute_dx, mhcpb_plan_split_count
from tests import gpu_harness as gh
from tests.oracle_checks import check_dw, check_dx

pytestmark = pytest.mark.gpu

SMALL = [
    # T, hidden, addend: every element against the oracle
    (1, 2, False),
    (17, 66, True),
    (513, 130, False),
    (2049, 34, True),
    (520, 5120, True),   # five-wave workgroups, slab group 0 adding its partials up
]
FULL = [
    # sampled rows and columns against the oracle
    (4096, 5120, False),
    (4095, 5120, True),
    (16384, 5120, False),
]


def _run_split(inp, plan):
    """dW-only then dX-only calls into fresh NaN-filled outputs; returns
    (dx, dw) and checks that neither call touched the other's output."""
    T, K = inp["x"].shape
    dx, dw, ws = gh.alloc_outputs(T, K, plan, "cuda")
    dx_sentinel = dx.clone()
    stream = torch.cuda.current_stream().cuda_stream
    mhcpb_execute_dw(plan.handle, inp["x"], inp["grad_proj"], dw, ws, ws.numel(), stream)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx_sentinel.view(torch.int16)), "dX touched"
    dw_done = dw.clone()
    dw.fill_(float("nan"))
    dw_sentinel = dw.clone()
    mhcpb_execute_dx(plan.handle, inp["x"], inp["w"], inp["grad_proj"], inp["grad_r"], inp["r"],
                     dx, inp.get("addend"), stream)
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dw_sentinel.view(torch.int32)), "dW touched"
    return dx, dw_done


def _fused_bits(inp, plan, dx, dw):
    dx0, dw0, _, _ = gh.run(inp, plan=plan)
    assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32))
    assert torch.equal(dx.view(torch.int16), dx0.view(torch.int16))


@pytest.mark.parametrize("T,hidden,addend", SMALL)
def test_split_forms_every_element(T, hidden, addend):
    wl = workloads.custom(T, 4, hidden, seed=T + 3 * hidden, addend=addend, rescale_rows=True)
    print(f"T={T} hidden={hidden} addend={addend}", flush=True)
    inp_c = workloads.make(wl, "cpu")
    inp = gh.to_device(inp_c, "cuda")
    from rms_backward_amd.wrapper import Plan
    plan = Plan(T, 4, hidden)
    dx, dw = _run_split(inp, plan)
    h = gh.host_rows(inp, list(range(T)))
    label = f"split T={T} hidden={hidden}"
    check_dx(gh.bf16_bits_np(dx), h, wl.K, label)
    S = mhcpb_plan_split_count(plan.handle)
    check_dw(gh.host(dw), gh.host_cols(inp, list(range(wl.K))), -(-T // S), S, label)
    _fused_bits(inp, plan, dx, dw)


@pytest.mark.parametrize("T,hidden,addend", FULL)
def test_split_forms_full_size_sampled(T, hidden, addend):
    wl = workloads.custom(T, 4, hidden, seed=T + 3 * hidden, addend=addend, rescale_rows=True)
    print(f"T={T} hidden={hidden} addend={addend}", flush=True)
    inp = workloads.make(wl, "cuda")
    from rms_backward_amd.wrapper import Plan
    plan = Plan(T, 4, hidden)
    dx, dw = _run_split(inp, plan)
    S = mhcpb_plan_split_count(plan.handle)
    L = -(-T // S)
    rng = np.random.default_rng(T)
    rows = gh.sample_rows(T, L, rng, extra=8)
    cols = gh.sample_cols(wl.K, rng, extra=16, whole_first=320)
    label = f"split T={T}"
    h = gh.host_rows(inp, rows)
    check_dx(gh.bf16_bits_np(dx.index_select(0, torch.as_tensor(rows, device="cuda"))), h, wl.K,
             label)
    check_dw(gh.host(dw)[:, cols], gh.host_cols(inp, cols), L, S, label, exact_cols=32)
    assert bool(torch.isfinite(dx.float()).all().item())
    assert bool(torch.isfinite(dw).all().item())
    _fused_bits(inp, plan, dx, dw)
