"""GPU parity: the HIP path through the C-ABI against the FP64 oracle.

Small shapes (several column tiles, several slabs, ragged row and column
tails) are compared element by element on every output.  The full-size
workloads (4096, 4095, 16384 and 65536 tokens at 4 streams x hidden 5120, one
with the fused BF16 addend) are compared on sampled rows of dX (every column)
and sampled columns of dW (every row), in the launch configuration the
benchmark times.

Bounds ("DSv4.1 mHC projection/RMS backward": TF32 products, FP32
accumulation, BF16 dX): relative Frobenius <= 4e-3 (dX) and <= 2e-3 (dW)
against both oracle modes; per element, dX within 2 BF16 ulps + 1e-4 max|ref|
of the TF32-mode oracle, and dW within the worst-case FP32 summation bound of
the TF32-mode oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from rms_backward_amd import mhcpb_plan_partial_slabs, mhcpb_plan_split_count
from tests import gpu_harness as gh
from tests.oracle_checks import check_dw as _check_dw
from tests.oracle_checks import check_dx as _check_dx

pytestmark = pytest.mark.gpu

SMALL = [
    # T, hidden, addend, rescale_rows
    (1, 2, False, False),
    (3, 6, False, False),
    (16, 64, False, False),
    (17, 66, True, False),
    (65, 10, False, False),       # 2 slabs of 33 and 32 rows: steps end inside a slab
    (100, 128, False, True),      # 2 slabs of 50 rows
    (300, 50, True, False),       # 5 slabs of 60 rows
    (449, 20, False, False),      # 8 slabs of 57 rows, the last 50
    (513, 130, False, False),     # 8 slabs of 65 rows (the last 58), ragged column tile
    (1100, 96, True, True),       # 8 slabs of 138 rows, the last 134
    (2049, 34, False, False),     # 8 slabs of 257 rows (the last 250), K = 136 < one tile
    (4097, 8, False, False),      # 9 slabs of 456 rows, the last 449
]


@pytest.mark.parametrize("T,hidden,addend,rescale", SMALL)
def test_small_shapes_every_element(T, hidden, addend, rescale):
    wl = workloads.custom(T, 4, hidden, seed=T * 7 + hidden, addend=addend,
                          rescale_rows=rescale)
    inp_c = workloads.make(wl, "cpu")
    inp = gh.to_device(inp_c, "cuda")
    dx, dw, ws, plan = gh.run(inp)
    K = wl.K
    h = {k: (v.numpy() if v is not None and k != "addend" else None) for k, v in inp_c.items()}
    if addend:
        h["addend"] = inp_c["addend"].view(torch.int16).numpy().view(np.uint16)
    label = f"T={T} hidden={hidden}"
    _check_dx(gh.bf16_bits_np(dx), h, K, label)
    S = mhcpb_plan_split_count(plan.handle)
    L = -(-T // S)
    _check_dw(gh.host(dw), dict(x=h["x"], grad_proj=h["grad_proj"]), L, S, label)


def _random_shapes(n, seed=20261203):
    """Seeded (T, hidden, addend, rescale) draws: T from 1 to 3000, uniform and
    log-uniform in turn (split counts 1 to 8, ragged last steps and slabs),
    hidden even from 2 to 700 (K from 8 to 2800: ragged column tiles, K below
    one wave's columns)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        if i % 2:
            T = max(1, int(round(float(np.exp(rng.uniform(0.0, np.log(3000.0)))))))
        else:
            T = int(rng.integers(1, 3001))
        hidden = 2 * int(rng.integers(1, 351))
        out.append((T, hidden, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("T,hidden,addend,rescale", _random_shapes(20))
def test_random_shapes_every_element(T, hidden, addend, rescale):
    test_small_shapes_every_element(T, hidden, addend, rescale)


def test_tiny_workload_every_element():
    wl = workloads.WORKLOADS["tiny"]
    inp = workloads.make(wl, "cuda")
    dx, dw, ws, plan = gh.run(inp)
    h = gh.host_rows(inp, list(range(wl.T)))
    _check_dx(gh.bf16_bits_np(dx), h, wl.K, "tiny")
    S = mhcpb_plan_split_count(plan.handle)
    _check_dw(gh.host(dw), gh.host_cols(inp, list(range(wl.K))), -(-wl.T // S), S, "tiny")


@pytest.mark.parametrize("name", ["train", "ragged", "long", "addend", "large"])
def test_full_size_sampled(name):
    wl = workloads.WORKLOADS[name]
    print(f"workload {name}: T={wl.T} K={wl.K}", flush=True)
    inp = workloads.make(wl, "cuda")
    dx, dw, ws, plan = gh.run(inp)
    S = mhcpb_plan_split_count(plan.handle)
    L = -(-wl.T // S)
    rng = np.random.default_rng(wl.seed)
    rows = gh.sample_rows(wl.T, L, rng, extra=16)
    # dW: every column of one or more whole workgroup tiles (each wave, lane
    # group and column variant), the last columns, and random ones
    whole = 512 if wl.T <= 16384 else 64
    cols = gh.sample_cols(wl.K, rng, extra=24, whole_first=whole)
    h = gh.host_rows(inp, rows)
    dx_rows = gh.bf16_bits_np(dx.index_select(0, torch.as_tensor(rows, device="cuda")))
    _check_dx(dx_rows, h, wl.K, name)
    _check_dw(gh.host(dw)[:, cols], gh.host_cols(inp, cols), L, S, name, exact_cols=48)
    # every dX and dW element is finite (the poison is gone everywhere)
    assert bool(torch.isfinite(dx.float()).all().item())
    assert bool(torch.isfinite(dw).all().item())


def test_max_hidden_sampled():
    """The widest supported row (hidden = 2^20, K = 4,194,304 columns) over 40
    tokens (three steps, the last one ragged): offsets and ranges at their
    largest.  Sampled dX rows (every column) and dW columns near both ends."""
    wl = workloads.custom(40, 4, 1 << 20, seed=77, rescale_rows=True)
    print(f"T={wl.T} K={wl.K}", flush=True)
    inp = workloads.make(wl, "cuda")
    dx, dw, ws, plan = gh.run(inp)
    S = mhcpb_plan_split_count(plan.handle)
    L = -(-wl.T // S)
    rows = [0, 15, 16, 31, 32, 39]
    h = gh.host_rows(inp, rows)
    dx_rows = gh.bf16_bits_np(dx.index_select(0, torch.as_tensor(rows, device="cuda")))
    _check_dx(dx_rows, h, wl.K, "max hidden")
    K = wl.K
    cols = sorted({0, 1, 2, 3, 319, 320, K // 2, K - 321, K - 320, K - 65, K - 64, K - 4,
                   K - 3, K - 2, K - 1})
    _check_dw(gh.host(dw)[:, cols], gh.host_cols(inp, cols), L, S, "max hidden")
    assert bool(torch.isfinite(dx.float()).all().item())
    assert bool(torch.isfinite(dw).all().item())


@pytest.mark.parametrize("T,hidden", [(600, 20480), (1300, 20800)])
def test_single_slab_group_sampled(T, hidden):
    """K >= 256 * 320 columns: the column tiles alone fill 256 CUs, so one slab
    group walks every slab of its tile and stores only their running sum (the
    whole ascending sum); kernel 2 then starts from the last slab.  Sampled
    dX rows (every column) and dW columns (every row), several whole tiles."""
    wl = workloads.custom(T, 4, hidden, seed=T + hidden, rescale_rows=True)
    print(f"T={wl.T} K={wl.K}", flush=True)
    inp = workloads.make(wl, "cuda")
    dx, dw, ws, plan = gh.run(inp)
    S = mhcpb_plan_split_count(plan.handle)
    assert S == 8
    L = -(-wl.T // S)
    rng = np.random.default_rng(wl.seed)
    rows = gh.sample_rows(wl.T, L, rng, extra=8)
    cols = gh.sample_cols(wl.K, rng, extra=24, whole_first=640)
    h = gh.host_rows(inp, rows)
    dx_rows = gh.bf16_bits_np(dx.index_select(0, torch.as_tensor(rows, device="cuda")))
    _check_dx(dx_rows, h, wl.K, f"T={T} hidden={hidden}")
    _check_dw(gh.host(dw)[:, cols], gh.host_cols(inp, cols), L, S, f"T={T} hidden={hidden}",
              exact_cols=48)
    assert bool(torch.isfinite(dx.float()).all().item())
    assert bool(torch.isfinite(dw).all().item())


def test_one_wave_workgroups_several_per_cu_every_element():
    """K = 3200 at 8 slabs: 320-column tiles would fill 80 CUs, so kernel 1
    runs 400 one-wave workgroups (50 tiles of 64 columns x 8 slabs), more
    than one per CU.  Every element against the oracle."""
    test_small_shapes_every_element(4096, 800, True, True)


@pytest.mark.parametrize("T,hidden,addend,rescale", [
    (1000, 3000, False, True),   # K = 12000: 38 tiles of 320 columns x 8 slabs, 6 slab groups
    (777, 2750, True, False),    # K = 11000, ragged last tile and last slab
    (520, 5120, True, True),     # K = 20480: 4 slab groups of 2 slabs, group 0 adds its two up
])
def test_five_wave_workgroups_every_element(T, hidden, addend, rescale):
    """Kernel 1 with five compute waves per workgroup (320-column tiles, one
    workgroup per CU; the two waves that share a SIMD take turns at a raised
    priority), every element against the oracle; at K = 20480 the workgroups
    of slab group 0 add the partials of slabs 0 and 1 before storing them."""
    if hidden == 5120:
        plan = gh.Plan(T, 4, hidden)
        assert mhcpb_plan_split_count(plan.handle) == 8
        assert mhcpb_plan_partial_slabs(plan.handle) == 7
    test_small_shapes_every_element(T, hidden, addend, rescale)


def test_uneven_slab_groups_sampled():
    """T = 4097: 9 slabs in 4 slab groups of 2, 2, 2 and 3 consecutive slabs;
    group 0 adds slabs 0 and 1 up before storing them."""
    wl = workloads.custom(4097, 4, 5120, seed=4097 + 5120, rescale_rows=True)
    print(f"T={wl.T} K={wl.K}", flush=True)
    inp = workloads.make(wl, "cuda")
    dx, dw, ws, plan = gh.run(inp)
    S = mhcpb_plan_split_count(plan.handle)
    assert S == 9
    L = -(-wl.T // S)
    rng = np.random.default_rng(wl.seed)
    rows = gh.sample_rows(wl.T, L, rng, extra=8)
    cols = gh.sample_cols(wl.K, rng, extra=24, whole_first=640)
    h = gh.host_rows(inp, rows)
    dx_rows = gh.bf16_bits_np(dx.index_select(0, torch.as_tensor(rows, device="cuda")))
    _check_dx(dx_rows, h, wl.K, "T=4097")
    _check_dw(gh.host(dw)[:, cols], gh.host_cols(inp, cols), L, S, "T=4097", exact_cols=48)
    assert bool(torch.isfinite(dx.float()).all().item())
    assert bool(torch.isfinite(dw).all().item())
