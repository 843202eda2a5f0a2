"""GPU parity of the deterministic BF16 RMSNorm backward against the FP64
oracle, through the C-ABI (the second workload: the
"flashinfer.cake_rmsnorm_det_train.cake_rmsnorm_det_train_backward" page's
operation, with the textbook gradient).

Per case:
* dx: every element within half a BF16 ulp of the oracle's exact value plus
  the worst-case FP32 error of the value before its single rounding (and at
  least 99% of the elements equal to the correctly rounded oracle value);
* dw: every element within the worst-case FP32 error of the fixed summation
  order (a wave's rows, then 8 waves, then groups of block partials), relative
  Frobenius error <= 1e-6;
* inputs whose every sum is exact give bit-exact dx and dw;
* the pages' widths (256 ... 6144) with BF16 and FP32 weights, with and
  without g_residual, ragged row counts and T = 0;
* rows do not depend on T or their neighbours; repeat runs give the same dw
  bits; the event-timed form gives the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import gpu_harness as gh
from tests import metrics as mt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _check(inp, dx, dw, label, rows=None, min_exact=0.99):
    ref_dx, ref_dw = gh.rms_oracle(inp, rows)
    got = gh.host(dx.float() if rows is None else dx[rows].float()).astype(np.float64)
    sel = (lambda t: t) if rows is None else (lambda t: t[rows])
    g = mt.bf16_bits_to_f64(gh.bf16_bits_np(sel(inp["g"])))
    x = mt.bf16_bits_to_f64(gh.bf16_bits_np(sel(inp["x"])))
    w = inp["w"].double().cpu().numpy()
    rstd = gh.host(sel(inp["rstd"])).astype(np.float64)
    res = (mt.bf16_bits_to_f64(gh.bf16_bits_np(sel(inp["res"])))
           if inp.get("res") is not None else None)
    H = x.shape[1]
    err = mt.rms_dx_fp32_error(g, x, w, rstd, res, H)
    bad = mt.rms_dx_violations(got, ref_dx, err)
    exact = np.mean(got == mt.bf16_round_f64(ref_dx)) if got.size else 1.0
    print(f"{label}: dx violations {len(bad)}, exact fraction {exact:.5f}")
    assert len(bad) == 0, f"{label}: first dx violations {bad[:5].tolist()}"
    assert exact >= min_exact, label
    if rows is None:
        T = x.shape[0]
        S = mt.rms_schedule(T, H)
        got_w = gh.host(dw).astype(np.float64)
        abs_sum = (np.abs(g * x) * rstd[:, None]).sum(axis=0)
        bound = mt.rms_dw_bound(abs_sum, T, S)
        viol = np.argwhere(~(np.abs(got_w - ref_dw) <= bound))
        fro = mt.rel_frobenius(got_w, ref_dw)
        print(f"{label}: dw frob {fro:.2e}, violations {len(viol)}")
        assert len(viol) == 0, f"{label}: dw violations {viol[:5].tolist()}"
        assert fro <= 1e-6 or T == 0, label


@pytest.mark.parametrize("T,H", [(1, 8), (3, 16), (17, 520), (40, 1536), (100, 4096),
                                 (33, 5120), (65, 6144), (300, 256), (257, 1032), (16, 512),
                                 (129, 2048), (50, 5632)])
@pytest.mark.parametrize("w_f32", [False, True])
def test_small_shapes_every_element(T, H, w_f32):
    wl = workloads.rms_custom(T, H, seed=T * 31 + H, w_f32=w_f32)
    inp = workloads.rms_inputs(wl, DEV)
    dx, dw = gh.run_rmsnorm(inp)
    _check(inp, dx, dw, f"T{T} H{H} w32={w_f32}")


@pytest.mark.parametrize("T,H", [(5, 8), (70, 1536), (33, 5120), (90, 6144), (200, 5632),
                                 (21, 4096)])
def test_residual_every_element(T, H):
    wl = workloads.rms_custom(T, H, seed=T + 7 * H, residual=True)
    inp = workloads.rms_inputs(wl, DEV)
    dx, dw = gh.run_rmsnorm(inp)
    _check(inp, dx, dw, f"res T{T} H{H}")
    # the residual gradient enters dx only: dw equals the run without it
    inp0 = dict(inp, res=None)
    dx0, dw0 = gh.run_rmsnorm(inp0)
    assert torch.equal(dw, dw0)
    assert not torch.equal(dx, dx0)


@pytest.mark.parametrize("name", ["rms_small", "rms_train", "rms_long", "rms_residual",
                                  "rms_w32"])
def test_workloads_every_element(name):
    """The pages' sizes, every element of dx and dw against the oracle."""
    wl = workloads.RMS_WORKLOADS[name]
    inp = workloads.rms_inputs(wl, DEV)
    dx, dw = gh.run_rmsnorm(inp)
    _check(inp, dx, dw, name)


@pytest.mark.parametrize("T,H", [(64, 512), (1000, 1024), (4096, 2048), (333, 4096)])
def test_exact_inputs_are_bit_exact(T, H):
    """Small integers for g and x, a small-integer weight, power-of-two rstd
    and H: every product and sum is exact in FP32 in any order, so dw is the
    exact value and dx the correctly rounded one, bit for bit."""
    gen = torch.Generator().manual_seed(T + H)
    g = torch.randint(-3, 4, (T, H), generator=gen).to(torch.bfloat16)
    x = torch.randint(-3, 4, (T, H), generator=gen).to(torch.bfloat16)
    w = torch.randint(-4, 5, (H,), generator=gen).to(torch.bfloat16)
    rstd = torch.pow(2.0, torch.randint(-3, 2, (T,), generator=gen).float())
    inp = {k: v.to(DEV) for k, v in dict(g=g, x=x, w=w, rstd=rstd).items()}
    dx, dw = gh.run_rmsnorm(inp)
    ref_dx, ref_dw = gh.rms_oracle(inp)
    got = gh.host(dx.float()).astype(np.float64)
    bad = np.argwhere(got != mt.bf16_round_f64(ref_dx))
    assert len(bad) == 0, bad[:5].tolist()
    assert np.array_equal(gh.host(dw).astype(np.float64), ref_dw)


def test_bf16_and_fp32_weights_agree():
    wl = workloads.rms_custom(500, 5120, seed=3)
    inp = workloads.rms_inputs(wl, DEV)
    dx1, dw1 = gh.run_rmsnorm(inp)
    dx2, dw2 = gh.run_rmsnorm(dict(inp, w=inp["w"].float()))
    assert torch.equal(dx1, dx2) and torch.equal(dw1, dw2)


def test_rows_do_not_depend_on_t_and_dw_is_reproducible():
    wl = workloads.RMS_WORKLOADS["rms_train"]
    inp = workloads.rms_inputs(wl, DEV)
    dx, dw = gh.run_rmsnorm(inp)
    for _ in range(2):
        dx2, dw2 = gh.run_rmsnorm(inp)
        assert torch.equal(dx, dx2) and torch.equal(dw, dw2)
    for lo, hi in ((0, 1), (5, 27), (1000, 1300), (4090, 4096)):
        sub = {k: (v[lo:hi].clone() if k != "w" and v is not None else v)
               for k, v in inp.items()}
        dxs, _ = gh.run_rmsnorm(sub)
        assert torch.equal(dxs, dx[lo:hi]), (lo, hi)


def test_zero_rows_give_zero_dw():
    H = 1536
    w = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    empty = torch.empty(0, H, dtype=torch.bfloat16, device=DEV)
    inp = dict(g=empty, x=empty.clone(), w=w, rstd=torch.empty(0, device=DEV))
    dx, dw = gh.run_rmsnorm(inp)
    assert dx.shape == (0, H)
    d = gh.host(dw)
    assert np.all(d == 0) and not np.signbit(d).any()


def test_non_finite_rows():
    T, H = 6, 1024
    wl = workloads.rms_custom(T, H, seed=11)
    inp = workloads.rms_inputs(wl)
    inp["x"][1, 7] = float("nan")
    inp["g"][3, 100] = float("inf")
    inp["rstd"][4] = float("inf")
    inp = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    dx, dw = gh.run_rmsnorm(inp)
    ref_dx, ref_dw = gh.rms_oracle(inp)
    got = gh.host(dx.float())
    assert np.array_equal(np.isnan(got), np.isnan(ref_dx))
    assert np.array_equal(np.isinf(got), np.isinf(ref_dx))
    gw = gh.host(dw)
    assert np.array_equal(np.isnan(gw), np.isnan(ref_dw))
    # the rows without a non-finite input are unaffected
    assert np.all(np.isfinite(got[[0, 2, 5]]))
    _check(inp, dx, None, "finite rows", rows=[0, 2, 5])


def test_events_form_gives_the_same_bits():
    import rms_backward_amd as m
    from bench import HipEvents
    wl = workloads.rms_custom(700, 3072, seed=5, residual=True)
    inp = workloads.rms_inputs(wl, DEV)
    dx1, dw1 = gh.run_rmsnorm(inp)
    T, H = 700, 3072
    ws = torch.empty(m.mhcpb_rmsnorm_backward_workspace_bytes(T, H), dtype=torch.uint8,
                     device=DEV)
    dx = torch.full_like(dx1, float("nan"))
    dw = torch.full_like(dw1, float("nan"))
    hev = HipEvents()
    ev = [hev.create() for _ in range(3)]
    m.mhcpb_rmsnorm_backward_with_events(T, H, inp["g"], inp["x"], inp["w"], m.MHCPB_DTYPE_BF16,
                                         inp["rstd"], inp["res"], dx, dw, ws, ws.numel(),
                                         torch.cuda.current_stream().cuda_stream, *ev)
    torch.cuda.synchronize()
    assert hev.elapsed_ms(ev[0], ev[1]) > 0 and hev.elapsed_ms(ev[1], ev[2]) > 0
    for e in ev:
        hev.destroy(e)
    assert torch.equal(dx1, dx) and torch.equal(dw1, dw)


def test_workspace_is_exactly_the_block_partials():
    import rms_backward_amd as m
    for T in (1, 16, 17, 100, 4096, 4097, 16384):
        for H in (520, 5120):
            S = mt.rms_schedule(T, H)
            assert m.mhcpb_rmsnorm_backward_workspace_bytes(T, H) == S * H * 4
    # a workspace of exactly that size is enough (no hidden padding)
    wl = workloads.rms_custom(4097, 520, seed=2)
    inp = workloads.rms_inputs(wl, DEV)
    ws = torch.empty(m.mhcpb_rmsnorm_backward_workspace_bytes(4097, 520), dtype=torch.uint8,
                     device=DEV)
    dx, dw = gh.run_rmsnorm(inp, workspace=ws)
    _check(inp, dx, dw, "exact workspace")


def test_one_workspace_many_calls():
    """One workspace serves calls of different shapes in turn, each giving the
    bits of a call with a fresh workspace."""
    import rms_backward_amd as m
    shapes = [(4096, 5120), (300, 1536), (17, 6144), (4097, 520), (4096, 5120)]
    need = max(m.mhcpb_rmsnorm_backward_workspace_bytes(T, H) for T, H in shapes)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    for i, (T, H) in enumerate(shapes):
        inp = workloads.rms_inputs(workloads.rms_custom(T, H, seed=40 + i), DEV)
        dx, dw = gh.run_rmsnorm(inp, workspace=ws)
        dx_f, dw_f = gh.run_rmsnorm(inp)
        assert torch.equal(dx, dx_f) and torch.equal(dw, dw_f), (T, H)


@pytest.mark.parametrize("T,H,residual", [(65536, 5120, False), (65535, 6144, True)])
def test_large_sampled(T, H, residual):
    """65536 rows (and a ragged 65535 with g_residual): dx of sampled rows
    against the oracle on those rows; dw of sampled columns against the
    oracle on those columns (each column of dw depends on its own column
    only, so a column-sliced oracle call gives it exactly)."""
    wl = workloads.rms_custom(T, H, seed=T + H, residual=residual)
    inp = workloads.rms_inputs(wl, DEV)
    dx, dw = gh.run_rmsnorm(inp)
    rng = np.random.default_rng(T)
    rows = sorted({0, 1, 3, T // 2, T - 2, T - 1} | {int(v) for v in rng.integers(0, T, 58)})
    _check(inp, dx, dw, f"large T{T} H{H} rows", rows=rows)
    cols = torch.as_tensor(sorted({0, 7, 8, H - 1} | {int(v) for v in rng.integers(0, H, 252)}),
                           device=DEV)
    g_c = gh.bf16_bits_np(inp["g"].index_select(1, cols))
    x_c = gh.bf16_bits_np(inp["x"].index_select(1, cols))
    w_c = inp["w"].index_select(0, cols).float().cpu().numpy()
    rstd = gh.host(inp["rstd"])
    _, ref_dw = oracle.rmsnorm_backward(g_c, x_c, w_c, rstd)
    got = gh.host(dw.index_select(0, cols)).astype(np.float64)
    gx = mt.bf16_bits_to_f64(g_c) * mt.bf16_bits_to_f64(x_c)
    abs_sum = (np.abs(gx) * rstd.astype(np.float64)[:, None]).sum(axis=0)
    bound = mt.rms_dw_bound(abs_sum, T, mt.rms_schedule(T, H))
    bad = np.argwhere(~(np.abs(got - ref_dw) <= bound))
    print(f"large T{T} H{H}: dw frob {mt.rel_frobenius(got, ref_dw):.2e}, violations {len(bad)}")
    assert len(bad) == 0
    assert mt.rel_frobenius(got, ref_dw) <= 1e-6
