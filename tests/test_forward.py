"""GPU parity of the forward map (proj = X W^T with TF32 operands, r = RMS)
against the FP64 oracle, through the C-ABI.

Checks, per case:
* proj columns 24..31 are +0 and nothing else is left unwritten;
* random inputs: relative Frobenius error of the 24 logits <= 1e-5 against
  the TF32-mode oracle, every row's relative error <= 1e-4, every element
  within 1e-4 of its row's largest logit; r within the worst-case FP32
  summation bound of its sum of squares (the GPU sums at most K/4 + 64 terms
  in a chain) plus the rounding of the division, eps and square root;
* exactly representable cases are bit-exact: odd integers up to 2047 (11
  significant bits, so both BF16 parts of every TF32 operand take part)
  against signs, whose sums stay below 2^24; one value per row, whose single
  product is exact, with random low bits and TF32 ties on both operands;
* the pages' sizes (4095, 4096, 16384 and 65536 tokens, K = 20480) on
  sampled rows;
* every row's bits are independent of T and of the other rows, repeat runs
  and the event-timed form give the same bits;
* non-finite and extreme rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import gpu_harness as gh
from tests import metrics as mt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EPS = 1e-6


def _oracle_rows(x_c, w_c, rows, eps=EPS, mode="tf32"):
    xs = x_c[rows].numpy() if rows is not None else x_c.numpy()
    return oracle.forward(xs, w_c.numpy(), eps=float(np.float32(eps)), mode=mode)


def _check_random(proj, r, ref_p, ref_r, K, label):
    got = proj[:, :24].astype(np.float64)
    assert np.all(proj[:, 24:] == 0) and not np.signbit(proj[:, 24:]).any(), label
    fro = mt.rel_frobenius(got, ref_p)
    row_err = np.linalg.norm(got - ref_p, axis=1) / np.maximum(np.linalg.norm(ref_p, axis=1), 1e-30)
    elem = np.abs(got - ref_p) / np.maximum(np.abs(ref_p).max(axis=1, keepdims=True), 1e-30)
    print(f"{label}: proj frob {fro:.2e} max row {row_err.max():.2e} max elem {elem.max():.2e}")
    assert fro <= mt.FWD_PROJ_FROB, label
    assert row_err.max() <= mt.FWD_PROJ_ROW, label
    assert elem.max() <= mt.FWD_PROJ_ELEM, label
    rel_r = np.abs(r.astype(np.float64) - ref_r) / ref_r
    bound = mt.fwd_r_rel_bound(K)
    print(f"{label}: r max rel {rel_r.max():.2e} (bound {bound:.2e})")
    assert np.all(rel_r <= bound), label


@pytest.mark.parametrize("T,hidden", [(1, 2), (16, 16), (17, 24), (40, 130), (300, 96),
                                      (64, 512), (33, 1030)])
def test_small_shapes_every_element(T, hidden):
    wl = workloads.custom(T, 4, hidden, seed=T * 7 + hidden)
    inp = workloads.forward_inputs(wl)
    proj, r, _ = gh.run_forward(inp["x"].to(DEV), inp["w"].to(DEV))
    ref_p, ref_r = _oracle_rows(inp["x"], inp["w"], None)
    _check_random(gh.host(proj), gh.host(r), ref_p, ref_r, wl.K, f"T{T} h{hidden}")


def _random_shapes(n, seed=20261204):
    """Seeded (T, hidden) draws: T from 1 to 2000, uniform and log-uniform in
    turn; hidden even from 2 to 1400 (K up to 5600: one to six 1024-column
    tiles, ragged in every position)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        if i % 2:
            T = max(1, int(round(float(np.exp(rng.uniform(0.0, np.log(2000.0)))))))
        else:
            T = int(rng.integers(1, 2001))
        out.append((T, 2 * int(rng.integers(1, 701))))
    return out


@pytest.mark.parametrize("T,hidden", _random_shapes(12))
def test_random_shapes_every_element(T, hidden):
    test_small_shapes_every_element(T, hidden)


@pytest.mark.parametrize("K,T", [(20480, 64), (4120, 33), (2048, 40)])
def test_integers_are_exact(K, T):
    """Odd integers against signs, both ways round: every partial sum is an
    integer below 2^24, so any FP32 order gives the exact logits."""
    for swap in (False, True):
        a = workloads.odd_integers((T, K) if not swap else (24, K), seed=K + T + swap)
        b = workloads.sparse_signs((24, K) if not swap else (T, K), seed=K * 3 + T + swap)
        x, w = (a, b) if not swap else (b, a)
        proj, r, _ = gh.run_forward(x.to(DEV), w.to(DEV), eps=0.25)
        ref_p, ref_r = oracle.forward(x.numpy(), w.numpy(), eps=0.25)
        got = gh.host(proj)
        assert np.array_equal(got[:, :24].astype(np.float64), ref_p), f"K{K} swap {swap}"
        assert np.all(got[:, 24:] == 0)
        if swap:  # x in {-1, 0, 1}: the sum of squares is exact, r within 2 ulp
            assert np.all(np.abs(gh.host(r) - ref_r) <= 2 * 2.0 ** -23 * ref_r)


@pytest.mark.parametrize("K,T", [(20480, 48), (520, 70)])
def test_one_value_per_row_is_bit_exact(K, T):
    """A single product per logit: the TF32 rounding of both operands (ties
    included) shows bit for bit."""
    x = workloads.one_hot_rows(T, K, seed=K + T)
    w = workloads.low_bit_values((24, K), seed=K - T)
    proj, r, _ = gh.run_forward(x.to(DEV), w.to(DEV))
    ref_p, _ = oracle.forward(x.numpy(), w.numpy(), eps=float(np.float32(EPS)))
    got = gh.host(proj)[:, :24].astype(np.float64)
    bad = np.argwhere(got != ref_p)
    assert len(bad) == 0, f"first mismatches {bad[:5].tolist()}"
    # and the exact-mode oracle differs: the TF32 rounding is really applied
    ex_p, _ = oracle.forward(x.numpy(), w.numpy(), mode="exact")
    assert np.count_nonzero(got != ex_p) > got.size // 2


@pytest.mark.parametrize("name", ["train", "long", "large", "ragged"])
def test_full_size_sampled(name):
    wl = workloads.WORKLOADS[name]
    inp = workloads.forward_inputs(wl, DEV)
    proj, r, _ = gh.run_forward(inp["x"], inp["w"])
    T = wl.T
    rng = np.random.default_rng(wl.seed)
    rows = sorted({0, 1, 15, 16, 17, T // 2, T - 17, T - 16, T - 1} |
                  {int(v) for v in rng.integers(0, T, size=40)})
    x_c = inp["x"][rows].cpu()
    ref_p, ref_r = oracle.forward(x_c.numpy(), inp["w"].cpu().numpy(),
                                  eps=float(np.float32(EPS)))
    p_h, r_h = gh.host(proj), gh.host(r)
    _check_random(p_h[rows], r_h[rows], ref_p, ref_r, wl.K, name)
    assert np.all(p_h[:, 24:] == 0) and np.all(np.isfinite(p_h)) and np.all(r_h > 0)


def test_rows_do_not_depend_on_t_or_neighbours():
    wl = workloads.WORKLOADS["train"]
    inp = workloads.forward_inputs(wl, DEV)
    x, w = inp["x"], inp["w"]
    p_all, r_all, _ = gh.run_forward(x, w)
    p_again, r_again, _ = gh.run_forward(x, w)
    assert torch.equal(p_all, p_again) and torch.equal(r_all, r_again)
    for lo, hi in ((0, 1), (5, 27), (1000, 1100), (4093, 4096)):
        p_sub, r_sub, _ = gh.run_forward(x[lo:hi].contiguous(), w)
        assert torch.equal(p_sub, p_all[lo:hi]) and torch.equal(r_sub, r_all[lo:hi]), (lo, hi)
    perm = torch.randperm(wl.T, generator=torch.Generator().manual_seed(3)).to(DEV)
    p_perm, r_perm, _ = gh.run_forward(x[perm].contiguous(), w)
    assert torch.equal(p_perm, p_all[perm]) and torch.equal(r_perm, r_all[perm])


def test_events_form_gives_the_same_bits():
    import rms_backward_amd as m
    from bench import HipEvents
    wl = workloads.custom(300, 4, 1030, seed=9)
    inp = workloads.forward_inputs(wl, DEV)
    p1, r1, plan = gh.run_forward(inp["x"], inp["w"])
    proj = torch.full_like(p1, float("nan"))
    r = torch.full_like(r1, float("nan"))
    ws = plan.alloc_forward_workspace(DEV)
    hev = HipEvents()
    ev = [hev.create() for _ in range(3)]
    m.mhcpb_forward_with_events(plan.handle, inp["x"], inp["w"], 1e-6, proj, r, ws, ws.numel(),
                                torch.cuda.current_stream().cuda_stream, *ev)
    torch.cuda.synchronize()
    assert hev.elapsed_ms(ev[0], ev[1]) > 0 and hev.elapsed_ms(ev[1], ev[2]) > 0
    for e in ev:
        hev.destroy(e)
    assert torch.equal(p1, proj) and torch.equal(r1, r)


def test_non_finite_and_extreme_rows():
    K = 2048
    T = 10
    x = workloads.low_bit_values((T, K), seed=1)
    w = workloads.low_bit_values((24, K), seed=2) * 0.02
    u = x.view(torch.int32)
    u[0, 5] = 0x7FFFFFFF           # NaN whose TF32 rounding would carry
    u[1, 100] = 0x7FC00000         # the canonical quiet NaN
    u[2, 2047] = -1                # 0xFFFFFFFF, a negative NaN
    x[3, 7] = float("inf")
    x[4, :] = 0.0                  # r = sqrt(eps)
    x[5, :] = 3e19                 # the sum of squares leaves the FP32 range
    x[6, :] *= 1e-30               # tiny but normal
    x[7, :] *= 1e15
    proj, r, _ = gh.run_forward(x.to(DEV), w.to(DEV), eps=0.5)
    p, rr = gh.host(proj), gh.host(r)
    ref_p, ref_r = oracle.forward(x.numpy(), w.numpy(), eps=0.5)
    for t in (0, 1, 2):
        assert np.all(np.isnan(p[t, :24])) and math.isnan(rr[t]), t
    assert np.all(~np.isfinite(p[3, :24])) and math.isinf(rr[3])
    assert np.all(p[4, :24] == 0) and rr[4] == np.float32(math.sqrt(0.5))
    assert math.isinf(rr[5]) and math.isinf(ref_r[5])
    assert np.all(p[:, 24:] == 0)
    ok = [6, 7, 8, 9]
    _check_random(p[ok], rr[ok], ref_p[ok], ref_r[ok], K, "extreme rows")


def test_zero_eps_zero_row():
    x = torch.zeros(3, 64)
    x[1, 3] = 2.0
    w = torch.ones(24, 64)
    proj, r, _ = gh.run_forward(x.to(DEV), w.to(DEV), eps=0.0)
    assert gh.host(r).tolist() == [0.0, np.float32(math.sqrt(4.0 / 64)), 0.0]
    assert np.all(gh.host(proj)[1, :24] == 2.0) and np.all(gh.host(proj)[[0, 2]] == 0)
