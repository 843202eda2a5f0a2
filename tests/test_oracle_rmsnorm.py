"""Pins of the oracle's BF16 RMSNorm backward (second workload).

The page ("flashinfer.cake_rmsnorm_det_train.cake_rmsnorm_det_train_backward",
signature and parameters) names the inputs and outputs but prints no formula;
the oracle implements the textbook gradient.  It is checked here against
facts outside its own code:

* central differences of <g, y> for the forward y = x rstd(x) w (rstd =
  (mean(x^2) + eps)^-1/2, recomputed from x) along random directions of x and
  of w equal <dx, d> and <dw, d>;
* the scale identity sum_h x dx = H eps rstd^3 c1 (the gradient is
  orthogonal to x when eps = 0), with c1 = sum_h w g x / H;
* a constant row, whose dx is rstd eps / (a^2 + eps) by hand;
* g_residual adds itself exactly.
"""
import math

import numpy as np
import pytest

import oracle


def bf16_bits(a):
    """BF16 bits of FP32 values rounded to nearest even (a test-side helper
    used only to draw BF16 inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _rstd(x, eps):
    return 1.0 / np.sqrt((x * x).mean(axis=1) + eps)


def _objective(x, w, g, eps):
    return float((g * x * _rstd(x, eps)[:, None] * w[None, :]).sum())


@pytest.mark.parametrize("T,H,eps", [(1, 8, 1e-6), (3, 16, 1e-5), (5, 64, 0.1), (2, 256, 1e-6)])
def test_backward_is_the_vjp_of_rmsnorm(T, H, eps):
    rng = np.random.default_rng(100 * T + H)
    xb = bf16_bits(rng.standard_normal((T, H)))
    gb = bf16_bits(rng.standard_normal((T, H)))
    w = rng.standard_normal(H).astype(np.float32)
    x, g = bits_to_f64(xb), bits_to_f64(gb)
    rstd = _rstd(x, eps)
    dx, dw = oracle.rmsnorm_backward(gb, xb, w, rstd.astype(np.float32))
    h = 1e-6
    w64 = w.astype(np.float64)
    for _ in range(3):
        d = rng.standard_normal((T, H))
        lhs = (_objective(x + h * d, w64, g, eps) - _objective(x - h * d, w64, g, eps)) / (2 * h)
        rhs = float((dx * d).sum())
        assert abs(lhs - rhs) <= 1e-6 * float((np.abs(dx) * np.abs(d)).sum()) + 1e-9, (lhs, rhs)
        dwd = rng.standard_normal(H)
        lhs_w = (_objective(x, w64 + h * dwd, g, eps) - _objective(x, w64 - h * dwd, g, eps)) / (2 * h)
        rhs_w = float((dw * dwd).sum())
        assert abs(lhs_w - rhs_w) <= 1e-6 * float((np.abs(dw) * np.abs(dwd)).sum()) + 1e-9


def test_scale_identity():
    rng = np.random.default_rng(5)
    T, H, eps = 4, 512, 1e-3
    xb = bf16_bits(rng.standard_normal((T, H)))
    gb = bf16_bits(rng.standard_normal((T, H)))
    w = rng.standard_normal(H).astype(np.float32)
    x, g = bits_to_f64(xb), bits_to_f64(gb)
    rstd = _rstd(x, eps).astype(np.float32).astype(np.float64)
    dx, _ = oracle.rmsnorm_backward(gb, xb, w, rstd.astype(np.float32))
    c1 = (w[None, :] * g * x).sum(axis=1) / H
    # sum_h x dx = rstd H c1 - rstd^3 c1 sum x^2, with the given rstd
    want = rstd * H * c1 - rstd ** 3 * c1 * (x * x).sum(axis=1)
    got = (x * dx).sum(axis=1)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-10 * np.abs(want).max())
    # and with the exact rstd of x that equals H eps rstd^3 c1 (zero when eps = 0)
    rs = _rstd(x, eps)
    assert np.allclose(rs * H * c1 - rs ** 3 * c1 * (x * x).sum(axis=1), H * eps * rs ** 3 * c1,
                       rtol=1e-9, atol=1e-12)


def test_constant_row_by_hand():
    H = 64
    a, eps = 1.0, 1.0
    xb = bf16_bits(np.full((1, H), a))
    gb = bf16_bits(np.ones((1, H)))
    w = np.ones(H, dtype=np.float32)
    rstd = np.array([1.0 / math.sqrt(a * a + eps)], dtype=np.float32)
    dx, dw = oracle.rmsnorm_backward(gb, xb, w, rstd)
    rs = float(rstd[0])
    assert np.allclose(dx, rs * (1.0 - rs * rs * a * a))       # = rstd eps / (a^2 + eps)
    assert abs(rs * (1.0 - rs * rs) - 0.5 / math.sqrt(2.0)) < 1e-7
    assert np.all(dw == a * rs)


def test_residual_is_added_once_and_dw_ignores_it():
    rng = np.random.default_rng(9)
    T, H = 3, 40
    xb = bf16_bits(rng.standard_normal((T, H)))
    gb = bf16_bits(rng.standard_normal((T, H)))
    rb = bf16_bits(rng.standard_normal((T, H)))
    w = rng.standard_normal(H).astype(np.float32)
    rstd = rng.uniform(0.5, 2.0, T).astype(np.float32)
    dx0, dw0 = oracle.rmsnorm_backward(gb, xb, w, rstd)
    dx1, dw1 = oracle.rmsnorm_backward(gb, xb, w, rstd, res_bits=rb)
    # (dx0 + res) - dx0 in FP64: exact up to one rounding of the sum
    assert np.allclose(dx1 - dx0, bits_to_f64(rb), rtol=0, atol=1e-14)
    assert not np.allclose(dx1, dx0)
    assert np.array_equal(dw0, dw1)


def test_rows_independent_and_dw_sums_rows():
    rng = np.random.default_rng(2)
    T, H = 6, 24
    xb = bf16_bits(rng.standard_normal((T, H)))
    gb = bf16_bits(rng.standard_normal((T, H)))
    w = rng.standard_normal(H).astype(np.float32)
    rstd = rng.uniform(0.5, 2.0, T).astype(np.float32)
    dx, dw = oracle.rmsnorm_backward(gb, xb, w, rstd)
    parts = [oracle.rmsnorm_backward(gb[t:t + 1], xb[t:t + 1], w, rstd[t:t + 1]) for t in range(T)]
    assert np.array_equal(np.vstack([p[0] for p in parts]), dx)
    assert np.allclose(sum(p[1] for p in parts), dw, rtol=1e-14, atol=0)
