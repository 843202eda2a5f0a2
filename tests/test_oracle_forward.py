"""Pins of the oracle's forward map (proj = X W^T, r = sqrt(mean(X^2) + eps)).

The forward is checked against facts other than its own code:

* it is the map whose vector-Jacobian product the backward oracle computes
  (the backward page, "DSv4.1 mHC projection/RMS backward", introduction,
  defines dX and dW as that product; the backward oracle is pinned on its own
  in test_oracle.py): central differences of <P, proj> + <grad_r, r> along
  random directions of X and of W must equal <dX, dX-direction> and
  <dW, dW-direction>, which fails for a dropped gate, a transposed operand, a
  wrong 1/K, a missing eps or a sign error;
* small-integer inputs, which both modes keep exact, against a Python integer
  brute force and exact rational RMS values;
* hand-derived TF32 ties (1 + 2^-11 rounds to 1, 1 + 3 2^-11 to 1 + 2^-9);
* closed forms of r (constant, zero and Pythagorean rows) and the FP32 range
  of the sum of squares;
* the TF32 result within the operand rounding bound of the exact one.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _direction(rng, shape, x, h):
    """FP32 points x +- h d and the exact FP64 difference between them."""
    d = rng.standard_normal(shape)
    xp = (x.astype(np.float64) + h * d).astype(np.float32)
    xm = (x.astype(np.float64) - h * d).astype(np.float32)
    return xp, xm, xp.astype(np.float64) - xm.astype(np.float64)


def _objective(x, w, gp, gr, eps):
    proj, r = oracle.forward(x, w, eps=eps, mode="exact")
    return float((gp[:, :24].astype(np.float64) * proj).sum() + (gr.astype(np.float64) * r).sum())


@pytest.mark.parametrize("T,K,eps", [(1, 8, 1e-6), (4, 16, 1e-6), (6, 40, 0.25), (3, 264, 1e-6)])
def test_backward_is_the_vjp_of_the_forward(T, K, eps):
    rng = np.random.default_rng(1000 * T + K)
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((24, K)) * 0.5).astype(np.float32)
    gp = np.zeros((T, 32), dtype=np.float32)
    gp[:, :24] = rng.standard_normal((T, 24)).astype(np.float32)
    gr = rng.standard_normal(T).astype(np.float32)
    _, r64 = oracle.forward(x, w, eps=eps, mode="exact")
    r = r64.astype(np.float32)
    dx = oracle.dx(x, w, gp, gr, r, K, mode="exact")
    dw = oracle.dw(x, gp, mode="exact")
    h = 2.0 ** -12
    for _ in range(3):
        xp, xm, delta = _direction(rng, x.shape, x, h)
        lhs = _objective(xp, w, gp, gr, eps) - _objective(xm, w, gp, gr, eps)
        rhs = float((dx * delta).sum())
        # r enters the backward in FP32 (relative 2^-24); the objective's
        # second-order terms vanish in a central difference of exact steps
        scale = float((np.abs(dx) * np.abs(delta)).sum())
        assert abs(lhs - rhs) <= 1e-6 * scale, (lhs, rhs)
        wp, wm, delta_w = _direction(rng, w.shape, w, h)
        lhs_w = _objective(x, wp, gp, gr, eps) - _objective(x, wm, gp, gr, eps)
        rhs_w = float((dw * delta_w).sum())
        scale_w = float((np.abs(dw) * np.abs(delta_w)).sum())
        assert abs(lhs_w - rhs_w) <= 1e-9 * scale_w, (lhs_w, rhs_w)


@pytest.mark.parametrize("mode", ["exact", "tf32"])
def test_integer_brute_force(mode):
    rng = np.random.default_rng(7)
    T, K = 5, 24
    xi = rng.integers(-2047, 2048, size=(T, K))
    wi = rng.integers(-2047, 2048, size=(24, K))
    eps = 0.25
    proj, r = oracle.forward(xi.astype(np.float32), wi.astype(np.float32), eps=eps, mode=mode)
    for t in range(T):
        for j in range(24):
            want = sum(int(xi[t, k]) * int(wi[j, k]) for k in range(K))
            assert proj[t, j] == want
        mean_sq = Fraction(sum(int(v) * int(v) for v in xi[t]), K) + Fraction(1, 4)
        assert abs(r[t] - math.sqrt(mean_sq)) <= 1e-15 * r[t]


def test_tf32_ties_round_to_even():
    K = 8
    w = np.zeros((24, K), dtype=np.float32)
    w[5, 3] = 1.0
    w[9, 3] = 3.0
    x = np.zeros((2, K), dtype=np.float32)
    x[0, 3] = 1.0 + 2.0 ** -11        # tie between 1 and 1 + 2^-10: even is 1
    x[1, 3] = 1.0 + 3 * 2.0 ** -11    # tie between 1 + 2^-10 and 1 + 2^-9
    proj, _ = oracle.forward(x, w, eps=0.0, mode="tf32")
    assert proj[0, 5] == 1.0 and proj[0, 9] == 3.0
    assert proj[1, 5] == 1.0 + 2.0 ** -9 and proj[1, 9] == 3.0 * (1.0 + 2.0 ** -9)
    exact, _ = oracle.forward(x, w, eps=0.0, mode="exact")
    assert exact[0, 5] == 1.0 + 2.0 ** -11 and exact[1, 9] == 3.0 * (1.0 + 3 * 2.0 ** -11)
    others = np.ones(24, dtype=bool)
    others[[5, 9]] = False
    assert np.all(proj[:, others] == 0.0)


def test_w_is_rounded_too():
    K = 16
    x = np.zeros((1, K), dtype=np.float32)
    x[0, 11] = 2.0
    w = np.zeros((24, K), dtype=np.float32)
    w[23, 11] = 1.0 + 2.0 ** -11 + 2.0 ** -20   # above the tie: rounds up
    proj, _ = oracle.forward(x, w, eps=0.0, mode="tf32")
    assert proj[0, 23] == 2.0 * (1.0 + 2.0 ** -10)


def test_r_closed_forms():
    K = 40
    x = np.zeros((5, K), dtype=np.float32)
    x[0, :] = 3.0                  # constant row
    x[2, 0], x[2, 7] = 3.0, 4.0    # 3-4-5
    x[3, :] = -0.5
    x[4, 1] = 1e20                 # its square leaves the FP32 range
    w = np.zeros((24, K), dtype=np.float32)
    eps = 1e-6
    _, r = oracle.forward(x, w, eps=np.float32(eps), mode="tf32")
    e = float(np.float32(eps))
    assert abs(r[0] - math.sqrt(9.0 + e)) <= 1e-15
    assert r[1] == math.sqrt(e)
    assert abs(r[2] - math.sqrt(25.0 / K + e)) <= 1e-15
    assert abs(r[3] - math.sqrt(0.25 + e)) <= 1e-15
    assert math.isinf(r[4]) and r[4] > 0


def test_non_finite_rows():
    K = 8
    x = np.ones((3, K), dtype=np.float32)
    x[0, 2] = np.nan
    x[1, 5] = np.inf
    w = np.full((24, K), 0.5, dtype=np.float32)
    proj, r = oracle.forward(x, w, eps=1e-6, mode="tf32")
    assert np.all(np.isnan(proj[0])) and math.isnan(r[0])
    assert np.all(np.isposinf(proj[1])) and math.isinf(r[1])
    assert np.all(proj[2] == K * 0.5) and np.isfinite(r[2])


def test_tf32_within_operand_rounding_bound():
    rng = np.random.default_rng(11)
    T, K = 6, 96
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = rng.standard_normal((24, K)).astype(np.float32)
    exact, r_e = oracle.forward(x, w, mode="exact")
    tf, r_t = oracle.forward(x, w, mode="tf32")
    # |TF32(a) TF32(b) - a b| <= (2 u + u^2) |a b|, u = 2^-11 (half a TF32 ulp)
    u = 2.0 ** -11
    bound = (2 * u + u * u) * (np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T)
    diff = np.abs(tf - exact)
    assert np.all(diff <= bound * (1 + 1e-12))
    assert diff.max() > 0          # the rounding does change the result
    assert np.array_equal(r_e, r_t)  # the RMS never sees TF32


def test_rows_are_independent_and_eps_is_checked():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 24)).astype(np.float32)
    w = rng.standard_normal((24, 24)).astype(np.float32)
    p_all, r_all = oracle.forward(x, w)
    p_sub, r_sub = oracle.forward(x[[5, 1]], w)
    assert np.array_equal(p_all[[5, 1]], p_sub) and np.array_equal(r_all[[5, 1]], r_sub)
    with pytest.raises(ValueError):
        oracle.forward(x, w, eps=-1.0)
    with pytest.raises(ValueError):
        oracle.forward(x, w, eps=float("nan"))
