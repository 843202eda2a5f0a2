"""Pins of the CPU oracle against what the pages and the mathematics fix.

The oracle (oracle/mhcpb_oracle.c) is the definition the GPU library is checked
against, so it is itself checked here against things other than its own code:

* the stage is the vector-Jacobian product of the forward map
  (X, W) -> (X W^T, r(X)), r(X) = sqrt(mean(X^2) + eps), for the cotangents
  (P, grad_r) -- "DSv4.1 mHC projection/RMS backward" page, introduction.
  Central finite differences and float64 autograd of that forward pin dX and
  dW, including the 1/K of the RMS term and every sign and index;
* hand-derived TF32 and BF16 bit tables (tests/golden/);
* one-hot cases that expose a single operand's TF32 value bit for bit;
* the tensor contract's invariants: the last 8 grad_proj columns are ignored
  even when NaN, and the RMS term uses raw FP32 x;
* the TF32 result stays within the rounding bound of the exact result;
* a tiny brute-force loop with TF32 rounding done on the bits (a method
  independent of the oracle's frexp/nearbyint one).
"""
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            a, b = line.split()[:2]
            rows.append((int(a, 16), b))
    return rows


def _f32_from_bits(u):
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


def _bits_from_f32(v):
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def _inputs(T, K, seed, p_scale=1.0, g_scale=1.0, eps=1e-6):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = rng.standard_normal((24, K)).astype(np.float32)
    gp = np.empty((T, 32), dtype=np.float32)
    gp[:, :24] = (rng.standard_normal((T, 24)) * p_scale).astype(np.float32)
    gp[:, 24:] = 0.0
    gr = (rng.standard_normal(T) * g_scale).astype(np.float32)
    r = np.sqrt((x.astype(np.float64) ** 2).mean(axis=1) + eps).astype(np.float32)
    return x, w, gp, gr, r


# ----------------------------------------------------------------- rounding --

def test_tf32_golden_table():
    table = _read_table("tf32_rne.txt")
    assert len(table) >= 25
    for inp, exp in table:
        got = np.float32(oracle.tf32(_f32_from_bits(inp)))
        if exp == "nan":
            assert math.isnan(got), hex(inp)
        else:
            assert _bits_from_f32(got) == int(exp, 16), (hex(inp), hex(_bits_from_f32(got)), exp)


def test_bf16_golden_table():
    table = _read_table("bf16_rne.txt")
    assert len(table) >= 20
    for inp, exp in table:
        got = oracle.bf16(_f32_from_bits(inp))
        if exp == "nan":
            assert math.isnan(got), hex(inp)
        else:
            assert oracle.bf16_bits(_f32_from_bits(inp)) == int(exp, 16), (hex(inp), exp)


def _tf32_bits_method(v):
    """TF32 by integer rounding on the FP32 bits (independent of the oracle)."""
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    if (u & 0x7F800000) == 0x7F800000:
        return struct.unpack("<f", struct.pack("<I", u | (0x400000 if u & 0x7FFFFF else 0)))[0]
    u = (u + 0xFFF + ((u >> 13) & 1)) & 0xFFFFE000
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def test_tf32_agrees_with_bit_method_on_random_values():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    # keep finite values, add many exact ties
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    ties = (bits[:4000] & np.uint32(0xFFFFE000)) | np.uint32(0x1000)
    tv = ties.view(np.float32)
    vals = np.concatenate([vals, tv[np.isfinite(tv)]])
    got = oracle.tf32_array(vals)
    ref = np.array([_tf32_bits_method(float(v)) for v in vals], dtype=np.float64)
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    assert np.all((got == ref) | both_inf)


# --------------------------------------------------- formula (VJP) pins ------

def _loss(x, w, gp, gr, eps):
    """<P, X W^T> + <grad_r, r(X)> in float64."""
    p = gp[:, :24]
    y = x @ w.T
    r = np.sqrt((x * x).mean(axis=1) + eps)
    return float((p * y).sum() + (gr * r).sum())


@pytest.mark.parametrize("T,K,eps", [(1, 8, 1e-6), (3, 8, 1e-6), (5, 16, 0.3), (7, 40, 1e-6)])
def test_vjp_finite_difference(T, K, eps):
    x, w, gp, gr, r = _inputs(T, K, seed=T * 100 + K, eps=eps)
    dx = oracle.dx(x, w, gp, gr, r, K, mode="exact")
    dw = oracle.dw(x, gp, mode="exact")
    x64, w64, gp64, gr64 = (a.astype(np.float64) for a in (x, w, gp, gr))
    h = 1e-5
    fd_x = np.empty_like(x64)
    for t in range(T):
        for k in range(K):
            e = np.zeros_like(x64)
            e[t, k] = h
            fd_x[t, k] = (_loss(x64 + e, w64, gp64, gr64, eps) -
                          _loss(x64 - e, w64, gp64, gr64, eps)) / (2 * h)
    fd_w = np.empty_like(w64)
    for j in range(24):
        for k in range(K):
            e = np.zeros_like(w64)
            e[j, k] = h
            fd_w[j, k] = (_loss(x64, w64 + e, gp64, gr64, eps) -
                          _loss(x64, w64 - e, gp64, gr64, eps)) / (2 * h)
    # r is handed to the oracle in FP32, so allow its 2^-24 relative error
    assert np.allclose(dx, fd_x, rtol=1e-6, atol=1e-6 * np.abs(fd_x).max())
    assert np.allclose(dw, fd_w, rtol=1e-7, atol=1e-7 * np.abs(fd_w).max())


@pytest.mark.parametrize("T,K", [(2, 8), (9, 24), (33, 64)])
def test_rms_term_alone_matches_finite_difference(T, K):
    """With P = 0 the only term left is grad_r * dr/dX = grad_r X / (r K)."""
    x, w, gp, gr, r = _inputs(T, K, seed=11 + T, p_scale=0.0)
    eps = 1e-6
    dx = oracle.dx(x, w, gp, gr, r, K, mode="exact")
    x64, gr64 = x.astype(np.float64), gr.astype(np.float64)
    h = 1e-6
    for t in range(T):
        for k in range(0, K, max(1, K // 8)):
            xp, xm = x64.copy(), x64.copy()
            xp[t, k] += h
            xm[t, k] -= h
            rp = np.sqrt((xp[t] ** 2).mean() + eps)
            rm = np.sqrt((xm[t] ** 2).mean() + eps)
            fd = gr64[t] * (rp - rm) / (2 * h)
            assert abs(dx[t, k] - fd) <= 2e-6 * abs(fd) + 1e-13


@pytest.mark.parametrize("T,K", [(4, 8), (6, 32), (3, 2048)])
def test_autograd_cross_check(T, K):
    x, w, gp, gr, r = _inputs(T, K, seed=3 * T + K)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    p = torch.tensor(gp[:, :24], dtype=torch.float64)
    g = torch.tensor(gr, dtype=torch.float64)
    y = xt @ wt.T
    rr = torch.sqrt((xt * xt).mean(dim=1) + 1e-6)
    ((p * y).sum() + (g * rr).sum()).backward()
    dx = oracle.dx(x, w, gp, gr, r, K, mode="exact")
    dw = oracle.dw(x, gp, mode="exact")
    assert np.allclose(dx, xt.grad.numpy(), rtol=1e-6, atol=1e-9)
    assert np.allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------- TF32 placement pins -------

def _odd_bits(rng, shape, low_mask=0x1FFF):
    """FP32 values whose low 13 fraction bits are nonzero (TF32 changes them)."""
    v = (rng.standard_normal(shape)).astype(np.float32)
    u = v.view(np.uint32)
    u |= np.uint32(0x0A55) & np.uint32(low_mask)
    return u.view(np.float32)


def test_one_hot_p_exposes_tf32_of_x_in_dw():
    rng = np.random.default_rng(1)
    K = 64
    x = _odd_bits(rng, (1, K))
    for j in (0, 7, 23):
        gp = np.zeros((1, 32), dtype=np.float32)
        gp[0, j] = 1.0
        dw = oracle.dw(x, gp, mode="tf32")
        expect = np.array([_tf32_bits_method(float(v)) for v in x[0]])
        assert np.array_equal(dw[j], expect)
        assert not np.array_equal(dw[j], x[0].astype(np.float64))  # rounding happened
        assert np.all(np.delete(dw, j, axis=0) == 0.0)


def test_one_hot_x_exposes_tf32_of_p_in_dw():
    rng = np.random.default_rng(2)
    K = 16
    gp = np.zeros((1, 32), dtype=np.float32)
    gp[0, :24] = _odd_bits(rng, 24)
    for k in (0, 5, 15):
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        dw = oracle.dw(x, gp, mode="tf32")
        expect = np.array([_tf32_bits_method(float(v)) for v in gp[0, :24]])
        assert np.array_equal(dw[:, k], expect)


def test_one_hot_p_exposes_tf32_of_w_in_dx():
    rng = np.random.default_rng(3)
    K = 32
    w = _odd_bits(rng, (24, K))
    x = rng.standard_normal((1, K)).astype(np.float32)
    gr = np.zeros(1, dtype=np.float32)
    r = np.ones(1, dtype=np.float32)
    for j in (0, 13, 23):
        gp = np.zeros((1, 32), dtype=np.float32)
        gp[0, j] = 1.0
        dx = oracle.dx(x, w, gp, gr, r, K, mode="tf32")
        expect = np.array([_tf32_bits_method(float(v)) for v in w[j]])
        assert np.array_equal(dx[0], expect)


def test_rms_term_uses_raw_x_in_tf32_mode():
    rng = np.random.default_rng(4)
    T, K = 3, 2048
    x = _odd_bits(rng, (T, K))
    w = rng.standard_normal((24, K)).astype(np.float32)
    gp = np.zeros((T, 32), dtype=np.float32)
    gr = np.array([0.5, -0.25, 2.0], dtype=np.float32)
    r = np.full(T, 2.0 ** -11, dtype=np.float32)    # r K = 1 at K = 2048
    dx_t = oracle.dx(x, w, gp, gr, r, K, mode="tf32")
    dx_e = oracle.dx(x, w, gp, gr, r, K, mode="exact")
    assert np.array_equal(dx_t, dx_e)
    assert np.array_equal(dx_t, gr[:, None].astype(np.float64) * x)


# ------------------------------------------------------- contract pins -------

@pytest.mark.parametrize("mode", ["exact", "tf32"])
def test_tail_columns_are_never_read(mode):
    x, w, gp, gr, r = _inputs(6, 40, seed=5)
    dx0 = oracle.dx(x, w, gp, gr, r, 40, mode=mode)
    dw0 = oracle.dw(x, gp, mode=mode)
    for garbage in (np.nan, np.inf, -np.inf, 1e30):
        g2 = gp.copy()
        g2[:, 24:] = garbage
        assert np.array_equal(oracle.dx(x, w, g2, gr, r, 40, mode=mode), dx0)
        assert np.array_equal(oracle.dw(x, g2, mode=mode), dw0)


def test_zero_grad_proj():
    x, w, gp, gr, r = _inputs(5, 24, seed=6, p_scale=0.0)
    dx = oracle.dx(x, w, gp, gr, r, 24, mode="tf32")
    dw = oracle.dw(x, gp, mode="tf32")
    w2 = np.random.default_rng(0).standard_normal(w.shape).astype(np.float32) * 1e3
    assert np.array_equal(oracle.dx(x, w2, gp, gr, r, 24, mode="tf32"), dx)
    assert np.all(dw == 0.0)


def test_rms_term_is_scale_invariant():
    """Scaling a row of X and its r by s leaves x / r, hence the RMS term, fixed."""
    x, w, gp, gr, r = _inputs(4, 64, seed=8, p_scale=0.0)
    s = np.array([1.0, 0.01, 100.0, 2.0 ** 20], dtype=np.float64)
    xs = (x * s[:, None]).astype(np.float32)
    rs = (r * s).astype(np.float32)
    a = oracle.dx(x, w, gp, gr, r, 64, mode="exact")
    b = oracle.dx(xs, w, gp, gr, rs, 64, mode="exact")
    assert np.allclose(a, b, rtol=3e-7, atol=0)


def test_addend_adds_exactly_once():
    x, w, gp, gr, r = _inputs(4, 16, seed=9)
    rng = np.random.default_rng(10)
    a = (rng.standard_normal((4, 16)) * 0.01).astype(np.float32)
    a_bits = (a.view(np.uint32) >> 16).astype(np.uint16)   # truncated to BF16
    a_val = (a_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    base = oracle.dx(x, w, gp, gr, r, 16, mode="tf32")
    with_a = oracle.dx(x, w, gp, gr, r, 16, addend=a_bits, mode="tf32")
    assert np.allclose(with_a - base, a_val, rtol=0, atol=1e-15)
    one = np.full((4, 16), 0x3F80, dtype=np.uint16)     # BF16 1.0
    assert np.allclose(oracle.dx(x, w, gp, gr, r, 16, addend=one, mode="tf32") - base,
                       1.0, rtol=0, atol=1e-14)


def test_tf32_within_rounding_bound_of_exact():
    """|TF32 result - exact| <= sum |p||w| (2^-10 + 2^-22), and it is not zero."""
    x, w, gp, gr, r = _inputs(16, 128, seed=12)
    dt = oracle.dx(x, w, gp, gr, r, 128, mode="tf32")
    de = oracle.dx(x, w, gp, gr, r, 128, mode="exact")
    bound = np.abs(gp[:, :24]).astype(np.float64) @ np.abs(w).astype(np.float64)
    bound *= 2.0 ** -10 + 2.0 ** -22
    assert np.all(np.abs(dt - de) <= bound * (1 + 1e-9))
    assert np.any(dt != de)
    wt = oracle.dw(x, gp, mode="tf32")
    we = oracle.dw(x, gp, mode="exact")
    bw = np.abs(gp[:, :24]).astype(np.float64).T @ np.abs(x).astype(np.float64)
    bw *= 2.0 ** -10 + 2.0 ** -22
    assert np.all(np.abs(wt - we) <= bw * (1 + 1e-9))
    assert np.any(wt != we)


def test_brute_force_tiny_with_bit_rounding():
    for T, K in ((1, 8), (2, 16), (3, 24), (5, 40), (7, 8)):
        x, w, gp, gr, r = _inputs(T, K, seed=T * K)
        tf = np.vectorize(lambda v: _tf32_bits_method(float(v)))
        xt, wt, pt = tf(x), tf(w), tf(gp[:, :24])
        dx_ref = np.zeros((T, K))
        dw_ref = np.zeros((24, K))
        for t in range(T):
            c = float(gr[t]) / (float(r[t]) * K)
            for k in range(K):
                s = 0.0
                for j in range(24):
                    s += pt[t, j] * wt[j, k]
                dx_ref[t, k] = s + c * float(x[t, k])
        for j in range(24):
            for k in range(K):
                s = 0.0
                for t in range(T):
                    s += pt[t, j] * xt[t, k]
                dw_ref[j, k] = s
        assert np.array_equal(oracle.dx(x, w, gp, gr, r, K, mode="tf32"), dx_ref)
        assert np.array_equal(oracle.dw(x, gp, mode="tf32"), dw_ref)
