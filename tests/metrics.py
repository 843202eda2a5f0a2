"""Error metrics used to compare the GPU result with the FP64 oracle.

Bounds (stated for this stage's outputs):
* dX: relative Frobenius error <= 4e-3 against both oracle modes, and per
  element |gpu - ref_tf32| <= 2 ulp_bf16(ref) + 1e-4 max|ref|;
* dW: relative Frobenius error <= 2e-3 against both oracle modes.
The per-element dX bound is applied against the TF32-mode oracle, because the
page defines the products on TF32 operands ("DSv4.1 mHC projection/RMS
backward", introduction).
"""
import numpy as np

DX_FROB = 4e-3
DW_FROB = 2e-3


def ulp_bf16(v):
    """2^(floor(log2|v|) - 7), floored at 2^-133 (the BF16 subnormal quantum)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    u = np.exp2(e - 7)
    return np.where(a > 0, np.maximum(u, 2.0 ** -133), 2.0 ** -133)


def rel_frobenius(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return float(num / den) if den > 0 else float(num)


def dx_violations(got, ref, max_abs_ref=None):
    """Indices where |got - ref| > 2 ulp_bf16(ref) + 1e-4 max|ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.abs(ref).max() if max_abs_ref is None else max_abs_ref
    bound = 2.0 * ulp_bf16(ref) + 1e-4 * m
    bad = ~(np.abs(got - ref) <= bound)
    return np.argwhere(bad)


def bf16_bits_to_f64(bits):
    """uint16/int16 BF16 bit patterns to float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


TINY = 2.0 ** -126  # the smallest normal FP32 (and BF16) number


def flush_bound(abs_a, abs_b, n_products):
    """Bound of what the matrix-unit products may lose against the oracle
    below the normal range (a known departure): the BF16 matrix units read
    subnormal inputs as zero, so a TF32 operand split into BF16 high and low
    parts loses any part below 2^-126, and a partial product or partial sum
    below 2^-126 may be lost as well.  Per product a * b that is at most
    2^-126 (|a| + |b| + 5); abs_a and abs_b bound |a| and |b| summed over the
    products (or elementwise, with n_products the product count)."""
    return TINY * (np.asarray(abs_a, dtype=np.float64) + np.asarray(abs_b, dtype=np.float64)
                   + 5.0 * n_products)


def dw_accumulation_bound(abs_sum, rows_per_slab, splits):
    """Worst-case FP32 summation error of the slab-then-fixed-order scheme:
    at most (rows_per_slab + splits + 64) roundings of 2^-24, each bounded by
    the sum of |products|.  Exact TF32 products are assumed."""
    return (rows_per_slab + splits + 64) * 2.0 ** -24 * np.asarray(abs_sum, dtype=np.float64)


# ---- forward map (proj = X W^T with TF32 operands, r = RMS) ----------------
# The GPU adds exact products in FP32 along chains of a few thousand
# additions, whose rounding errors grow like 2^-24 sqrt(n) relative to the
# partial sums: about 1e-6 of a logit at K = 20480.  The bounds below sit a
# decade or more above that and a decade below what a dropped BF16 low part
# (about 1e-3) or skipped TF32 rounding (about 3e-4) would give.
FWD_PROJ_FROB = 1e-5
FWD_PROJ_ROW = 1e-4
FWD_PROJ_ELEM = 1e-4


def fwd_r_rel_bound(K):
    """Worst-case relative error of r: the FP32 sum of K positive squares in
    chains of at most K/4 + 64 additions (relative error <= n 2^-24), halved
    by the square root, plus one rounding each for the division by K, eps
    and the square root."""
    u = 2.0 ** -24
    return (K / 4 + 64) * u / 2 + 3 * u


# ---- BF16 RMSNorm backward ---------------------------------------------------
U32 = 2.0 ** -24


def rms_dx_fp32_error(g, x, w, rstd, res, H):
    """Worst-case error of the FP32 value the GPU rounds to BF16, per element.

    c1 = sum_h w g x / H is summed with fused multiply-adds over at most 96
    terms per lane and a 6-level tree across 64 lanes (<= 103 roundings), then
    divided by H and multiplied by rstd three times (4 roundings); the value
    rstd w g - k x takes three roundings and the residual one more."""
    g, x, w = (np.asarray(a, dtype=np.float64) for a in (g, x, w))
    rs = np.asarray(rstd, dtype=np.float64)[:, None]
    a_row = np.abs(w[None, :] * g * x).sum(axis=1, keepdims=True)
    k_abs = rs ** 3 * a_row / H
    val = np.abs(rs * w[None, :] * g) + k_abs * np.abs(x)
    if res is not None:
        val = val + np.abs(np.asarray(res, dtype=np.float64))
    return U32 * (3.0 * val) + 110.0 * U32 * k_abs * np.abs(x)


def rms_dx_violations(got, ref, fp32_err):
    """Indices where |got - ref| > half a BF16 ulp of |ref| + err, plus twice
    err (the rounded value can sit one BF16 step away only when ref is within
    err of a rounding boundary)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = 0.5 * ulp_bf16(np.abs(ref) + fp32_err) + 2.0 * fp32_err
    return np.argwhere(~(np.abs(got - ref) <= bound))


def rms_dw_bound(abs_sum, T, S):
    """Worst-case FP32 error of dw: a block's rows in sequence (at most
    ceil(T / S) fused multiply-adds per column), then ceil(S / 16) block
    partials per group and 16 groups, each step one rounding bounded by the
    sum of |g x rstd|."""
    depth = -(-T // S) + (-(-S // 16)) + 16 + 2
    return depth * U32 * np.asarray(abs_sum, dtype=np.float64)


def rms_schedule(T, H):
    """Blocks S of the RMSNorm backward: min(ceil(T / 16), 256 P) with
    P = max(1, 12 // ceil(H / 512)) (rows dealt round-robin)."""
    if T == 0:
        return 0
    nc = -(-H // 512)
    per = max(1, 12 // nc)
    return min(-(-T // 16), 256 * per)


def bf16_round_f64(v):
    """FP64 values rounded once to the nearest BF16 (ties to even), as FP64:
    8 significant bits, quantum at least 2^-133, beyond the range +-inf."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(v / q) * q
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
