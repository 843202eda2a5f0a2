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
