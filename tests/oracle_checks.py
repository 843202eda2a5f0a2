"""Comparisons of GPU outputs with the FP64 oracle, shared by the GPU parity
tests (test infrastructure; the bounds are stated in tests/metrics.py).

check_dx: dX rows against both oracle modes (relative Frobenius) and, per
element, within 2 BF16 ulps + 1e-4 max|ref| of the TF32-mode oracle.
check_dw: dW columns per element within the worst-case FP32 summation bound of
the TF32-mode oracle, and relative Frobenius against both modes.
"""
import numpy as np

import oracle
from tests import metrics as mt


def check_dx(got_bits, inp_h, K, label, full_ref_max=None):
    got = mt.bf16_bits_to_f64(got_bits)
    ref_t = oracle.dx(inp_h["x"], inp_h["w"], inp_h["grad_proj"], inp_h["grad_r"],
                      inp_h["r"], K, addend=inp_h["addend"], mode="tf32")
    ref_e = oracle.dx(inp_h["x"], inp_h["w"], inp_h["grad_proj"], inp_h["grad_r"],
                      inp_h["r"], K, addend=inp_h["addend"], mode="exact")
    assert np.all(np.isfinite(got)), f"{label}: non-finite dX"
    f_t = mt.rel_frobenius(got, ref_t)
    f_e = mt.rel_frobenius(got, ref_e)
    bad = mt.dx_violations(got, ref_t, full_ref_max)
    print(f"{label}: dX frob tf32 {f_t:.3e} exact {f_e:.3e} violations {len(bad)}")
    assert f_t <= mt.DX_FROB and f_e <= mt.DX_FROB, label
    assert len(bad) == 0, f"{label}: first violations {bad[:5].tolist()}"


def check_dw(got, inp_c, rows_per_slab, splits, label, exact_cols=None):
    """Per element against the TF32-mode oracle (worst-case FP32 summation
    bound) on every given column; relative Frobenius against both modes (the
    exact mode on at most `exact_cols` of them, to bound the oracle's time)."""
    ref_t = oracle.dw(inp_c["x"], inp_c["grad_proj"], mode="tf32")
    assert np.all(np.isfinite(got)), f"{label}: non-finite dW"
    f_t = mt.rel_frobenius(got, ref_t)
    sel = slice(None) if exact_cols is None else slice(0, exact_cols)
    ref_e = oracle.dw(inp_c["x"][:, sel], inp_c["grad_proj"], mode="exact")
    f_e = mt.rel_frobenius(got[:, sel], ref_e)
    gp_abs = np.abs(inp_c["grad_proj"])
    gp_abs[:, 24:] = 0.0
    abs_sum = oracle.dw(np.abs(inp_c["x"]), gp_abs, mode="tf32")
    bound = mt.dw_accumulation_bound(abs_sum, rows_per_slab, splits)
    err = np.abs(got - ref_t)
    print(f"{label}: dW frob tf32 {f_t:.3e} exact {f_e:.3e} "
          f"max err/bound {float((err / np.maximum(bound, 1e-300)).max()):.3e} "
          f"({got.shape[1]} columns)")
    assert f_t <= mt.DW_FROB and f_e <= mt.DW_FROB, label
    assert np.all(err <= bound), label
