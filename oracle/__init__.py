"""ctypes loader for the FP64 CPU oracle in ``mhcpb_oracle.c``.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it; the GPU library never does.  It follows the
formula of the "DSv4.1 mHC projection/RMS backward" cuDNN Frontend page
(introduction):  P = grad_proj[:, :24], dX = P W + grad_r / (r K) X,
dW = P^T X, with TF32 operands in ``mode="tf32"`` and exact FP32 operands in
``mode="exact"``; results are FP64 with no final rounding.  ``forward`` is
the map those are the gradient of: proj = X W^T (24 gate logits, TF32 operands
in ``mode="tf32"``) and r = sqrt(mean(X^2) + eps) per row, the logits and RMS
the "mhc_projection" entry of the prime-kernels pull request 15 page computes
in one read of the streams.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mhcpb_oracle.c")
_LIB = os.path.join(_HERE, "libmhcpb_oracle.so")

_MODES = {"exact": 0, "tf32": 1}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libmhcpb_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i64 = ctypes.c_int64
        lib.oracle_tf32.argtypes = [ctypes.c_float]
        lib.oracle_tf32.restype = ctypes.c_double
        lib.oracle_bf16.argtypes = [ctypes.c_float]
        lib.oracle_bf16.restype = ctypes.c_float
        lib.oracle_dx.argtypes = [ctypes.c_int, i64, i64, i64, f32p, f32p, f32p,
                                  f32p, f32p, u16p, f64p]
        lib.oracle_dx.restype = ctypes.c_int
        lib.oracle_dw.argtypes = [ctypes.c_int, i64, i64, f32p, f32p, f64p]
        lib.oracle_dw.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [ctypes.c_int, i64, i64, f32p, f32p,
                                       ctypes.c_double, f64p, f64p]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_rmsnorm_backward.argtypes = [i64, i64, u16p, u16p, f32p, f32p, u16p, f64p,
                                                f64p]
        lib.oracle_rmsnorm_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def tf32(v: float) -> float:
    """TF32 value (round-to-nearest-even of the fraction to 10 bits)."""
    return _load().oracle_tf32(float(np.float32(v)))


def tf32_array(a) -> np.ndarray:
    """Elementwise TF32 values of an FP32 array, as float64."""
    lib = _load()
    flat = np.ascontiguousarray(a, dtype=np.float32).ravel()
    out = np.array([lib.oracle_tf32(float(v)) for v in flat], dtype=np.float64)
    return out.reshape(np.shape(a))


def bf16(v: float) -> np.float32:
    """BF16 value (round to nearest even) of an FP32 value, as float32."""
    return np.float32(_load().oracle_bf16(float(np.float32(v))))


def bf16_bits(v: float) -> int:
    """The 16 BF16 bits of ``bf16(v)``."""
    return int(np.array([bf16(v)], dtype=np.float32).view(np.uint32)[0] >> 16)


def dx(x, w, grad_proj, grad_r, r, K: int, addend=None, mode: str = "tf32"):
    """dX in FP64 for the rows and columns given.

    x [rows, cols] FP32, w [24, cols] FP32 (the same columns), grad_proj
    [rows, 32] FP32 (columns 24..31 are never read), grad_r and r [rows],
    addend [rows, cols] as BF16 bits (uint16) or None; K is the full row
    width used in grad_r / (r K).
    """
    lib = _load()
    x, xp = _f32(x)
    rows, cols = x.shape
    w, wp = _f32(w)
    gp, gpp = _f32(grad_proj)
    gr, grp = _f32(grad_r)
    rr, rp = _f32(r)
    assert w.shape == (24, cols) and gp.shape == (rows, 32)
    assert gr.shape == (rows,) and rr.shape == (rows,)
    ap = None
    if addend is not None:
        addend = np.ascontiguousarray(addend, dtype=np.uint16)
        assert addend.shape == (rows, cols)
        ap = addend.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))
    out = np.empty((rows, cols), dtype=np.float64)
    rc = lib.oracle_dx(_MODES[mode], rows, cols, int(K), xp, wp, gpp, grp, rp, ap,
                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError("oracle_dx rejected its arguments")
    return out


def dw(x, grad_proj, mode: str = "tf32"):
    """dW [24, cols] in FP64, summed over every row of x [rows, cols]."""
    lib = _load()
    x, xp = _f32(x)
    rows, cols = x.shape
    gp, gpp = _f32(grad_proj)
    assert gp.shape == (rows, 32)
    out = np.empty((24, cols), dtype=np.float64)
    rc = lib.oracle_dw(_MODES[mode], rows, cols, xp, gpp,
                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError("oracle_dw rejected its arguments")
    return out


def backward(x, w, grad_proj, grad_r, r, addend=None, mode: str = "tf32"):
    """(dX, dW) in FP64 over a whole [T, K] problem."""
    K = np.shape(x)[1]
    return (dx(x, w, grad_proj, grad_r, r, K, addend=addend, mode=mode),
            dw(x, grad_proj, mode=mode))


def forward(x, w, eps: float = 1e-6, mode: str = "tf32"):
    """(proj [rows, 24], r [rows]) in FP64 for x [rows, K] and w [24, K].

    ``eps`` is taken as given (pass the FP32 value a GPU call uses, widened).
    """
    lib = _load()
    x, xp = _f32(x)
    rows, K = x.shape
    w, wp = _f32(w)
    assert w.shape == (24, K)
    proj = np.empty((rows, 24), dtype=np.float64)
    r = np.empty((rows,), dtype=np.float64)
    rc = lib.oracle_forward(_MODES[mode], rows, K, xp, wp, float(eps),
                            proj.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                            r.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError("oracle_forward rejected its arguments")
    return proj, r


def rmsnorm_backward(g_bits, x_bits, w, rstd, res_bits=None):
    """(dx [rows, H], dw [H]) in FP64 for the BF16 RMSNorm backward: g, x and
    res as BF16 bit patterns (uint16), w the weight's values (FP32 array;
    BF16 weights widened), rstd [rows] FP32 from the forward."""
    lib = _load()
    g_bits = np.ascontiguousarray(g_bits, dtype=np.uint16)
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, H = x_bits.shape
    assert g_bits.shape == (rows, H)
    w, wp = _f32(w)
    rs, rsp = _f32(rstd)
    assert w.shape == (H,) and rs.shape == (rows,)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    rp = None
    if res_bits is not None:
        res_bits = np.ascontiguousarray(res_bits, dtype=np.uint16)
        assert res_bits.shape == (rows, H)
        rp = res_bits.ctypes.data_as(u16p)
    dx = np.empty((rows, H), dtype=np.float64)
    dw = np.empty((H,), dtype=np.float64)
    rc = lib.oracle_rmsnorm_backward(rows, H, g_bits.ctypes.data_as(u16p),
                                     x_bits.ctypes.data_as(u16p), wp, rsp, rp,
                                     dx.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                     dw.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError("oracle_rmsnorm_backward rejected its arguments")
    return dx, dw
