"""MI355X (gfx950) DSv4.1 mHC projection/RMS backward.

A thin ctypes binding over the C-ABI of ``libmhcpb.so`` (declared in
``include/mhcpb.h``), with the same function names.  Every step of the stage
runs in the library's HIP kernels; this module only marshals arguments.  If the
library has not been built, importing this package raises: there is no other
implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import os

try:
    # When PyTorch is present, load its HIP runtime first so that this
    # library binds to the same libamdhip64 instance as torch's allocations.
    import torch  # noqa: F401
except ImportError:  # the library itself does not need torch
    torch = None

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmhcpb.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python rms_backward_amd/build.py` "
        "(hipcc, gfx950) before using rms_backward_amd")

_lib = ctypes.CDLL(LIB_PATH)

MHCPB_SUCCESS = 0
MHCPB_ERROR_INVALID_ARGUMENT = 1
MHCPB_ERROR_UNSUPPORTED = 2
MHCPB_ERROR_MISALIGNED = 3
MHCPB_ERROR_OVERLAP = 4
MHCPB_ERROR_WORKSPACE = 5
MHCPB_ERROR_LAUNCH = 6

EXPORTED = (
    "mhcpb_plan_create", "mhcpb_plan_destroy", "mhcpb_workspace_bytes",
    "mhcpb_plan_split_count", "mhcpb_plan_partial_slabs", "mhcpb_execute",
    "mhcpb_execute_with_events",
    "mhcpb_execute_noalloc", "mhcpb_execute_dx", "mhcpb_execute_dw", "mhcpb_status_string",
    "mhcpb_forward_workspace_bytes", "mhcpb_forward", "mhcpb_forward_with_events",
    "mhcpb_rmsnorm_backward_workspace_bytes", "mhcpb_rmsnorm_backward",
    "mhcpb_rmsnorm_backward_with_events",
)

MHCPB_DTYPE_BF16 = 0
MHCPB_DTYPE_F32 = 1

_vp = ctypes.c_void_p
_lib.mhcpb_plan_create.argtypes = [ctypes.POINTER(_vp), ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_int32]
_lib.mhcpb_plan_create.restype = ctypes.c_int
_lib.mhcpb_plan_destroy.argtypes = [_vp]
_lib.mhcpb_plan_destroy.restype = ctypes.c_int
_lib.mhcpb_workspace_bytes.argtypes = [_vp, ctypes.POINTER(ctypes.c_size_t)]
_lib.mhcpb_workspace_bytes.restype = ctypes.c_int
_lib.mhcpb_plan_split_count.argtypes = [_vp, ctypes.POINTER(ctypes.c_int32)]
_lib.mhcpb_plan_split_count.restype = ctypes.c_int
_lib.mhcpb_plan_partial_slabs.argtypes = [_vp, ctypes.POINTER(ctypes.c_int32)]
_lib.mhcpb_plan_partial_slabs.restype = ctypes.c_int
_EXEC_ARGS = [_vp] * 10 + [ctypes.c_size_t, _vp]
_lib.mhcpb_execute.argtypes = _EXEC_ARGS
_lib.mhcpb_execute.restype = ctypes.c_int
_lib.mhcpb_execute_with_events.argtypes = _EXEC_ARGS + [_vp, _vp, _vp]
_lib.mhcpb_execute_with_events.restype = ctypes.c_int
_lib.mhcpb_execute_noalloc.argtypes = [_vp] * 10
_lib.mhcpb_execute_noalloc.restype = ctypes.c_int
_lib.mhcpb_execute_dx.argtypes = [_vp] * 8 + [_vp]
_lib.mhcpb_execute_dx.restype = ctypes.c_int
_lib.mhcpb_execute_dw.argtypes = [_vp] * 5 + [ctypes.c_size_t, _vp]
_lib.mhcpb_execute_dw.restype = ctypes.c_int
_lib.mhcpb_forward_workspace_bytes.argtypes = [_vp, ctypes.POINTER(ctypes.c_size_t)]
_lib.mhcpb_forward_workspace_bytes.restype = ctypes.c_int
_FWD_ARGS = [_vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.mhcpb_forward.argtypes = _FWD_ARGS
_lib.mhcpb_forward.restype = ctypes.c_int
_lib.mhcpb_forward_with_events.argtypes = _FWD_ARGS + [_vp, _vp, _vp]
_lib.mhcpb_forward_with_events.restype = ctypes.c_int
_lib.mhcpb_rmsnorm_backward_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32,
                                                        ctypes.POINTER(ctypes.c_size_t)]
_lib.mhcpb_rmsnorm_backward_workspace_bytes.restype = ctypes.c_int
_RMS_ARGS = [ctypes.c_int64, ctypes.c_int32, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
             _vp, ctypes.c_size_t, _vp]
_lib.mhcpb_rmsnorm_backward.argtypes = _RMS_ARGS
_lib.mhcpb_rmsnorm_backward.restype = ctypes.c_int
_lib.mhcpb_rmsnorm_backward_with_events.argtypes = _RMS_ARGS + [_vp, _vp, _vp]
_lib.mhcpb_rmsnorm_backward_with_events.restype = ctypes.c_int
_lib.mhcpb_status_string.argtypes = [ctypes.c_int]
_lib.mhcpb_status_string.restype = ctypes.c_char_p


class MhcpbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mhcpb_status_string(status)} (status {status})")


def mhcpb_status_string(status: int) -> str:
    return _lib.mhcpb_status_string(int(status)).decode()


def _ptr(t) -> int | None:
    """Device address of a tensor (torch) or an int address; None stays NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def mhcpb_plan_create(T: int, streams: int, hidden: int) -> int:
    """Create a plan; returns its opaque handle.  Raises MhcpbError on error."""
    h = _vp()
    st = _lib.mhcpb_plan_create(ctypes.byref(h), int(T), int(streams), int(hidden))
    if st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_plan_create")
    return h.value


def mhcpb_plan_create_status(T: int, streams: int, hidden: int) -> tuple[int, int | None]:
    """(status, handle-or-None) without raising, for argument-check tests."""
    h = _vp()
    st = _lib.mhcpb_plan_create(ctypes.byref(h), int(T), int(streams), int(hidden))
    return st, h.value


def mhcpb_plan_destroy(plan: int | None) -> None:
    _lib.mhcpb_plan_destroy(plan)


def mhcpb_workspace_bytes(plan: int) -> int:
    n = ctypes.c_size_t()
    st = _lib.mhcpb_workspace_bytes(plan, ctypes.byref(n))
    if st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_workspace_bytes")
    return n.value


def mhcpb_plan_split_count(plan: int) -> int:
    n = ctypes.c_int32()
    st = _lib.mhcpb_plan_split_count(plan, ctypes.byref(n))
    if st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_plan_split_count")
    return n.value


def mhcpb_plan_partial_slabs(plan: int) -> int:
    n = ctypes.c_int32()
    st = _lib.mhcpb_plan_partial_slabs(plan, ctypes.byref(n))
    if st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_plan_partial_slabs")
    return n.value


def mhcpb_execute(plan, x, w, grad_proj, grad_r, r, dx, dw, grad_x_addend, workspace,
                  workspace_size: int, stream: int = 0, check: bool = True) -> int:
    """Enqueue the stage.  Tensors are passed by device address (torch tensors
    or ints); ``stream`` is a raw hipStream_t (0 = null stream).  Returns the
    status; raises MhcpbError on a non-zero status when ``check`` is set."""
    st = _lib.mhcpb_execute(plan, _ptr(x), _ptr(w), _ptr(grad_proj), _ptr(grad_r), _ptr(r),
                            _ptr(dx), _ptr(dw), _ptr(grad_x_addend), _ptr(workspace),
                            int(workspace_size), stream)
    if check and st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_execute")
    return st


def mhcpb_execute_with_events(plan, x, w, grad_proj, grad_r, r, dx, dw, grad_x_addend,
                              workspace, workspace_size: int, stream: int,
                              before_k1: int | None, after_k1: int | None,
                              after_k2: int | None, check: bool = True) -> int:
    """mhcpb_execute that also attaches three caller-owned hipEvent_t handles
    to the kernel dispatches (start and end of kernel 1, end of kernel 2)."""
    st = _lib.mhcpb_execute_with_events(
        plan, _ptr(x), _ptr(w), _ptr(grad_proj), _ptr(grad_r), _ptr(r), _ptr(dx), _ptr(dw),
        _ptr(grad_x_addend), _ptr(workspace), int(workspace_size), stream,
        before_k1, after_k1, after_k2)
    if check and st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_execute_with_events")
    return st


def mhcpb_execute_noalloc(plan, x, w, grad_proj, grad_r, r, dx, dw, grad_x_addend,
                          stream: int = 0, check: bool = True) -> int:
    """mhcpb_execute with the library's static per-GPU workspace (64 MiB) in
    place of a caller workspace: allocates nothing.  Calls that overlap on one
    GPU race on that workspace."""
    st = _lib.mhcpb_execute_noalloc(plan, _ptr(x), _ptr(w), _ptr(grad_proj), _ptr(grad_r),
                                    _ptr(r), _ptr(dx), _ptr(dw), _ptr(grad_x_addend), stream)
    if check and st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_execute_noalloc")
    return st


def mhcpb_execute_dx(plan, x, w, grad_proj, grad_r, r, dx, grad_x_addend, stream: int = 0,
                     check: bool = True) -> int:
    """The split form that writes dX only (one kernel, no workspace)."""
    st = _lib.mhcpb_execute_dx(plan, _ptr(x), _ptr(w), _ptr(grad_proj), _ptr(grad_r), _ptr(r),
                               _ptr(dx), _ptr(grad_x_addend), stream)
    if check and st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_execute_dx")
    return st


def mhcpb_execute_dw(plan, x, grad_proj, dw, workspace, workspace_size: int, stream: int = 0,
                     check: bool = True) -> int:
    """The split form that writes dW only (partial slabs, then the reduce)."""
    st = _lib.mhcpb_execute_dw(plan, _ptr(x), _ptr(grad_proj), _ptr(dw), _ptr(workspace),
                               int(workspace_size), stream)
    if check and st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_execute_dw")
    return st


def mhcpb_forward_workspace_bytes(plan: int) -> int:
    n = ctypes.c_size_t()
    st = _lib.mhcpb_forward_workspace_bytes(plan, ctypes.byref(n))
    if st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_forward_workspace_bytes")
    return n.value


def mhcpb_forward(plan, x, w, eps: float, proj, r, workspace, workspace_size: int,
                  stream: int = 0, check: bool = True) -> int:
    """Enqueue the forward map (pass over X, then the sum of the tiles)."""
    st = _lib.mhcpb_forward(plan, _ptr(x), _ptr(w), float(eps), _ptr(proj), _ptr(r),
                            _ptr(workspace), int(workspace_size), stream)
    if check and st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_forward")
    return st


def mhcpb_forward_with_events(plan, x, w, eps: float, proj, r, workspace, workspace_size: int,
                              stream: int, before_k1: int | None, after_k1: int | None,
                              after_k2: int | None, check: bool = True) -> int:
    """mhcpb_forward with caller-owned hipEvent_t handles on the dispatches
    (start and end of kernel 1, end of kernel 2)."""
    st = _lib.mhcpb_forward_with_events(plan, _ptr(x), _ptr(w), float(eps), _ptr(proj),
                                        _ptr(r), _ptr(workspace), int(workspace_size), stream,
                                        before_k1, after_k1, after_k2)
    if check and st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_forward_with_events")
    return st


def mhcpb_rmsnorm_backward_workspace_bytes(T: int, H: int, check: bool = True):
    """Workspace bytes of the RMSNorm backward for T rows of width H; with
    ``check`` False returns (status, bytes) instead of raising."""
    n = ctypes.c_size_t()
    st = _lib.mhcpb_rmsnorm_backward_workspace_bytes(int(T), int(H), ctypes.byref(n))
    if not check:
        return st, n.value
    if st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_rmsnorm_backward_workspace_bytes")
    return n.value


def mhcpb_rmsnorm_backward(T: int, H: int, g, x, w, w_dtype: int, rstd, g_residual, dx, dw,
                           workspace, workspace_size: int, stream: int = 0,
                           check: bool = True) -> int:
    """Enqueue the BF16 RMSNorm backward (dx BF16, dw FP32).  BF16 tensors are
    passed by device address (torch bfloat16 or int16 tensors, or ints)."""
    st = _lib.mhcpb_rmsnorm_backward(int(T), int(H), _ptr(g), _ptr(x), _ptr(w), int(w_dtype),
                                     _ptr(rstd), _ptr(g_residual), _ptr(dx), _ptr(dw),
                                     _ptr(workspace), int(workspace_size), stream)
    if check and st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_rmsnorm_backward")
    return st


def mhcpb_rmsnorm_backward_with_events(T: int, H: int, g, x, w, w_dtype: int, rstd, g_residual,
                                       dx, dw, workspace, workspace_size: int, stream: int,
                                       before_k1: int | None, after_k1: int | None,
                                       after_k2: int | None, check: bool = True) -> int:
    """mhcpb_rmsnorm_backward with caller-owned hipEvent_t handles on the
    dispatches (start and end of kernel 1, end of kernel 2)."""
    st = _lib.mhcpb_rmsnorm_backward_with_events(
        int(T), int(H), _ptr(g), _ptr(x), _ptr(w), int(w_dtype), _ptr(rstd), _ptr(g_residual),
        _ptr(dx), _ptr(dw), _ptr(workspace), int(workspace_size), stream, before_k1, after_k1,
        after_k2)
    if check and st != MHCPB_SUCCESS:
        raise MhcpbError(st, "mhcpb_rmsnorm_backward_with_events")
    return st
