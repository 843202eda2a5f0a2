"""Allocating convenience call over the C-ABI, for PyTorch callers.

Mirrors the page's allocating wrapper ("DSv4.1 mHC projection/RMS backward",
"Allocating wrapper" section): it allocates dX, dW and the workspace with torch
on the tensors' device, enqueues the stage on the current (or given) stream and
returns (dx, dw).  The caller orders streams and keeps tensors alive.  All
arithmetic happens in the library's kernels.
"""
from __future__ import annotations

import torch

from . import (MHCPB_DTYPE_BF16, MHCPB_DTYPE_F32, mhcpb_execute, mhcpb_forward,
               mhcpb_forward_workspace_bytes, mhcpb_plan_create, mhcpb_plan_destroy,
               mhcpb_rmsnorm_backward, mhcpb_rmsnorm_backward_workspace_bytes,
               mhcpb_workspace_bytes)

PROJ_COLS = 24


class Plan:
    """Owns a plan handle for one (T, streams, hidden)."""

    def __init__(self, T: int, streams: int, hidden: int):
        self.T, self.streams, self.hidden = int(T), int(streams), int(hidden)
        self.K = self.streams * self.hidden
        self.handle = mhcpb_plan_create(self.T, self.streams, self.hidden)
        self.workspace_bytes = mhcpb_workspace_bytes(self.handle)
        self.forward_workspace_bytes = mhcpb_forward_workspace_bytes(self.handle)

    def close(self):
        if self.handle:
            mhcpb_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_workspace(self, device) -> torch.Tensor:
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=device)

    def alloc_forward_workspace(self, device) -> torch.Tensor:
        return torch.empty(self.forward_workspace_bytes, dtype=torch.uint8, device=device)

    def forward(self, x, w, eps, proj, r, workspace, stream=None):
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        return mhcpb_forward(self.handle, x, w, eps, proj, r, workspace, workspace.numel(),
                             s.cuda_stream)

    def execute(self, x, w, grad_proj, grad_r, r, dx, dw, workspace,
                grad_x_addend=None, stream=None):
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        return mhcpb_execute(self.handle, x, w, grad_proj, grad_r, r, dx, dw,
                             grad_x_addend, workspace, workspace.numel(), s.cuda_stream)


def mhc_projection_backward(x, w, grad_proj, grad_r, r, grad_x_addend=None, stream=None):
    """Allocate outputs and workspace, run the stage, return (dx, dw).

    dx is BF16 [T, K], dw is FP32 [24, K].
    """
    T, K = x.shape
    assert K % 4 == 0
    plan = Plan(T, 4, K // 4)
    dx = torch.empty(T, K, dtype=torch.bfloat16, device=x.device)
    dw = torch.empty(PROJ_COLS, K, dtype=torch.float32, device=x.device)
    ws = plan.alloc_workspace(x.device)
    plan.execute(x, w, grad_proj, grad_r, r, dx, dw, ws, grad_x_addend, stream)
    return dx, dw


def mhc_projection_forward(x, w, eps: float = 1e-6, stream=None):
    """Allocate outputs and workspace, run the forward map, return (proj, r).

    proj is FP32 [T, 32] (logits in columns 0..23, zeros in 24..31), r is
    FP32 [T]; the workspace holds the per-tile partials.
    """
    T, K = x.shape
    assert K % 4 == 0
    plan = Plan(T, 4, K // 4)
    proj = torch.empty(T, 32, dtype=torch.float32, device=x.device)
    r = torch.empty(T, dtype=torch.float32, device=x.device)
    ws = plan.alloc_forward_workspace(x.device)
    plan.forward(x, w, eps, proj, r, ws, stream)
    return proj, r


def rmsnorm_backward(g, x, w, rstd, g_residual=None, workspace=None, dx=None, dw=None,
                     stream=None):
    """The deterministic BF16 RMSNorm backward: returns (dx, dw), dx BF16 of
    x's shape [T, H], dw FP32 [H].  g, x (and g_residual) are compact BF16
    [T, H]; w is BF16 or FP32 [H]; rstd FP32 [T].  Outputs and the workspace
    are allocated when not given."""
    T, H = x.shape
    dev = x.device
    if w.dtype == torch.float32:
        wd = MHCPB_DTYPE_F32
    elif w.dtype == torch.bfloat16:
        wd = MHCPB_DTYPE_BF16
    else:
        raise TypeError(f"w must be bfloat16 or float32, got {w.dtype}")
    if dx is None:
        dx = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    if dw is None:
        dw = torch.empty(H, dtype=torch.float32, device=dev)
    if workspace is None:
        nbytes = mhcpb_rmsnorm_backward_workspace_bytes(T, H)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    mhcpb_rmsnorm_backward(T, H, g, x, w, wd, rstd, g_residual, dx, dw, workspace,
                           workspace.numel(), s.cuda_stream)
    return dx, dw
