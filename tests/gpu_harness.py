"""Helpers that run the stage on the GPU through the C-ABI and fetch samples
for the oracle.  Used only by tests marked ``gpu``."""
import numpy as np
import torch

from rms_backward_amd.wrapper import Plan

PROJ_COLS = 24


def to_device(inp, device):
    return {k: (v.to(device) if v is not None else None) for k, v in inp.items()}


def alloc_outputs(T, K, plan, device, poison=True):
    dx = torch.empty(T, K, dtype=torch.bfloat16, device=device)
    dw = torch.empty(PROJ_COLS, K, dtype=torch.float32, device=device)
    ws = plan.alloc_workspace(device)
    if poison:
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
        ws.fill_(0xFF)  # all-ones FP32 words are NaN
    return dx, dw, ws


def run(inp, plan=None, poison=True, outputs=None, sync=True):
    """Execute once on the current stream; returns (dx, dw, ws, plan)."""
    x = inp["x"]
    T, K = x.shape
    if plan is None:
        plan = Plan(T, 4, K // 4)
    if outputs is None:
        outputs = alloc_outputs(T, K, plan, x.device, poison)
    dx, dw, ws = outputs
    plan.execute(x, inp["w"], inp["grad_proj"], inp["grad_r"], inp["r"], dx, dw, ws,
                 inp.get("addend"))
    if sync:
        torch.cuda.synchronize()
    return dx, dw, ws, plan


def host(t):
    return t.detach().cpu().numpy()


def bf16_bits_np(t):
    """BF16 tensor -> numpy uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_rows(inp, rows):
    """Oracle inputs for a subset of rows and every column."""
    idx = torch.as_tensor(rows, device=inp["x"].device, dtype=torch.long)
    out = dict(x=host(inp["x"].index_select(0, idx)), w=host(inp["w"]),
               grad_proj=host(inp["grad_proj"].index_select(0, idx)),
               grad_r=host(inp["grad_r"].index_select(0, idx)),
               r=host(inp["r"].index_select(0, idx)), addend=None)
    if inp.get("addend") is not None:
        out["addend"] = bf16_bits_np(inp["addend"].index_select(0, idx))
    return out


def host_cols(inp, cols):
    """Oracle inputs for dW on a subset of columns over every row."""
    idx = torch.as_tensor(cols, device=inp["x"].device, dtype=torch.long)
    return dict(x=host(inp["x"].index_select(1, idx)), grad_proj=host(inp["grad_proj"]))


def sample_rows(T, L, rng, extra=24):
    """First, last, slab-boundary and random rows."""
    rows = {0, 1, T - 1, max(0, T - 2)}
    for b in range(L, T, L):
        rows.update({b - 1, b, min(T - 1, b + 1)})
    rows.update(int(v) for v in rng.integers(0, T, size=extra))
    rows = sorted(r for r in rows if 0 <= r < T)
    return rows


def sample_cols(K, rng, extra=24, tile=256, whole_first=0):
    """Edge columns, tile boundaries, random columns, and optionally every
    column of [0, whole_first), interleaved so that any prefix of the list
    mixes the whole block with the scattered columns."""
    head = list(range(min(whole_first, K)))
    cols = {0, 1, 2, 3, K - 4, K - 3, K - 2, K - 1}
    for b in (tile, 2 * tile, K // 2, K - tile):
        for d in (-4, -1, 0, 1, 4):
            if 0 <= b + d < K:
                cols.add(b + d)
    cols.update(int(v) for v in rng.integers(0, K, size=extra))
    rest = sorted(c for c in cols if c >= len(head))
    # keep a spread of columns (not only the head block) among the first ones
    return [v for pair in zip(rest, head) for v in pair] + rest[len(head):] + head[len(rest):]


def run_forward(x, w, eps=1e-6, plan=None, sync=True):
    """Forward map once on the current stream over NaN-filled outputs and a
    NaN-filled workspace; returns (proj [T, 32], r [T], plan)."""
    T, K = x.shape
    if plan is None:
        plan = Plan(T, 4, K // 4)
    proj = torch.full((T, 32), float("nan"), dtype=torch.float32, device=x.device)
    r = torch.full((T,), float("nan"), dtype=torch.float32, device=x.device)
    ws = plan.alloc_forward_workspace(x.device)
    ws.fill_(0xFF)
    plan.forward(x, w, eps, proj, r, ws)
    if sync:
        torch.cuda.synchronize()
    return proj, r, plan


def run_rmsnorm(inp, poison=True, sync=True, workspace=None):
    """RMSNorm backward once on the current stream; returns (dx, dw)."""
    from rms_backward_amd.wrapper import rmsnorm_backward
    x = inp["x"]
    T, H = x.shape
    dx = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    dw = torch.empty(H, dtype=torch.float32, device=x.device)
    if poison:
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
    rmsnorm_backward(inp["g"], x, inp["w"], inp["rstd"], inp.get("res"), workspace=workspace,
                     dx=dx, dw=dw)
    if sync:
        torch.cuda.synchronize()
    return dx, dw


def rms_oracle(inp, rows=None):
    """Oracle (dx [rows, H], dw [H] over the given rows) from device inputs."""
    import oracle
    sel = (lambda t: t) if rows is None else (lambda t: t[rows])
    g = bf16_bits_np(sel(inp["g"]))
    x = bf16_bits_np(sel(inp["x"]))
    w = inp["w"].float().cpu().numpy()
    rstd = host(sel(inp["rstd"]))
    res = bf16_bits_np(sel(inp["res"])) if inp.get("res") is not None else None
    return oracle.rmsnorm_backward(g, x, w, rstd, res_bits=res)
