"""Seeded synthetic inputs for the DSv4.1 mHC projection/RMS backward.

This module only draws inputs; it holds none of the backward's arithmetic.
Both the GPU path (through the C-ABI) and the CPU oracle consume what it makes.

Shapes and distributions (the stage's supported training profile is 4 streams
x hidden 5120 x 4096 tokens, "DSv4.1 mHC projection/RMS backward" page,
introduction; the other sizes widen that profile):

  X          FP32 [T, K], K = streams * hidden, N(0, 1)
  W          FP32 [24, K], N(0, 0.02)  (0.02 is the standard deviation)
  grad_proj  FP32 [T, 32], columns 0..23 N(0, 0.01); columns 24..31 hold
             garbage (NaN in even columns, 1e30 in odd ones): the page says
             they are ignored even if nonzero
  grad_r     FP32 [T], N(0, 0.01)
  r          FP32 [T], sqrt(mean(X^2, row) + 1e-6) computed in FP64 (the
             positive forward RMS the page asks for)
  addend     BF16 [T, K], N(0, 0.01) (the fused stream gradient,
             prime-kernels pull request 15), only where a workload has one
  rescale    where a workload asks for it, each X row is multiplied by
             10^U(-2, 2) before r is computed, which stresses grad_r / (r K)

Random numbers come from torch generators seeded per workload; a generator on
the GPU draws different numbers from one on the CPU, so a test draws on one
device and copies to the other.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

PROJ_COLS = 24
PROJ_STRIDE = 32
SEED_BASE = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    streams: int
    hidden: int
    seed: int
    addend: bool = False
    rescale_rows: bool = False

    @property
    def K(self) -> int:
        return self.streams * self.hidden


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny", 512, 4, 512, SEED_BASE + 0),
        Workload("train", 4096, 4, 5120, SEED_BASE + 1),
        Workload("long", 16384, 4, 5120, SEED_BASE + 2),
        Workload("addend", 16384, 4, 5120, SEED_BASE + 3, addend=True),
        Workload("large", 65536, 4, 5120, SEED_BASE + 4, rescale_rows=True),
        Workload("ragged", 4095, 4, 5120, SEED_BASE + 14, rescale_rows=True),
    )
}


def custom(T: int, streams: int = 4, hidden: int = 512, seed: int = 1,
           addend: bool = False, rescale_rows: bool = False) -> Workload:
    """A workload of any shape, drawn from the same distributions."""
    return Workload(f"T{T}_s{streams}_h{hidden}", T, streams, hidden, seed,
                    addend, rescale_rows)


def garbage_tail(T: int, device="cpu") -> torch.Tensor:
    """[T, 8] FP32 garbage for the ignored grad_proj columns 24..31."""
    tail = torch.empty(T, PROJ_STRIDE - PROJ_COLS, dtype=torch.float32, device=device)
    tail[:, 0::2] = float("nan")
    tail[:, 1::2] = 1e30
    return tail


def make(w: Workload, device="cpu") -> dict:
    """Draw every input of workload ``w`` on ``device`` (torch tensors)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    T, K = w.T, w.K
    x = torch.randn(T, K, generator=g, device=dev, dtype=torch.float32)
    if w.rescale_rows:
        expo = torch.rand(T, 1, generator=g, device=dev, dtype=torch.float64) * 4.0 - 2.0
        x.mul_(torch.pow(10.0, expo).to(torch.float32))
    wt = torch.randn(PROJ_COLS, K, generator=g, device=dev, dtype=torch.float32) * 0.02
    gp = torch.empty(T, PROJ_STRIDE, device=dev, dtype=torch.float32)
    gp[:, :PROJ_COLS] = torch.randn(T, PROJ_COLS, generator=g, device=dev,
                                    dtype=torch.float32) * 0.01
    gp[:, PROJ_COLS:] = garbage_tail(T, dev)
    grad_r = torch.randn(T, generator=g, device=dev, dtype=torch.float32) * 0.01
    r = forward_rms(x)
    out = dict(x=x, w=wt, grad_proj=gp, grad_r=grad_r, r=r, addend=None)
    if w.addend:
        a = torch.randn(T, K, generator=g, device=dev, dtype=torch.float32) * 0.01
        out["addend"] = a.to(torch.bfloat16)
    return out


def forward_rms(x: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """The forward's positive RMS per row, in FP64, stored as FP32."""
    rows = []
    step = 1024
    for i in range(0, x.shape[0], step):
        xx = x[i:i + step].to(torch.float64)
        rows.append(torch.sqrt((xx * xx).mean(dim=1) + eps).to(torch.float32))
    if not rows:
        return torch.empty(0, dtype=torch.float32, device=x.device)
    return torch.cat(rows)


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """Reinterpret a BF16 tensor as its uint16 bit patterns (int16 storage)."""
    return t.view(torch.int16)


# ---- inputs of the forward map (X and W as above, plus structured cases) ----

def forward_inputs(w: Workload, device="cpu") -> dict:
    """X [T, K] and W [24, K] of workload ``w`` (the same draws as make())."""
    full = make(w, device)
    return dict(x=full["x"], w=full["w"])


def odd_integers(shape, seed: int, limit: int = 2047) -> torch.Tensor:
    """Odd integers in [-limit, limit] as FP32 (11 significant bits at most,
    so a TF32 value has both a BF16 high and a nonzero low part)."""
    g = torch.Generator()
    g.manual_seed(seed)
    v = torch.randint(0, (limit + 1) // 2, shape, generator=g) * 2 + 1
    sign = torch.randint(0, 2, shape, generator=g) * 2 - 1
    return (v * sign).to(torch.float32)


def sparse_signs(shape, seed: int, nonzero: float = 0.25) -> torch.Tensor:
    """Entries in {-1, 0, +1} with the given fraction of nonzeros, FP32."""
    g = torch.Generator()
    g.manual_seed(seed)
    keep = torch.rand(shape, generator=g) < nonzero
    sign = torch.randint(0, 2, shape, generator=g) * 2 - 1
    return (keep * sign).to(torch.float32)


def low_bit_values(shape, seed: int) -> torch.Tensor:
    """N(0, 1) FP32 values whose low 13 fraction bits are random, with a
    quarter of them set to exact TF32 ties (bit 12 set, bits 0..11 clear)."""
    g = torch.Generator()
    g.manual_seed(seed)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    u = v.view(torch.int32)
    tie = torch.rand(shape, generator=g) < 0.25
    u[tie] = (u[tie] & ~0x1FFF) | 0x1000
    return v


def one_hot_rows(T: int, K: int, seed: int) -> torch.Tensor:
    """[T, K] FP32 with one low-bit value per row at a random column."""
    g = torch.Generator()
    g.manual_seed(seed)
    cols = torch.randint(0, K, (T,), generator=g)
    x = torch.zeros(T, K, dtype=torch.float32)
    x[torch.arange(T), cols] = low_bit_values((T,), seed + 1)
    return x


# ---- second workload: the BF16 RMSNorm backward --------------------------------
# Inputs of the backward named on the
# "flashinfer.cake_rmsnorm_det_train.cake_rmsnorm_det_train_backward" page:
#
#   g           BF16 [T, H], N(0, 1)  (the gradient of y; its scale does not
#               matter for relative errors)
#   x           BF16 [T, H], N(0, 1)  (the normalised input)
#   w           [H], 1 + N(0, 0.1), BF16 or FP32 (a trained RMSNorm weight
#               near its initial value 1)
#   rstd        FP32 [T], (mean(x^2) + 1e-6)^(-1/2) of the BF16 x, computed in
#               FP64 and rounded once (what the forward returns)
#   g_residual  BF16 [T, H], N(0, 1), only where a workload has one
#
# The widths are the page's (256 ... 6144); 5120 is the hidden size of the
# projection stage above, and T = 4096 and 16384 its token counts.

@dataclass(frozen=True)
class RmsWorkload:
    name: str
    T: int
    H: int
    seed: int
    w_f32: bool = False
    residual: bool = False


RMS_WORKLOADS = {
    w.name: w
    for w in (
        RmsWorkload("rms_small", 300, 1536, SEED_BASE + 20),
        RmsWorkload("rms_train", 4096, 5120, SEED_BASE + 21),
        RmsWorkload("rms_long", 16384, 5120, SEED_BASE + 22),
        RmsWorkload("rms_residual", 4096, 6144, SEED_BASE + 23, residual=True),
        RmsWorkload("rms_w32", 4096, 5120, SEED_BASE + 24, w_f32=True),
    )
}


def rms_custom(T: int, H: int, seed: int = 1, w_f32: bool = False,
               residual: bool = False) -> RmsWorkload:
    return RmsWorkload(f"rms_T{T}_H{H}", T, H, seed, w_f32, residual)


def rms_inputs(w: RmsWorkload, device="cpu") -> dict:
    """Draw g, x, w, rstd (and g_residual) of ``w`` on the CPU, then move them
    to ``device``; BF16 tensors are torch.bfloat16."""
    gen = torch.Generator()
    gen.manual_seed(w.seed)
    T, H = w.T, w.H
    g = torch.randn(T, H, generator=gen).to(torch.bfloat16)
    x = torch.randn(T, H, generator=gen).to(torch.bfloat16)
    wt = 1.0 + 0.1 * torch.randn(H, generator=gen)
    wt = wt.to(torch.float32) if w.w_f32 else wt.to(torch.bfloat16)
    rstd = rms_rstd(x)
    res = torch.randn(T, H, generator=gen).to(torch.bfloat16) if w.residual else None
    out = dict(g=g, x=x, w=wt, rstd=rstd, res=res)
    return {k: (v.to(device) if v is not None else None) for k, v in out.items()}


def rms_rstd(x: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """(mean(x^2) + eps)^(-1/2) per row of a BF16 x, in FP64, stored as FP32."""
    rows = []
    for i in range(0, x.shape[0], 1024):
        xx = x[i:i + 1024].to(torch.float64)
        rows.append(torch.rsqrt((xx * xx).mean(dim=1) + eps).to(torch.float32))
    if not rows:
        return torch.empty(0, dtype=torch.float32, device=x.device)
    return torch.cat(rows)
