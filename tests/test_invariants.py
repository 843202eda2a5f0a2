"""GPU checks of the stage's contract and of bit-level rounding, through the
C-ABI ("DSv4.1 mHC projection/RMS backward" page: introduction and
"Requirements and tensor contract"; prime-kernels pull request 15, "fused mHC
stream gradient" item for the addend).

* grad_proj = 0 leaves only the RMS term, grad_r / (r K) * x: the one check
  that sees it (it is ~1e-3 of |dX| at the workloads' scales);
* columns 24..31 of grad_proj are never read, even when NaN or infinite;
* outputs and workspace prefilled with anything are fully overwritten;
* hand-derived TF32 and BF16 bit tables (tests/golden/) hold through the GPU
  path: TF32 of x and of P through dW, TF32 of W and BF16 rounding through dX;
* the addend is added to the FP32 dX before one rounding to BF16;
* non-finite inputs give non-finite outputs exactly where IEEE arithmetic on
  TF32 operands does, and leave every other output unchanged.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import gpu_harness as gh
from tests import metrics as mt

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            a, b = line.split()[:2]
            rows.append((int(a, 16), b))
    return rows


def _f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def _inputs(T, hidden, seed=3):
    return workloads.make(workloads.custom(T, 4, hidden, seed=seed), "cuda")


def _bits16(t):
    return t.view(torch.int16)


def _bits32(t):
    return t.view(torch.int32)


# ------------------------------------------------------------ RMS term -------

@pytest.mark.parametrize("T,hidden", [(300, 64), (4096, 5120)])
def test_zero_grad_proj_leaves_rms_term(T, hidden):
    inp = _inputs(T, hidden)
    inp["grad_proj"][:, :24] = 0.0
    dx, dw, _, plan = gh.run(inp)
    assert bool((dw == 0).all().item())
    K = 4 * hidden
    rng = np.random.default_rng(T)
    rows = sorted(set([0, T - 1] + rng.integers(0, T, 24).tolist()))
    h = gh.host_rows(inp, rows)
    ref = oracle.dx(h["x"], h["w"], h["grad_proj"], h["grad_r"], h["r"], K, mode="tf32")
    got = mt.bf16_bits_to_f64(gh.bf16_bits_np(dx.index_select(0, torch.as_tensor(rows,
                                                                                 device="cuda"))))
    bad = mt.dx_violations(got, ref)
    assert len(bad) == 0, bad[:5].tolist()
    # every element: one rounding of the RMS term, within 1 BF16 ulp of it
    c = inp["grad_r"].double() / (inp["r"].double() * K)
    exact = c[:, None] * inp["x"].double()
    err = (dx.double() - exact).abs()
    a = exact.abs()
    e = torch.floor(torch.log2(torch.where(a > 0, a, torch.ones_like(a))))
    ulp = torch.clamp(torch.exp2(e - 7), min=2.0 ** -133)
    assert bool((err <= ulp * 1.0001 + 1e-30).all().item())


# ------------------------------------------------------- contract -----------

def test_tail_columns_never_read():
    inp = _inputs(700, 200, seed=9)
    base = dict(inp)
    gp0 = inp["grad_proj"].clone()
    gp0[:, 24:] = 0.0
    base["grad_proj"] = gp0
    dx0, dw0, _, _ = gh.run(base)
    for garbage in (float("nan"), float("inf"), float("-inf"), 1e30):
        g = gp0.clone()
        g[:, 24:] = garbage
        other = dict(inp)
        other["grad_proj"] = g
        dx1, dw1, _, _ = gh.run(other)
        assert torch.equal(_bits16(dx1), _bits16(dx0)), garbage
        assert torch.equal(_bits32(dw1), _bits32(dw0)), garbage


def test_prefilled_outputs_and_workspace_are_overwritten():
    inp = _inputs(1100, 96, seed=11)
    dx0, dw0, ws, plan = gh.run(inp, poison=False)
    dx0, dw0 = dx0.clone(), dw0.clone()
    T, K = inp["x"].shape
    for fill in (float("nan"), 0.0, -1.0e38):
        dx, dw, ws = gh.alloc_outputs(T, K, plan, "cuda", poison=False)
        dx.fill_(fill)
        dw.fill_(fill)
        ws.view(torch.float32).fill_(fill)
        gh.run(inp, plan=plan, outputs=(dx, dw, ws))
        assert torch.equal(_bits16(dx), _bits16(dx0))
        assert torch.equal(_bits32(dw), _bits32(dw0))


# ------------------------------------------------- rounding tables ----------

def _finite_tf32_cases():
    out = []
    for inp, exp in _table("tf32_rne.txt"):
        if exp == "nan":
            continue
        e = int(exp, 16)
        if (e & 0x7F800000) == 0x7F800000:  # results that overflow to infinity
            continue
        if (inp & 0x7F800000) == 0 and (inp & 0x7FFFFF) != 0:
            continue  # subnormal inputs: test_subnormal_tf32_operands_against_oracle
        out.append((inp, e))
    return out


def test_tf32_of_x_through_dw():
    cases = _finite_tf32_cases()
    n = len(cases)
    hidden = ((n + 3) // 4 + 1) // 2 * 2
    K = 4 * hidden
    T = 1
    x = np.ones((T, K), dtype=np.float32)
    x[0, :n] = _f32([c[0] for c in cases])
    gp = np.zeros((T, 32), dtype=np.float32)
    j = 5
    gp[0, j] = 1.0
    inp = dict(x=torch.tensor(x, device="cuda"),
               w=torch.zeros(24, K, device="cuda"),
               grad_proj=torch.tensor(gp, device="cuda"),
               grad_r=torch.zeros(T, device="cuda"), r=torch.ones(T, device="cuda"), addend=None)
    _, dw, _, _ = gh.run(inp)
    got = gh.host(dw)[j, :n].view(np.uint32)
    # a sum that starts from +0 turns -0 into +0: signed zeros compare equal
    canon = lambda v: 0 if (int(v) & 0x7FFFFFFF) == 0 else int(v)
    assert [hex(canon(v)) for v in got] == [hex(canon(c[1])) for c in cases]


def test_tf32_of_p_through_dw():
    cases = _finite_tf32_cases()
    n = len(cases)
    T = (n + 23) // 24
    K = 8 * ((T + 7) // 8)
    vals = np.ones(T * 24, dtype=np.float32)
    vals[:n] = _f32([c[0] for c in cases])
    gp = np.zeros((T, 32), dtype=np.float32)
    gp[:, :24] = vals.reshape(T, 24)
    x = np.zeros((T, K), dtype=np.float32)
    for t in range(T):
        x[t, t] = 1.0            # row t of P lands in column t of dW
    inp = dict(x=torch.tensor(x, device="cuda"), w=torch.zeros(24, K, device="cuda"),
               grad_proj=torch.tensor(gp, device="cuda"),
               grad_r=torch.zeros(T, device="cuda"), r=torch.ones(T, device="cuda"), addend=None)
    _, dw, _, _ = gh.run(inp)
    got = gh.host(dw)
    canon = lambda v: 0 if (int(v) & 0x7FFFFFFF) == 0 else int(v)
    for idx, (inp_bits, exp_bits) in enumerate(cases):
        t, jj = divmod(idx, 24)
        g = int(got[jj, t:t + 1].view(np.uint32)[0])
        assert canon(g) == canon(exp_bits), hex(inp_bits)


def test_bf16_rounding_through_dx():
    """P = 0, r K = 1, grad_r = 1: dX = BF16(x) bit for bit."""
    table = [(i, e) for i, e in _table("bf16_rne.txt")
             if not ((i & 0x7F800000) == 0 and (i & 0x7FFFFF) != 0)]
    n = len(table)
    hidden = 512
    K = 4 * hidden
    x = np.full((1, K), 1.0, dtype=np.float32)
    x[0, :n] = _f32([c[0] for c in table])
    inp = dict(x=torch.tensor(x, device="cuda"), w=torch.zeros(24, K, device="cuda"),
               grad_proj=torch.zeros(1, 32, device="cuda"),
               grad_r=torch.ones(1, device="cuda"),
               r=torch.full((1,), 2.0 ** -11, device="cuda"), addend=None)
    dx, _, _, _ = gh.run(inp)
    got = gh.bf16_bits_np(dx)[0, :n]
    for (inp_bits, exp), g in zip(table, got):
        if exp == "nan":
            assert (int(g) & 0x7F80) == 0x7F80 and (int(g) & 0x7F) != 0, hex(inp_bits)
        elif int(exp, 16) in (0x0000, 0x8000):
            assert int(g) & 0x7FFF == 0, hex(inp_bits)        # +-0 compare equal
        else:
            assert int(g) == int(exp, 16), (hex(inp_bits), hex(int(g)), exp)


def test_tf32_of_w_through_dx():
    """One-hot P, grad_r = 0: dX = BF16(TF32(w)); 0x3F817FFF gives 0x3F82
    where BF16(w) alone would be 0x3F81."""
    K = 64
    rng = np.random.default_rng(5)
    w = rng.standard_normal((24, K)).astype(np.float32)
    w[7, 0] = _f32([0x3F817FFF])[0]
    gp = np.zeros((1, 32), dtype=np.float32)
    gp[0, 7] = 1.0
    inp = dict(x=torch.ones(1, K, device="cuda"), w=torch.tensor(w, device="cuda"),
               grad_proj=torch.tensor(gp, device="cuda"), grad_r=torch.zeros(1, device="cuda"),
               r=torch.ones(1, device="cuda"), addend=None)
    dx, _, _, _ = gh.run(inp)
    got = gh.bf16_bits_np(dx)[0]
    assert int(got[0]) == 0x3F82
    expect = [oracle.bf16_bits(np.float32(oracle.tf32(v))) for v in w[7]]
    assert [int(v) for v in got] == expect


def test_subnormal_tf32_operands_against_oracle():
    """Subnormal x (the subnormal rows of the hand-derived TF32 table) times a
    one-hot P: dW against the TF32-mode oracle, within the stated bound of
    the known departure of the matrix-unit path (metrics.flush_bound: every
    product may lose the parts of its BF16 operands and partial products that
    lie below the smallest normal number, 2^-126).  The oracle keeps these
    products; the GPU's BF16 matrix units read subnormal inputs as zero, so
    they come out as zero, within that bound.  Operands that round up to the
    smallest normal number (0x007FF000 -> 0x00800000) are exact."""
    tf = [(i, int(e, 16)) for i, e in _table("tf32_rne.txt")
          if (i & 0x7F800000) == 0 and (i & 0x7FFFFF) != 0]
    assert tf
    K = 2048
    x = np.ones((1, K), dtype=np.float32)
    x[0, :len(tf)] = _f32([c[0] for c in tf])
    gp = np.zeros((1, 32), dtype=np.float32)
    gp[0, 2] = 1.0
    inp = dict(x=torch.tensor(x, device="cuda"), w=torch.zeros(24, K, device="cuda"),
               grad_proj=torch.tensor(gp, device="cuda"), grad_r=torch.zeros(1, device="cuda"),
               r=torch.ones(1, device="cuda"), addend=None)
    _, dw, _, _ = gh.run(inp)
    got = gh.host(dw).astype(np.float64)
    ref = oracle.dw(x, gp, mode="tf32")
    gp_abs = np.abs(gp)
    gp_abs[:, 24:] = 0.0
    # one product per element: |P[0, j]| and |x[0, k]| bound its operands
    abs_p = np.abs(gp[0, :24])[:, None] * np.ones((1, K))
    abs_x = np.ones((24, 1)) * np.abs(x[0].astype(np.float64))[None, :]
    bound = (mt.dw_accumulation_bound(oracle.dw(np.abs(x), gp_abs, mode="tf32"), 1, 1)
             + mt.flush_bound(abs_p, abs_x, 1))
    err = np.abs(got - ref)
    assert np.all(err <= bound), (err / bound).max()
    # the table's subnormal inputs all lie below 2^-126: their products are
    # the only elements allowed to differ, and the normal ones are exact
    normal = np.abs(ref) >= 2.0 ** -126
    assert np.array_equal(got[normal], ref[normal])
    # the rows whose TF32 value is normal (a carry out of the fraction)
    expect_normal = [e for _, e in tf if (e & 0x7F800000) != 0]
    got_bits = gh.host(dw)[2, :len(tf)].view(np.uint32)
    assert [int(v) for v, (_, e) in zip(got_bits, tf) if (e & 0x7F800000) != 0] == expect_normal


def test_subnormal_bf16_rounding_through_dx():
    """BF16 rounding of subnormal FP32 dX values at the fraction field."""
    bf = [(i, int(e, 16)) for i, e in _table("bf16_rne.txt")
          if (i & 0x7F800000) == 0 and (i & 0x7FFFFF) != 0]
    assert bf
    K = 2048
    x = np.ones((1, K), dtype=np.float32)
    x[0, :len(bf)] = _f32([c[0] for c in bf])
    inp = dict(x=torch.tensor(x, device="cuda"), w=torch.zeros(24, K, device="cuda"),
               grad_proj=torch.zeros(1, 32, device="cuda"), grad_r=torch.ones(1, device="cuda"),
               r=torch.full((1,), 2.0 ** -11, device="cuda"), addend=None)
    dx, _, _, _ = gh.run(inp)
    got = gh.bf16_bits_np(dx)[0, :len(bf)]
    assert [hex(int(v)) for v in got] == [hex(e) for _, e in bf]


# ----------------------------------------------------------- addend ---------

def test_addend_is_added_before_one_rounding():
    hidden = 512
    K = 4 * hidden
    T = 37
    rng = np.random.default_rng(8)
    x = rng.standard_normal((T, K)).astype(np.float32)
    a = (rng.standard_normal((T, K)) * 1e-3).astype(np.float32)
    a_bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    a_val = (a_bits.astype(np.uint32) << 16).view(np.float32)
    e = np.array([2.0 ** -(t % 5) for t in range(T)], dtype=np.float32)
    base = dict(x=torch.tensor(x, device="cuda"), w=torch.zeros(24, K, device="cuda"),
                grad_proj=torch.zeros(T, 32, device="cuda"), grad_r=torch.tensor(e, device="cuda"),
                r=torch.full((T,), 2.0 ** -11, device="cuda"), addend=None)
    with_a = dict(base, addend=torch.tensor(a_bits.view(np.int16), device="cuda").view(torch.bfloat16))
    dx, _, _, _ = gh.run(with_a)
    got = gh.bf16_bits_np(dx)
    # c = grad_r exactly, so the FP32 value before rounding is fl32(c x + a)
    pre = (e[:, None].astype(np.float64) * x + a_val).astype(np.float32)
    expect = np.array([[oracle.bf16_bits(v) for v in row] for row in pre], dtype=np.uint16)
    assert np.array_equal(got, expect)
    # grad_r = 0: dX is the addend itself
    dx0, _, _, _ = gh.run(dict(with_a, grad_r=torch.zeros(T, device="cuda")))
    same = gh.bf16_bits_np(dx0)
    assert np.all((same == a_bits) | (((same | a_bits) & 0x7FFF) == 0))
    # a zero addend changes nothing (up to the sign of zero)
    zero = dict(base, addend=torch.zeros(T, K, device="cuda", dtype=torch.bfloat16))
    dz, _, _, _ = gh.run(zero)
    dn, _, _, _ = gh.run(base)
    bz, bn = gh.bf16_bits_np(dz), gh.bf16_bits_np(dn)
    assert np.all((bz == bn) | (((bz | bn) & 0x7FFF) == 0))


# ------------------------------------------------------- non-finite ---------

def test_non_finite_inputs_stay_local():
    inp_c = workloads.make(workloads.custom(64, 4, 64, seed=21), "cpu")
    x = inp_c["x"].numpy().copy()
    gp = inp_c["grad_proj"].numpy().copy()
    x[3, 17] = np.inf
    x[40, 100] = np.nan
    x[10, 5] = -np.inf
    gp[20, 4] = np.inf
    inp_c["x"] = torch.tensor(x)
    inp_c["grad_proj"] = torch.tensor(gp)
    inp = gh.to_device(inp_c, "cuda")
    dx, dw, _, _ = gh.run(inp)
    K = x.shape[1]
    with np.errstate(invalid="ignore", over="ignore"):
        ref_dx = oracle.dx(x, inp_c["w"].numpy(), gp, inp_c["grad_r"].numpy(),
                           inp_c["r"].numpy(), K)
        ref_dw = oracle.dw(x, gp)
    got_dx = mt.bf16_bits_to_f64(gh.bf16_bits_np(dx))
    got_dw = gh.host(dw).astype(np.float64)
    # the non-finite outputs are exactly where IEEE arithmetic puts them; a
    # NaN of the oracle is a NaN, an infinity of the oracle is the same
    # infinity or a NaN (the known departure of the matrix-unit path: the
    # BF16 split of an infinite operand meets zero parts, inf x 0 = NaN)
    assert np.array_equal(~np.isfinite(got_dx), ~np.isfinite(ref_dx))
    assert np.array_equal(~np.isfinite(got_dw), ~np.isfinite(ref_dw))
    for got, ref in ((got_dx, ref_dx), (got_dw, ref_dw)):
        assert np.all(np.isnan(got[np.isnan(ref)]))
        inf = np.isinf(ref)
        assert np.all(np.isnan(got[inf]) | (got[inf] == ref[inf]))
    fin = np.isfinite(ref_dx)
    assert len(mt.dx_violations(got_dx[fin], ref_dx[fin], np.abs(ref_dx[fin]).max())) == 0
    finw = np.isfinite(ref_dw)
    assert mt.rel_frobenius(got_dw[finw], ref_dw[finw]) < 1e-5


@pytest.mark.parametrize("T,hidden", [(4096, 5120), (4097, 5120), (512, 512), (600, 20480)])
def test_workspace_slabs_written_match_partial_slab_count(T, hidden):
    """Kernel 1 writes exactly mhcpb_plan_partial_slabs of the S workspace
    slabs: the slab group holding slabs 0 .. n-1 of each column tile stores
    only their sum, in slab n - 1, and never touches slabs 0 .. n - 2.  The
    workspace is prefilled with all-ones words (NaN); written slabs hold the
    finite partials."""
    from rms_backward_amd import mhcpb_plan_partial_slabs, mhcpb_plan_split_count
    wl = workloads.custom(T, 4, hidden, seed=T + 3 * hidden)
    inp = workloads.make(wl, "cuda")
    dx, dw, ws, plan = gh.run(inp)
    S = mhcpb_plan_split_count(plan.handle)
    moved = mhcpb_plan_partial_slabs(plan.handle)
    slabs = ws.view(torch.int32)[: S * 24 * wl.K].view(S, 24 * wl.K)
    untouched = [bool((slabs[s] == -1).all().item()) for s in range(S)]
    written = [bool(torch.isfinite(slabs[s].view(torch.float32)).all().item()) for s in range(S)]
    first = S - moved
    assert untouched == [s < first for s in range(S)]
    assert written == [s >= first for s in range(S)]
    assert bool(torch.isfinite(dw).all().item())
