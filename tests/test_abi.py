"""Host-side checks of the C-ABI library (no kernel is ever launched here).

* the library loads and exports every function include/mhcpb.h declares;
* plan creation accepts the supported domain and rejects the rest;
* the workspace at the page's supported profile is the printed 15,728,640
  bytes ("DSv4.1 mHC projection/RMS backward", "Prepared class API");
* the split schedule depends on T only;
* execute() rejects NULL, misaligned and overlapping pointers and a short
  workspace before touching the GPU ("Requirements and tensor contract").
"""
import ctypes
import os
import re

import pytest

import rms_backward_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "mhcpb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhcpb_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert "mhcpb_execute" in names and "mhcpb_plan_create" in names
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(m.EXPORTED)


def test_workspace_at_supported_profile_matches_page():
    line = [l for l in open(os.path.join(ROOT, "tests", "golden", "workspace_profile.txt"))
            if l.strip() and not l.startswith("#")][0]
    T, streams, hidden, ws = (int(v) for v in line.split())
    plan = m.mhcpb_plan_create(T, streams, hidden)
    try:
        assert m.mhcpb_workspace_bytes(plan) == ws == 15728640
        assert m.mhcpb_plan_split_count(plan) == 8
    finally:
        m.mhcpb_plan_destroy(plan)


@pytest.mark.parametrize("T,hidden,moved", [
    # 64 tiles of 320 columns x 8 slabs: 4 slab groups of 2; group 0 stores
    # only the sum of slabs 0 and 1.
    (4096, 5120, 7),
    # 32 slabs in 4 groups of 8: group 0 leaves one of its 8.
    (16384, 5120, 25), (65536, 5120, 25),
    # 256 tiles alone fill the GPU: one group walks all 8 slabs.
    (4096, 20480, 1),
    # tiny: 32 tiles of 64 columns x 8 slabs, one slab per group.
    (512, 512, 8),
    # 9 slabs in 4 groups of 2, 2, 2 and 3: group 0 stores the sum of 0 and 1.
    (4097, 5120, 8),
    # 16 or 30 tiles of 320 columns, 8 groups of one slab.
    (1024, 1280, 8), (4096, 2400, 8),
    # one slab: nothing to fold.
    (40, 1 << 20, 1), (16, 64, 1),
])
def test_partial_slabs_moved(T, hidden, moved):
    plan = m.mhcpb_plan_create(T, 4, hidden)
    try:
        assert m.mhcpb_plan_partial_slabs(plan) == moved
        assert 1 <= moved <= m.mhcpb_plan_split_count(plan)
    finally:
        m.mhcpb_plan_destroy(plan)


@pytest.mark.parametrize("T,expect", [(1, 1), (64, 1), (65, 2), (300, 5), (448, 7), (449, 8),
                                      (511, 8), (512, 8), (513, 8), (4095, 8), (4096, 8),
                                      (4097, 9), (16383, 32), (16384, 32), (65536, 32),
                                      (2**31 - 1, 32)])
def test_split_count_depends_on_T_only(T, expect):
    for hidden in (2, 512, 5120):
        plan = m.mhcpb_plan_create(T, 4, hidden)
        try:
            assert m.mhcpb_plan_split_count(plan) == expect
            assert m.mhcpb_workspace_bytes(plan) == expect * 24 * 4 * hidden * 4
        finally:
            m.mhcpb_plan_destroy(plan)


def test_split_schedule_properties():
    """Over every T up to 20000 and a sample beyond: S never decreases as T
    grows, stays within 1..32, gives every slab at least one row (the kernel
    takes rows [s L, min((s+1) L, T)) with L = ceil(T / S)), keeps the slabs
    at 512 rows or fewer from T = 4096 up to the cap, and does not depend on
    hidden."""
    prev = 0
    Ts = list(range(1, 20001)) + [2**k + d for k in range(15, 31) for d in (-1, 0, 1)]
    for T in Ts:
        plan = m.mhcpb_plan_create(T, 4, 2)
        try:
            S = m.mhcpb_plan_split_count(plan)
        finally:
            m.mhcpb_plan_destroy(plan)
        L = -(-T // S)
        assert 1 <= S <= 32 and S <= T, T
        assert (S - 1) * L < T, f"T={T}: slab {S - 1} would be empty"
        if T <= 20000:
            assert S >= prev, T
            prev = S
        if 4096 <= T <= 32 * 512:
            assert L <= 512, T
    for T in (7, 300, 4096, 16385):
        counts = set()
        for hidden in (2, 64, 5120, 2**20):
            plan = m.mhcpb_plan_create(T, 4, hidden)
            try:
                counts.add(m.mhcpb_plan_split_count(plan))
            finally:
                m.mhcpb_plan_destroy(plan)
        assert len(counts) == 1, T


@pytest.mark.parametrize("T,streams,hidden,status", [
    (0, 4, 512, m.MHCPB_ERROR_INVALID_ARGUMENT),
    (-5, 4, 512, m.MHCPB_ERROR_INVALID_ARGUMENT),
    (2**31, 4, 512, m.MHCPB_ERROR_UNSUPPORTED),
    (16, 3, 512, m.MHCPB_ERROR_UNSUPPORTED),
    (16, 8, 512, m.MHCPB_ERROR_UNSUPPORTED),
    (16, 4, 511, m.MHCPB_ERROR_UNSUPPORTED),
    (16, 4, 0, m.MHCPB_ERROR_UNSUPPORTED),
    (16, 4, 2**20 + 2, m.MHCPB_ERROR_UNSUPPORTED),
])
def test_plan_create_rejects(T, streams, hidden, status):
    st, h = m.mhcpb_plan_create_status(T, streams, hidden)
    assert st == status
    assert h is None


def test_status_strings():
    for st in range(7):
        assert m.mhcpb_status_string(st)
    assert "align" in m.mhcpb_status_string(m.MHCPB_ERROR_MISALIGNED)


def _no_gpu_visible():
    import torch
    return torch.cuda.device_count() == 0


# The calls below hand the library fake device addresses that it only checks.
# Each one must fail validation before any launch; as a second guard they are
# never run where a GPU is visible.
fake_addresses = pytest.mark.skipif(not _no_gpu_visible(),
                                    reason="fake device addresses are used only without a GPU")


class _FakeBuffers:
    """Disjoint, aligned fake device addresses: validation never dereferences
    them, and none of these calls reaches a launch."""

    def __init__(self, T, hidden):
        K = 4 * hidden
        sizes = dict(x=T * K * 4, w=24 * K * 4, grad_proj=T * 128, grad_r=T * 4, r=T * 4,
                     dx=T * K * 2, dw=24 * K * 4, addend=T * K * 2,
                     ws=m.mhcpb_workspace_bytes(m.mhcpb_plan_create(T, 4, hidden)) + 256)
        base = 1 << 40
        self.addr = {}
        for k, n in sizes.items():
            self.addr[k] = base
            base += (n + 4095) // 4096 * 4096 + 4096
        self.ws_size = sizes["ws"]
        self.ws_needed = sizes["ws"] - 256

    def args(self, **over):
        a = dict(self.addr)
        a.update(over)
        return a


def _exec(plan, a, ws_size):
    return m.mhcpb_execute(plan, a["x"], a["w"], a["grad_proj"], a["grad_r"], a["r"],
                           a["dx"], a["dw"], a.get("addend"), a["ws"], ws_size, 0,
                           check=False)


@pytest.mark.parametrize("field", ["x", "w", "grad_proj", "grad_r", "r", "dx", "dw", "ws",
                                   "addend"])
@fake_addresses
def test_execute_rejects_misaligned(field):
    plan = m.mhcpb_plan_create(64, 4, 64)
    fb = _FakeBuffers(64, 64)
    try:
        for off in (1, 4, 8):
            a = fb.args(**{field: fb.addr[field] + off})
            assert _exec(plan, a, fb.ws_size) == m.MHCPB_ERROR_MISALIGNED
    finally:
        m.mhcpb_plan_destroy(plan)


@pytest.mark.parametrize("field", ["x", "w", "grad_proj", "grad_r", "r", "dx", "dw", "ws"])
@fake_addresses
def test_execute_rejects_null(field):
    plan = m.mhcpb_plan_create(64, 4, 64)
    fb = _FakeBuffers(64, 64)
    try:
        a = fb.args(**{field: None})
        assert _exec(plan, a, fb.ws_size) == m.MHCPB_ERROR_INVALID_ARGUMENT
        assert _exec(None, fb.args(), fb.ws_size) == m.MHCPB_ERROR_INVALID_ARGUMENT
    finally:
        m.mhcpb_plan_destroy(plan)


@pytest.mark.parametrize("a,b", [("x", "dx"), ("dx", "dw"), ("ws", "dw"), ("addend", "dx"),
                                 ("r", "grad_r"), ("w", "grad_proj"), ("x", "addend")])
@fake_addresses
def test_execute_rejects_overlap(a, b):
    plan = m.mhcpb_plan_create(64, 4, 64)
    fb = _FakeBuffers(64, 64)
    try:
        # b starts 16 bytes before the end of a
        K = 256
        size = dict(x=64 * K * 4, dx=64 * K * 2, ws=fb.ws_needed, addend=64 * K * 2,
                    r=64 * 4, w=24 * K * 4)[a]
        args = fb.args(**{b: fb.addr[a] + size - 16})
        assert _exec(plan, args, fb.ws_size) == m.MHCPB_ERROR_OVERLAP
        args = fb.args(**{b: fb.addr[a]})
        assert _exec(plan, args, fb.ws_size) == m.MHCPB_ERROR_OVERLAP
    finally:
        m.mhcpb_plan_destroy(plan)


@fake_addresses
def test_execute_rejects_short_workspace():
    plan = m.mhcpb_plan_create(4096, 4, 5120)
    fb = _FakeBuffers(4096, 5120)
    try:
        need = m.mhcpb_workspace_bytes(plan)
        assert _exec(plan, fb.args(), need - 1) == m.MHCPB_ERROR_WORKSPACE
        assert _exec(plan, fb.args(), 0) == m.MHCPB_ERROR_WORKSPACE
    finally:
        m.mhcpb_plan_destroy(plan)


def test_null_plan_queries():
    lib = ctypes.CDLL(m.LIB_PATH)
    n = ctypes.c_size_t()
    lib.mhcpb_workspace_bytes.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    assert lib.mhcpb_workspace_bytes(None, ctypes.byref(n)) == m.MHCPB_ERROR_INVALID_ARGUMENT
    lib.mhcpb_plan_create.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int32]
    assert lib.mhcpb_plan_create(None, 16, 4, 64) == m.MHCPB_ERROR_INVALID_ARGUMENT
    assert m.mhcpb_plan_destroy(None) is None


def _exec_dx(plan, a):
    return m.mhcpb_execute_dx(plan, a["x"], a["w"], a["grad_proj"], a["grad_r"], a["r"],
                              a["dx"], a.get("addend"), 0, check=False)


def _exec_dw(plan, a, ws_size):
    return m.mhcpb_execute_dw(plan, a["x"], a["grad_proj"], a["dw"], a["ws"], ws_size, 0,
                              check=False)


@fake_addresses
def test_split_forms_validate_their_own_operands():
    """dX only needs x, w, grad_proj, grad_r, r, dx (and checks the addend when
    given); dW only needs x, grad_proj, dw and the workspace.  Every error is
    reported before a launch."""
    plan = m.mhcpb_plan_create(64, 4, 64)
    fb = _FakeBuffers(64, 64)
    try:
        for field in ("x", "w", "grad_proj", "grad_r", "r", "dx"):
            assert _exec_dx(plan, fb.args(**{field: None})) == m.MHCPB_ERROR_INVALID_ARGUMENT
            assert _exec_dx(plan, fb.args(**{field: fb.addr[field] + 4})) == m.MHCPB_ERROR_MISALIGNED
        assert _exec_dx(plan, fb.args(addend=fb.addr["addend"] + 8)) == m.MHCPB_ERROR_MISALIGNED
        assert _exec_dx(plan, fb.args(dx=fb.addr["x"] + 16)) == m.MHCPB_ERROR_OVERLAP
        assert _exec_dx(plan, fb.args(addend=fb.addr["dx"])) == m.MHCPB_ERROR_OVERLAP
        assert _exec_dx(None, fb.args()) == m.MHCPB_ERROR_INVALID_ARGUMENT
        for field in ("x", "grad_proj", "dw", "ws"):
            assert _exec_dw(plan, fb.args(**{field: None}), fb.ws_size) == \
                m.MHCPB_ERROR_INVALID_ARGUMENT
            assert _exec_dw(plan, fb.args(**{field: fb.addr[field] + 4}), fb.ws_size) == \
                m.MHCPB_ERROR_MISALIGNED
        assert _exec_dw(plan, fb.args(), fb.ws_needed - 1) == m.MHCPB_ERROR_WORKSPACE
        assert _exec_dw(plan, fb.args(dw=fb.addr["ws"]), fb.ws_size) == m.MHCPB_ERROR_OVERLAP
        assert _exec_dw(plan, fb.args(grad_proj=fb.addr["x"]), fb.ws_size) == m.MHCPB_ERROR_OVERLAP
        assert _exec_dw(None, fb.args(), fb.ws_size) == m.MHCPB_ERROR_INVALID_ARGUMENT
    finally:
        m.mhcpb_plan_destroy(plan)


def test_forward_workspace_is_the_tile_partials():
    for T, hidden in ((1, 2), (4096, 5120), (65536, 512), (17, 300)):
        plan = m.mhcpb_plan_create(T, 4, hidden)
        try:
            tiles = (4 * hidden + 1023) // 1024   # partials per 1024-column tile
            steps = (T + 15) // 16                # 16-token steps: 8 blocks of 64 FP32
            assert m.mhcpb_forward_workspace_bytes(plan) == tiles * steps * 8 * 64 * 4
        finally:
            m.mhcpb_plan_destroy(plan)


class _FakeForward:
    """Disjoint, aligned fake device addresses for the forward's operands."""

    def __init__(self, T, hidden):
        K = 4 * hidden
        plan = m.mhcpb_plan_create(T, 4, hidden)
        self.ws_needed = m.mhcpb_forward_workspace_bytes(plan)
        m.mhcpb_plan_destroy(plan)
        sizes = dict(x=T * K * 4, w=24 * K * 4, proj=T * 128, r=T * 4, ws=self.ws_needed)
        base = 1 << 41
        self.addr, self.size = {}, sizes
        for k, n in sizes.items():
            self.addr[k] = base
            base += (n + 4095) // 4096 * 4096 + 4096

    def args(self, **over):
        a = dict(self.addr)
        a.update(over)
        return a


def _fwd(plan, a, ws_size, eps=1e-6):
    return m.mhcpb_forward(plan, a["x"], a["w"], eps, a["proj"], a["r"], a["ws"], ws_size, 0,
                           check=False)


@fake_addresses
def test_forward_validates_before_any_launch():
    plan = m.mhcpb_plan_create(64, 4, 64)
    fb = _FakeForward(64, 64)
    ws = fb.ws_needed
    try:
        assert _fwd(None, fb.args(), ws) == m.MHCPB_ERROR_INVALID_ARGUMENT
        for field in ("x", "w", "proj", "r", "ws"):
            assert _fwd(plan, fb.args(**{field: None}), ws) == m.MHCPB_ERROR_INVALID_ARGUMENT
            for off in (4, 8):
                assert _fwd(plan, fb.args(**{field: fb.addr[field] + off}), ws) == \
                    m.MHCPB_ERROR_MISALIGNED
        for eps in (-1e-6, float("nan"), float("inf"), -float("inf")):
            assert _fwd(plan, fb.args(), ws, eps=eps) == m.MHCPB_ERROR_INVALID_ARGUMENT
        assert _fwd(plan, fb.args(), ws - 1) == m.MHCPB_ERROR_WORKSPACE
        for a, b in (("x", "proj"), ("proj", "r"), ("ws", "w"), ("x", "ws"), ("r", "x")):
            over = {b: fb.addr[a] + fb.size[a] - 16}
            assert _fwd(plan, fb.args(**over), ws) == m.MHCPB_ERROR_OVERLAP, (a, b)
        # too many units of work (tiles x 16-token steps >= 2^31)
        big = m.mhcpb_plan_create(2**31 - 1, 4, 2**20)
        try:
            assert _fwd(big, fb.args(), 1 << 62) == m.MHCPB_ERROR_UNSUPPORTED
        finally:
            m.mhcpb_plan_destroy(big)
    finally:
        m.mhcpb_plan_destroy(plan)


# ---- BF16 RMSNorm backward -----------------------------------------------------

def _rms_schedule(T, H):
    nc = -(-H // 512)
    return min(-(-T // 16), 256 * max(1, 12 // nc)) if T else 0


@pytest.mark.parametrize("T,H,S", [(1, 5120, 1), (16, 5120, 1), (17, 5120, 2), (100, 5120, 7),
                                   (4096, 5120, 256), (4097, 5120, 256), (16384, 5120, 256),
                                   (16384, 6144, 256), (16384, 2048, 768), (16384, 256, 1024),
                                   (65536, 512, 3072), (65536, 1536, 1024), (65536, 2560, 512)])
def test_rmsnorm_blocks_depend_on_t_and_h_only(T, H, S):
    assert _rms_schedule(T, H) == S
    assert m.mhcpb_rmsnorm_backward_workspace_bytes(T, H) == S * H * 4


@pytest.mark.parametrize("T,H,status", [(-1, 512, 1), (10, 0, 1), (10, -8, 1), (10, 4, 2),
                                        (10, 12, 2), (10, 6152, 2), (2**31, 512, 2),
                                        (0, 512, 0), (10, 6144, 0), (10, 8, 0)])
def test_rmsnorm_shape_checks(T, H, status):
    st, n = m.mhcpb_rmsnorm_backward_workspace_bytes(T, H, check=False)
    assert st == status
    if status == 0:
        assert n == _rms_schedule(T, H) * H * 4


class _FakeRms:
    def __init__(self, T, H, w_f32=False):
        S = _rms_schedule(T, H)
        self.ws_needed = S * H * 4
        sizes = dict(g=T * H * 2, x=T * H * 2, w=H * (4 if w_f32 else 2), rstd=T * 4,
                     res=T * H * 2, dx=T * H * 2, dw=H * 4, ws=self.ws_needed)
        base = 1 << 42
        self.addr, self.size = {}, sizes
        for k, n in sizes.items():
            self.addr[k] = base
            base += (n + 4095) // 4096 * 4096 + 4096

    def call(self, T, H, ws_size=None, w_dtype=0, **over):
        a = dict(self.addr)
        a.update(over)
        return m.mhcpb_rmsnorm_backward(T, H, a["g"], a["x"], a["w"], w_dtype, a["rstd"],
                                        a["res"], a["dx"], a["dw"], a["ws"],
                                        self.ws_needed if ws_size is None else ws_size, 0,
                                        check=False)


@fake_addresses
def test_rmsnorm_validates_before_any_launch():
    T, H = 64, 1024
    f = _FakeRms(T, H)
    for field in ("g", "x", "w", "rstd", "dx", "dw", "ws"):
        assert f.call(T, H, **{field: None}) == m.MHCPB_ERROR_INVALID_ARGUMENT, field
        for off in (2, 4, 8):
            assert f.call(T, H, **{field: f.addr[field] + off}) == m.MHCPB_ERROR_MISALIGNED
    assert f.call(T, H, res=f.addr["res"] + 8) == m.MHCPB_ERROR_MISALIGNED
    assert f.call(T, H, w_dtype=2) == m.MHCPB_ERROR_INVALID_ARGUMENT
    assert f.call(T, H, w_dtype=-1) == m.MHCPB_ERROR_INVALID_ARGUMENT
    assert f.call(T, H, ws_size=f.ws_needed - 1) == m.MHCPB_ERROR_WORKSPACE
    for a, b in (("g", "dx"), ("x", "res"), ("dw", "ws"), ("rstd", "w"), ("dx", "x"),
                 ("res", "dw")):
        over = {b: f.addr[a] + f.size[a] - 16}
        assert f.call(T, H, **over) == m.MHCPB_ERROR_OVERLAP, (a, b)
    # an FP32 weight is twice as long: overlapping only at its second half
    f32 = _FakeRms(T, H, w_f32=True)
    assert f32.call(T, H, w_dtype=1, dw=f32.addr["w"] + 2 * H) == m.MHCPB_ERROR_OVERLAP
    assert f.call(T, 12) == m.MHCPB_ERROR_UNSUPPORTED
    assert f.call(T, 6160) == m.MHCPB_ERROR_UNSUPPORTED


@fake_addresses
def test_rmsnorm_zero_rows_needs_only_w_and_dw():
    f = _FakeRms(64, 512)
    # T = 0: the row operands may be NULL, the workspace too (0 bytes)
    st = m.mhcpb_rmsnorm_backward(0, 512, None, None, f.addr["w"], 0, None, None, None,
                                  f.addr["dw"], None, 0, 0, check=False)
    assert st == m.MHCPB_ERROR_LAUNCH  # validation passed; no GPU here to launch on
    assert m.mhcpb_rmsnorm_backward(0, 512, None, None, None, 0, None, None, None,
                                    f.addr["dw"], None, 0, 0, check=False) == \
        m.MHCPB_ERROR_INVALID_ARGUMENT
    assert m.mhcpb_rmsnorm_backward(0, 512, None, None, f.addr["w"], 0, None, None, None,
                                    f.addr["w"] + 512, None, 0, 0, check=False) == \
        m.MHCPB_ERROR_OVERLAP
