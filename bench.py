"""Benchmark of the DSv4.1 mHC projection/RMS backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train]
                    [--stage backward|forward|rmsnorm] [--form fused|split]

One step is one call of mhcpb_execute (kernel 1 + kernel 2) on the synthetic
workload, with every input already resident in HBM.  Prints ONE JSON line:
microseconds per call, achieved GB/s of algorithmic bytes (value), the
roofline of the dominant kernel (kernel 1) and the CPU oracle timed on a
bounded sample of the same workload over the host's cores.

Timing.  The library's code object is loaded first (one call on a 16-token
problem).  Before the warm-up the GPU then runs about 300 ms of BF16 matrix
products on scratch matrices (torch, none of the library's kernels, inputs or
outputs): after an idle spell the GPU's power management slows calls 10 to
150 by up to 35 % (measured on the box: a transient after idle, gone after a
few tens of milliseconds of compute-heavy work, such as the GEMMs that
surround this stage in a training step), and the settle takes the device out
of it without running extra steps of the path.  Then W warm-up calls and
exactly K timed calls back to back on one stream, bracketed by events.  The
roofline's kernel-1 duration comes from an event pass right after the timed
calls (at least 100 more calls, each with HIP events the library attaches to
its two dispatches): attaching events to a call costs about 4 us per call
(measured), so the timed calls run without them; the fraction is reported
only if kernel 1 and kernel 2 of that pass fit in the timed time per call.

Algorithmic bytes per call (T tokens, K columns, S splits):
    X T*K*4 + dX T*K*2 [+ addend T*K*2] + W 24*K*4 + P 24*T*4 + grad_r, r 2*T*4
    + partial dW slabs written and read 2*S*24*K*4 + dW 24*K*4
Kernel 1 moves everything but the slab reads and the dW write.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0
METRIC = "µs/call and achieved HBM GB/s (% of peak) at T=4096, K=4×5120"
KERNEL_SOURCES = [os.path.join(ROOT, "rms_backward_amd", "csrc", n)
                  for n in ("mhcpb_kernels.hip", "mhcpb_device.h")]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "projection_train_counters.json")
TRACE_FILE = os.path.join(ROOT, "profiles", "projection_train_kernel_stats.json")
SETTLE_MS = 300.0


def algorithmic_bytes(T: int, K: int, moved: int, addend: bool) -> tuple[int, int]:
    """(whole call, kernel 1) algorithmic bytes: X read and dX written once
    (and the addend read), W, P, grad_r and r read, the `moved` partial slabs
    (mhcpb_plan_partial_slabs) written by kernel 1 and read by kernel 2, and
    dW written."""
    big = T * K * 4 + T * K * 2 + (T * K * 2 if addend else 0)
    small = 24 * K * 4 + 24 * T * 4 + 2 * T * 4
    slabs = moved * 24 * K * 4
    k1 = big + small + slabs
    call = k1 + slabs + 24 * K * 4
    return call, k1


def cycling(calls_ev):
    """Given one call (taking three event handles) per buffer set, returns
    (call_ev, call) that go through the sets in turn."""
    state = [0]

    def call_ev(a, b, c):
        f = calls_ev[state[0] % len(calls_ev)]
        state[0] += 1
        return f(a, b, c)

    return call_ev, (lambda: call_ev(None, None, None))


INFINITY_CACHE_BYTES = 256 << 20


def buffer_sets(requested: int, set_bytes: int) -> int:
    """Buffer sets the calls cycle through: `requested`, or by default (0) as
    many as make the sets' large buffers at least twice the 256 MB Infinity
    Cache (two at least), so that no call finds data of an earlier call in
    that cache."""
    if requested > 0:
        return requested
    return max(2, -(-2 * INFINITY_CACHE_BYTES // max(1, set_bytes)))


def buffer_sets_note(n: int, set_bytes: int) -> str:
    if n <= 1:
        return "one set of inputs and outputs, the same buffers every call"
    return (f"the calls cycle through {n} copies of the large inputs and outputs "
            f"({n * set_bytes / 1e6:.0f} MB in all), so that no call finds the data of an "
            f"earlier call in the 256 MB Infinity Cache")


def source_hash(paths) -> str:
    """Hash of kernel sources with comments, blank lines and trailing spaces
    removed: it changes with the code, not with its comments."""
    text = ""
    for path in paths:
        with open(path, encoding="utf-8") as f:
            text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def kernel_source_hash() -> str:
    return source_hash(KERNEL_SOURCES)


def _profile_record(path: str, workload: str, sha: str):
    """A committed profile summary (JSON) taken on the current kernel source
    and workload, else None."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != sha or rec.get("workload") != workload:
        return None
    return rec


def measured_traffic(workload: str):
    """HBM bytes per kernel-1 launch from the committed counter summary, if it
    was taken on the current kernel source; otherwise None."""
    rec = _profile_record(COUNTERS_FILE, workload, kernel_source_hash())
    return rec.get("hbm_bytes_per_launch") if rec else None


def profiled_kernel1_us(workload: str):
    """Kernel 1's average duration in the committed rocprofv3 kernel trace of
    the current source, in microseconds, if there is one; otherwise None."""
    rec = _profile_record(TRACE_FILE, workload, kernel_source_hash())
    return rec.get("kernel1_avg_us") if rec else None


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        h = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return h.value

    def elapsed_ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def destroy(self, h: int):
        self.lib.hipEventDestroy(h)


def device_settle(ms: float) -> dict:
    """About `ms` milliseconds of BF16 matrix products on scratch matrices
    (none of the library's kernels, inputs or outputs), so that the timed
    calls do not start inside the GPU's power-management transient after
    idle (fills of memory alone leave about a third of it)."""
    import torch
    if ms <= 0:
        return {"ms": 0}
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    c = a @ a  # the GEMM library's own start-up, outside the settle time
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < ms / 1e3:
        c = a @ a
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) * 1e3
    del a, c
    return {"ms": round(dt, 1), "bf16_gemms_8192": n}


def load_kernels(stage: str):
    """One call of the stage's entry point on a 16-token problem, so that the
    runtime loads the library's code object on the GPU before the settle (the
    load happens at a module's first launch and takes tens of milliseconds,
    long enough for the GPU to leave the state the settle put it in)."""
    import torch
    import workloads
    from tests import gpu_harness as gh
    if stage == "rmsnorm":
        gh.run_rmsnorm(workloads.rms_inputs(workloads.rms_custom(16, 64), "cuda"))
    elif stage == "forward":
        inp = workloads.forward_inputs(workloads.custom(16, 4, 16), "cuda")
        gh.run_forward(inp["x"], inp["w"])
    else:
        gh.run(workloads.make(workloads.custom(16, 4, 16), "cuda"))
    torch.cuda.synchronize()


def timed_calls(call, steps: int):
    """Exactly `steps` calls back to back on the current stream, bracketed by
    torch events; returns (µs per call, wall seconds)."""
    import torch
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps, time.perf_counter() - t0


def event_pass(call_with_events, calls: int):
    """`calls` calls, each with three HIP events attached to its dispatches by
    the library (kernel 1 start, kernel 1 end, kernel 2 end); returns the
    kernel-1 and kernel-2 (with the gap before it) durations in µs."""
    import torch
    hev = HipEvents()
    evs = [(hev.create(), hev.create(), hev.create()) for _ in range(calls)]
    torch.cuda.synchronize()
    for a, b, c in evs:
        call_with_events(a, b, c)
    torch.cuda.synchronize()
    k1 = [hev.elapsed_ms(a, b) * 1e3 for a, b, _ in evs]
    k2 = [hev.elapsed_ms(b, c) * 1e3 for _, b, c in evs]
    for trio in evs:
        for e in trio:
            hev.destroy(e)
    return k1, k2


def _median(v):
    s = sorted(v)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def roofline(kernel: str, bytes_per_launch: int, k1: list, k2: list, us_per_call: float,
             traffic, profile_us) -> dict:
    """Roofline object of kernel 1 from its durations in the event pass.  A
    fraction is only reported when kernel 1 and kernel 2 fit in the timed
    time per call (durations that do not fit are not evidence)."""
    k1_mean = sum(k1) / len(k1)
    k2_mean = sum(k2) / len(k2)
    consistent = k1_mean + k2_mean <= us_per_call * 1.02
    achieved = bytes_per_launch / (k1_mean * 1e-6) / 1e9
    out = {
        "bound": "hbm",
        "achieved": round(achieved, 2) if consistent else None,
        "peak": PEAK_HBM_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBPS, 4) if consistent else None,
        "traffic": traffic,
        "kernel": kernel,
        "bytes_per_launch": bytes_per_launch,
        "kernel_us_mean": round(k1_mean, 2),
        "kernel_us_median": round(_median(k1), 2),
        "timing": (f"HIP events attached by the library to the kernel's dispatch, mean over "
                   f"the {len(k1)} calls of the event pass after the timed calls"),
    }
    if not consistent:
        out["note"] = (f"kernel 1 + kernel 2 ({k1_mean + k2_mean:.2f} us) exceed the time per "
                       f"call ({us_per_call:.2f} us): no fraction reported")
    if profile_us:
        out["profile_kernel_us"] = profile_us
        out["profile_frac"] = round(bytes_per_launch / (profile_us * 1e-6) / 1e9 /
                                    PEAK_HBM_GBPS, 4)
    return out


def _oracle_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def threaded_oracle(work, chunks, threads: int) -> float:
    """Run work(chunk) for every chunk on `threads` host threads (the oracle's
    C calls release the GIL); returns the wall seconds."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for f in [ex.submit(work, c) for c in chunks]:
            f.result()
    return time.perf_counter() - t0


def _row_chunks(rows: int, parts: int):
    step = -(-rows // parts)
    return [(a, min(rows, a + step)) for a in range(0, rows, step)]


def cpu_baseline(inp, rows: int, T: int, K: int, moved: int, addend: bool):
    """Time the FP64 oracle (as it is) on the first `rows` rows of the
    workload, dX rows and their dW contribution, on every host core the
    process may use (one thread per core, rows split into equal chunks);
    also one thread on a slice, for the per-core rate."""
    import oracle
    from tests import gpu_harness as gh

    rows = min(rows, T)
    h = gh.host_rows(inp, list(range(rows)))

    def work(span):
        a, b = span
        ad = h["addend"][a:b] if h["addend"] is not None else None
        oracle.dx(h["x"][a:b], h["w"], h["grad_proj"][a:b], h["grad_r"][a:b], h["r"][a:b], K,
                  addend=ad, mode="tf32")
        oracle.dw(h["x"][a:b], h["grad_proj"][a:b], mode="tf32")

    one_rows = min(rows, 64)
    dt1 = threaded_oracle(work, [(0, one_rows)], 1)
    cores = _oracle_threads()
    dt = threaded_oracle(work, _row_chunks(rows, cores), cores)
    call_bytes, _ = algorithmic_bytes(T, K, moved, addend)
    return {
        "value": round(call_bytes * (rows / T) / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"first {rows} of {T} rows, all {K} columns: dX rows and their dW "
                   f"contribution, TF32-mode FP64 oracle, {cores} threads (one per core of "
                   f"the process's CPU affinity) on equal row chunks, {dt:.2f} s; one thread on "
                   f"{one_rows} rows: {dt1:.2f} s"),
        "one_thread_value": round(call_bytes * (one_rows / T) / dt1 / 1e9, 6),
        "us_per_call_extrapolated": round(dt / (rows / T) * 1e6, 1),
    }


def split_bytes(T: int, K: int, moved: int, addend: bool) -> tuple[int, int]:
    """Algorithmic bytes of (mhcpb_execute_dx, mhcpb_execute_dw) calls."""
    dx = T * K * 4 + T * K * 2 + (T * K * 2 if addend else 0) + 24 * K * 4 + 24 * T * 4 + 2 * T * 4
    dw = T * K * 4 + 24 * T * 4 + 2 * moved * 24 * K * 4 + 24 * K * 4
    return dx, dw


def run_split(args, wl, inp, plan, S, dx, dw, ws, settle) -> dict:
    """The split form: per step the dX-only call then the dW-only call."""
    import torch
    from rms_backward_amd import mhcpb_execute_dw, mhcpb_execute_dx, mhcpb_plan_partial_slabs
    T, K = wl.T, wl.K
    stream = torch.cuda.current_stream()
    h = plan.handle
    call_dx = lambda: mhcpb_execute_dx(h, inp["x"], inp["w"], inp["grad_proj"], inp["grad_r"],
                                       inp["r"], dx, inp.get("addend"), stream.cuda_stream)
    call_dw = lambda: mhcpb_execute_dw(h, inp["x"], inp["grad_proj"], dw, ws, ws.numel(),
                                       stream.cuda_stream)

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    for _ in range(args.warmup):
        call_dx()
        call_dw()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    us_per_step = timed(lambda: (call_dx(), call_dw()), args.steps)
    wall = time.perf_counter() - t0
    dx_us = timed(call_dx, args.steps)
    dw_us = timed(call_dw, args.steps)
    dx_bytes, dw_bytes = split_bytes(T, K, mhcpb_plan_partial_slabs(plan.handle), wl.addend)
    gbps = (dx_bytes + dw_bytes) / (us_per_step * 1e-6) / 1e9
    dx_gbps = dx_bytes / (dx_us * 1e-6) / 1e9
    return {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_step / 1e3, 6),
        "us_per_call": round(us_per_step, 2),
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "tf32",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name}: T={T} tokens, {wl.streams} streams x hidden "
                         f"{wl.hidden} (K={K}); split form (dX call, then dW call)"
                         + (", BF16 addend" if wl.addend else "")),
            "form": "split", "T": T, "K": K, "splits": S,
            "buffer_sets": 1, "buffers": buffer_sets_note(1, 0),
            "bytes_per_step": dx_bytes + dw_bytes,
            "dx_call_bytes": dx_bytes, "dw_call_bytes": dw_bytes,
            "dx_call_us": round(dx_us, 2), "dw_call_us": round(dw_us, 2),
            "timed_wall_s": round(wall, 4),
            "device_settle": settle,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(dx_gbps, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(dx_gbps / PEAK_HBM_GBPS, 4),
            "traffic": None,
            "kernel": "projection, dX-only form (one kernel per call, timed over the calls)",
            "bytes_per_launch": dx_bytes,
        },
    }


FORWARD_METRIC = ("forward map: µs/call and achieved HBM GB/s (% of peak) at "
                  "T=4096, K=4×5120")
FORWARD_SOURCES = [os.path.join(ROOT, "rms_backward_amd", "csrc", n)
                   for n in ("mhcpb_forward.hip", "mhcpb_device.h")]
FORWARD_COUNTERS_FILE = os.path.join(ROOT, "profiles", "forward_train_counters.json")
FORWARD_TRACE_FILE = os.path.join(ROOT, "profiles", "forward_train_kernel_stats.json")


def forward_bytes(T: int, K: int) -> tuple[int, int, int]:
    """(whole call, kernel 1, partial-free) algorithmic bytes of the forward
    map: X and W read once, proj [T, 32] and r written, and the partials of
    the 1024-column tiles (24 logits, a sum of squares and padding, 32 floats
    per tile and token) written by kernel 1 and read by kernel 2."""
    tiles = (K + 1023) // 1024
    partials = tiles * ((T + 15) // 16) * 16 * 32 * 4
    io = T * K * 4 + 24 * K * 4 + T * 32 * 4 + T * 4
    k1 = T * K * 4 + 24 * K * 4 + partials
    return io + 2 * partials, k1, io


def forward_source_hash() -> str:
    return source_hash(FORWARD_SOURCES)


def forward_cpu_baseline(x, w, rows: int, T: int, K: int):
    """Time the FP64 oracle's forward (as it is) on `rows` rows over the
    host's cores (equal row chunks), and one thread on a slice."""
    import oracle
    rows = min(rows, T)
    xs = x[:rows].cpu().numpy()
    ws = w.cpu().numpy()
    work = lambda span: oracle.forward(xs[span[0]:span[1]], ws, eps=1e-6, mode="tf32")
    one_rows = min(rows, 64)
    dt1 = threaded_oracle(work, [(0, one_rows)], 1)
    cores = _oracle_threads()
    dt = threaded_oracle(work, _row_chunks(rows, cores), cores)
    call_bytes, _, _ = forward_bytes(T, K)
    return {
        "value": round(call_bytes * (rows / T) / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"first {rows} of {T} rows, all {K} columns: proj and r, TF32-mode FP64 "
                   f"oracle, {cores} threads on equal row chunks, {dt:.2f} s; one thread on "
                   f"{one_rows} rows: {dt1:.2f} s"),
        "one_thread_value": round(call_bytes * (one_rows / T) / dt1 / 1e9, 6),
        "us_per_call_extrapolated": round(dt / (rows / T) * 1e6, 1),
    }


def run_forward(args, wl, settle) -> dict:
    """The forward map: per step one mhcpb_forward call (the pass over X,
    then the sum of the tiles' partials)."""
    import torch
    import workloads
    from rms_backward_amd import mhcpb_forward_with_events
    from rms_backward_amd.wrapper import Plan

    T, K = wl.T, wl.K
    inp = workloads.forward_inputs(wl, "cuda")
    x, w = inp["x"], inp["w"]
    plan = Plan(T, wl.streams, wl.hidden)
    proj = torch.full((T, 32), float("nan"), dtype=torch.float32, device="cuda")
    r = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    ws = plan.alloc_forward_workspace("cuda")
    eps = 1e-6
    stream = torch.cuda.current_stream()
    set_bytes = T * K * 4
    n_sets = buffer_sets(args.buffer_sets, set_bytes)
    xsets = [x] + [x.clone() for _ in range(n_sets - 1)]
    call_ev, call = cycling([
        (lambda a, b, c, xs=xs: mhcpb_forward_with_events(plan.handle, xs, w, eps, proj, r, ws,
                                                          ws.numel(), stream.cuda_stream, a, b, c))
        for xs in xsets])
    load_kernels(args.stage)
    settle.update(device_settle(SETTLE_MS if not args.no_settle else 0))
    for _ in range(args.warmup):
        call()
    us_per_call, wall = timed_calls(call, args.steps)
    k1, k2 = event_pass(call_ev, max(args.steps, 100))
    call_bytes, k1_bytes, io_bytes = forward_bytes(T, K)
    gbps = call_bytes / (us_per_call * 1e-6) / 1e9
    sha = forward_source_hash()
    rec_c = _profile_record(FORWARD_COUNTERS_FILE, wl.name, sha)
    rec_t = _profile_record(FORWARD_TRACE_FILE, wl.name, sha)
    return {
        "metric": FORWARD_METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_call / 1e3, 6),
        "us_per_call": round(us_per_call, 2),
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "tf32",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name} forward: T={T} tokens, {wl.streams} streams x hidden "
                         f"{wl.hidden} (K={K}); X, W FP32 in, proj [T, 32] and r FP32 out"),
            "stage": "forward", "T": T, "K": K,
            "buffer_sets": n_sets, "buffers": buffer_sets_note(n_sets, set_bytes),
            "bytes_per_call": call_bytes,
            "bytes_per_call_without_partials": io_bytes,
            "k1_us": round(sum(k1) / len(k1), 2), "k2_us": round(sum(k2) / len(k2), 2),
            "timed_wall_s": round(wall, 4),
            "device_settle": settle,
        },
        "roofline": roofline("forward pass over X (forward_tiles, kernel 1)", k1_bytes, k1, k2,
                             us_per_call, rec_c.get("hbm_bytes_per_launch") if rec_c else None,
                             rec_t.get("kernel1_avg_us") if rec_t else None),
        "_inputs": (x, w),
    }


RMS_METRIC = ("BF16 RMSNorm backward: µs/call and achieved HBM GB/s (% of peak) at "
              "T=4096, H=5120")
RMS_SOURCES = [os.path.join(ROOT, "rms_backward_amd", "csrc", n)
               for n in ("mhcpb_rmsnorm.hip", "mhcpb_device.h")]
RMS_COUNTERS_FILE = os.path.join(ROOT, "profiles", "rmsnorm_train_counters.json")
RMS_TRACE_FILE = os.path.join(ROOT, "profiles", "rmsnorm_train_kernel_stats.json")


def rms_schedule(T: int, H: int) -> int:
    """Blocks S of the RMSNorm backward (a function of T and H only)."""
    if T == 0:
        return 0
    nc = -(-H // 512)
    return min(-(-T // 16), 256 * max(1, 12 // nc))


def rms_bytes(T: int, H: int, w_f32: bool, residual: bool) -> tuple[int, int, int]:
    """(whole call, kernel 1, partial-free) algorithmic bytes of the RMSNorm
    backward: g, x (and g_residual) read and dx written once (BF16), w and
    rstd read, dw written, and the S block partials of dw written by kernel 1
    and read by kernel 2."""
    S = rms_schedule(T, H)
    rows = T * H * 2 * (3 + (1 if residual else 0))
    small = H * (4 if w_f32 else 2) + T * 4
    partials = S * H * 4
    io = rows + small + H * 4
    return io + 2 * partials, rows + small + partials, io


def rms_source_hash() -> str:
    return source_hash(RMS_SOURCES)


def rms_cpu_baseline(inp, wl, min_seconds: float = 2.0):
    """Time the FP64 oracle (as it is) on the whole workload over the host's
    cores (equal row chunks), repeated until at least `min_seconds` have
    passed, and one thread on one call."""
    import oracle
    from tests import gpu_harness as gh
    g = gh.bf16_bits_np(inp["g"])
    x = gh.bf16_bits_np(inp["x"])
    w = inp["w"].float().cpu().numpy()
    rstd = inp["rstd"].cpu().numpy()
    res = gh.bf16_bits_np(inp["res"]) if inp.get("res") is not None else None

    def work(span):
        a, b = span
        oracle.rmsnorm_backward(g[a:b], x[a:b], w, rstd[a:b],
                                res_bits=res[a:b] if res is not None else None)

    dt1 = threaded_oracle(work, [(0, wl.T)], 1)
    cores = _oracle_threads()
    chunks = _row_chunks(wl.T, cores)
    reps = 0
    dt = 0.0
    while dt < min_seconds:
        dt += threaded_oracle(work, chunks, cores)
        reps += 1
    call_bytes, _, _ = rms_bytes(wl.T, wl.H, wl.w_f32, wl.residual)
    return {
        "value": round(call_bytes * reps / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"the whole workload (all {wl.T} rows, dx and dw), FP64 oracle, {cores} "
                   f"threads on equal row chunks, {reps} call(s) in {dt:.2f} s; one thread: "
                   f"{dt1:.2f} s per call"),
        "one_thread_value": round(call_bytes / dt1 / 1e9, 6),
        "us_per_call_extrapolated": round(dt / reps * 1e6, 1),
    }


def run_rmsnorm(args, wl, settle) -> dict:
    """The second workload: per step one mhcpb_rmsnorm_backward call (the rows
    kernel, then the fixed-order sum of the block partials)."""
    import torch
    import workloads
    import rms_backward_amd as m

    T, H = wl.T, wl.H
    inp = workloads.rms_inputs(wl, "cuda")
    dx = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((H,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, m.mhcpb_rmsnorm_backward_workspace_bytes(T, H)), dtype=torch.uint8,
                     device="cuda")
    wd = m.MHCPB_DTYPE_F32 if wl.w_f32 else m.MHCPB_DTYPE_BF16
    sh = torch.cuda.current_stream().cuda_stream
    set_bytes = T * H * 2 * (3 + (1 if wl.residual else 0))
    n_sets = buffer_sets(args.buffer_sets, set_bytes)
    sets = [(inp["g"], inp["x"], inp["res"], dx)]
    for _ in range(n_sets - 1):
        sets.append((inp["g"].clone(), inp["x"].clone(),
                     inp["res"].clone() if inp["res"] is not None else None, torch.empty_like(dx)))
    call_ev, call = cycling([
        (lambda a, b, c, g=g, xs=xs, res=res, dxs=dxs: m.mhcpb_rmsnorm_backward_with_events(
            T, H, g, xs, inp["w"], wd, inp["rstd"], res, dxs, dw, ws, ws.numel(), sh, a, b, c))
        for g, xs, res, dxs in sets])
    load_kernels(args.stage)
    settle.update(device_settle(SETTLE_MS if not args.no_settle else 0))
    for _ in range(args.warmup):
        call()
    us_per_call, wall = timed_calls(call, args.steps)
    k1, k2 = event_pass(call_ev, max(args.steps, 100))
    S = rms_schedule(T, H)
    call_bytes, k1_bytes, io_bytes = rms_bytes(T, H, wl.w_f32, wl.residual)
    gbps = call_bytes / (us_per_call * 1e-6) / 1e9
    sha = rms_source_hash()
    rec_c = _profile_record(RMS_COUNTERS_FILE, wl.name, sha)
    rec_t = _profile_record(RMS_TRACE_FILE, wl.name, sha)
    return {
        "metric": RMS_METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_call / 1e3, 6),
        "us_per_call": round(us_per_call, 2),
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name} RMSNorm backward: T={T} rows, H={H}; g, x BF16, w "
                         f"{'FP32' if wl.w_f32 else 'BF16'}, rstd FP32"
                         + (", g_residual BF16" if wl.residual else "")
                         + "; dx BF16, dw FP32"),
            "stage": "rmsnorm", "T": T, "H": H, "blocks": S,
            "buffer_sets": n_sets, "buffers": buffer_sets_note(n_sets, set_bytes),
            "bytes_per_call": call_bytes,
            "bytes_per_call_without_partials": io_bytes,
            "k1_us": round(sum(k1) / len(k1), 2), "k2_us": round(sum(k2) / len(k2), 2),
            "timed_wall_s": round(wall, 4),
            "device_settle": settle,
        },
        "roofline": roofline("RMSNorm backward rows (rmsnorm_bwd_rows, kernel 1)", k1_bytes, k1,
                             k2, us_per_call,
                             rec_c.get("hbm_bytes_per_launch") if rec_c else None,
                             rec_t.get("kernel1_avg_us") if rec_t else None),
        "_inputs": inp,
    }


def run_copy_calibration(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def workload_by_name(name: str):
    """A workload of the stage named T<T>_s4_h<hidden> (the naming of
    workloads.custom), beside the named ones."""
    import re
    import workloads
    m = re.fullmatch(r"T(\d+)_s4_h(\d+)", name)
    if not m:
        raise SystemExit(f"bench.py: unknown workload {name!r}")
    return workloads.custom(int(m.group(1)), 4, int(m.group(2)))


def rms_workload_by_name(name: str):
    """An RMSNorm workload named rms_T<T>_H<H> (workloads.rms_custom)."""
    import re
    import workloads
    m = re.fullmatch(r"rms_T(\d+)_H(\d+)", name)
    if not m:
        raise SystemExit(f"bench.py: unknown RMSNorm workload {name!r}")
    return workloads.rms_custom(int(m.group(1)), int(m.group(2)))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed calls before the timed ones (default: about 50 ms of "
                         "calls: 500 for the stage, 600 for the forward, 2000 for the RMSNorm "
                         "backward)")
    ap.add_argument("--workload", default="train")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="rows of the workload the CPU oracle baseline times")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--buffer-sets", type=int, default=0,
                    help="copies of the large inputs and outputs the calls cycle through (1: "
                         "the same buffers every call; default: enough that they total twice "
                         "the 256 MB Infinity Cache, at least 2)")
    ap.add_argument("--no-settle", action="store_true",
                    help="skip the ~300 ms of BF16 matrix products before the warm-up")
    ap.add_argument("--form", choices=("fused", "split"), default="fused",
                    help="fused: mhcpb_execute per step; split: mhcpb_execute_dx then "
                         "mhcpb_execute_dw per step (X read twice)")
    ap.add_argument("--stage", choices=("backward", "forward", "rmsnorm"), default="backward",
                    help="backward: the stage (default); forward: the map it differentiates "
                         "(mhcpb_forward: proj = X W^T and r per step); rmsnorm: the BF16 "
                         "RMSNorm backward (workloads rms_*, default rms_train)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (counter scaling)")
    args = ap.parse_args(argv)
    if args.warmup is None:
        args.warmup = {"backward": 500, "forward": 600, "rmsnorm": 2000}[args.stage]

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs on one GPU and is measured on one GPU only; "
              "--gpus must be 1", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        run_copy_calibration(args.copy_calibration, max(1, args.steps))
        return 0

    import workloads
    from rms_backward_amd import (mhcpb_execute_with_events, mhcpb_plan_partial_slabs,
                                  mhcpb_plan_split_count)
    from rms_backward_amd.wrapper import Plan
    from tests import gpu_harness as gh

    settle = {}
    if args.stage == "rmsnorm":
        name = "rms_train" if args.workload == "train" else args.workload
        wl = workloads.RMS_WORKLOADS.get(name) or rms_workload_by_name(name)
        print(f"bench: workload {wl.name} T={wl.T} H={wl.H} stage rmsnorm", file=sys.stderr,
              flush=True)
        out = run_rmsnorm(args, wl, settle)
        inp = out.pop("_inputs")
        if not args.no_cpu_baseline:
            print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
            out["cpu_baseline"] = rms_cpu_baseline(inp, wl)
        else:
            out["cpu_baseline"] = None
        print(json.dumps(out), flush=True)
        return 0

    wl = workloads.WORKLOADS.get(args.workload) or workload_by_name(args.workload)
    T, K = wl.T, wl.K
    print(f"bench: workload {wl.name} T={T} K={K} stage {args.stage}", file=sys.stderr,
          flush=True)
    if args.stage == "forward":
        out = run_forward(args, wl, settle)
        x, w = out.pop("_inputs")
        if not args.no_cpu_baseline:
            print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
            out["cpu_baseline"] = forward_cpu_baseline(x, w, args.cpu_rows, T, K)
        else:
            out["cpu_baseline"] = None
        print(json.dumps(out), flush=True)
        return 0
    inp = workloads.make(wl, "cuda")
    plan = Plan(T, wl.streams, wl.hidden)
    S = mhcpb_plan_split_count(plan.handle)
    dx, dw, ws = gh.alloc_outputs(T, K, plan, "cuda", poison=True)
    if args.form == "split":
        load_kernels(args.stage)
        settle.update(device_settle(SETTLE_MS if not args.no_settle else 0))
        out = run_split(args, wl, inp, plan, S, dx, dw, ws, settle)
        if not args.no_cpu_baseline:
            print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
            out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows, T, K, mhcpb_plan_partial_slabs(plan.handle),
                                          wl.addend)
        else:
            out["cpu_baseline"] = None
        print(json.dumps(out), flush=True)
        return 0
    stream = torch.cuda.current_stream()
    set_bytes = T * K * 4 + T * K * 2 + (T * K * 2 if wl.addend else 0)
    n_sets = buffer_sets(args.buffer_sets, set_bytes)
    sets = [(inp["x"], inp.get("addend"), dx)]
    for _ in range(n_sets - 1):
        ad = inp.get("addend")
        sets.append((inp["x"].clone(), ad.clone() if ad is not None else None,
                     torch.empty_like(dx)))
    call_ev, call = cycling([
        (lambda a, b, c, xs=xs, ad=ad, dxs=dxs: mhcpb_execute_with_events(
            plan.handle, xs, inp["w"], inp["grad_proj"], inp["grad_r"], inp["r"], dxs, dw,
            ad, ws, ws.numel(), stream.cuda_stream, a, b, c))
        for xs, ad, dxs in sets])
    load_kernels(args.stage)
    settle.update(device_settle(SETTLE_MS if not args.no_settle else 0))
    for _ in range(args.warmup):
        call()
    # timed region: exactly `steps` calls
    us_per_call, wall = timed_calls(call, args.steps)
    # kernel durations: the event pass right after
    k1, k2 = event_pass(call_ev, max(args.steps, 100))

    moved = mhcpb_plan_partial_slabs(plan.handle)
    call_bytes, k1_bytes = algorithmic_bytes(T, K, moved, wl.addend)
    gbps = call_bytes / (us_per_call * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_call / 1e3, 6),
        "us_per_call": round(us_per_call, 2),
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "tf32",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name}: T={T} tokens, {wl.streams} streams x hidden "
                         f"{wl.hidden} (K={K}); X/W/grad_proj/grad_r/r FP32, dX BF16, "
                         f"dW FP32" + (", BF16 addend" if wl.addend else "")),
            "T": T, "K": K, "splits": S,
            "partial_slabs_moved": moved,
            "buffer_sets": n_sets, "buffers": buffer_sets_note(n_sets, set_bytes),
            "bytes_per_call": call_bytes,
            "bytes_per_call_without_partials": call_bytes - 2 * moved * 24 * K * 4,
            "k1_us": round(sum(k1) / len(k1), 2), "k2_us": round(sum(k2) / len(k2), 2),
            "timed_wall_s": round(wall, 4),
            "device_settle": settle,
        },
        "roofline": roofline("projection (kernel 1)", k1_bytes, k1, k2, us_per_call,
                             measured_traffic(wl.name), profiled_kernel1_us(wl.name)),
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows, T, K, mhcpb_plan_partial_slabs(plan.handle),
                                          wl.addend)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
