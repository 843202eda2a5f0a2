"""The benchmark on the GPU: one short run of ``bench.py`` in a child process,
and its JSON line checked against the contract it promises (one GPU, the
stage's algorithmic bytes over the timed time per call, a kernel-1 roofline
whose figures agree with each other and fit inside the call, and the FP64
oracle timed on the host as the CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_on_the_gpu():
    cmd = [sys.executable, "bench.py", "--gpus", "1", "--steps", "5", "--warmup", "2"]
    print("running:", " ".join(cmd), flush=True)
    run = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, run.stderr[-3000:]
    lines = [ln for ln in run.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, run.stdout[-3000:]
    d = json.loads(lines[0])

    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["unit"] == "GB/s"
    cfg = d["config"]
    assert cfg["T"] == 4096 and cfg["K"] == 20480 and cfg["splits"] == 8
    assert cfg["partial_slabs_moved"] == 7

    # value = algorithmic bytes per call / time per call
    us = d["us_per_call"]
    assert us > 0 and abs(d["ms_per_step"] * 1e3 - us) <= 0.01 * us
    assert abs(d["value"] - cfg["bytes_per_call"] / (us * 1e3)) <= 0.01 * d["value"]

    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    if rf["frac"] is not None:
        # kernel 1 alone: its bytes over its event-timed duration, inside the call
        assert abs(rf["achieved"] - rf["bytes_per_launch"] / (rf["kernel_us_mean"] * 1e3)) \
            <= 0.01 * rf["achieved"]
        assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) <= 1e-3
        assert cfg["k1_us"] + cfg["k2_us"] <= 1.02 * us
        assert 0.3 < rf["frac"] < 1.0

    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert cb["sample"]
