"""Host-side checks of the benchmark's command line (no GPU is touched).

The benchmark measures one GPU: asked for more it must refuse with a message
and a non-zero status before any GPU work, and its byte accounting must
follow the algorithmic byte counts of the three stages."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in (p.stdout + p.stderr)


def test_stage_bytes_at_the_supported_profile():
    T, K = 4096, 20480
    # 7 of the 8 slabs move at this profile (mhcpb_plan_partial_slabs; see
    # tests/test_abi.py).
    call, k1 = bench.algorithmic_bytes(T, K, 7, False)
    x, dx = T * K * 4, T * K * 2
    small = 24 * K * 4 + 24 * T * 4 + 2 * T * 4   # W, P columns 0..23, grad_r and r
    slabs = 7 * 24 * K * 4
    assert k1 == x + dx + small + slabs == 519471104
    assert call == k1 + slabs + 24 * K * 4 == 535199744
    call_a, k1_a = bench.algorithmic_bytes(T, K, 7, True)
    assert k1_a - k1 == T * K * 2 and call_a - call == T * K * 2   # the BF16 addend


def test_forward_and_rmsnorm_bytes():
    call, k1, io = bench.forward_bytes(4096, 20480)
    assert io == 4096 * 20480 * 4 + 24 * 20480 * 4 + 4096 * 32 * 4 + 4096 * 4
    assert call > k1 > 4096 * 20480 * 4
    S = bench.rms_schedule(4096, 5120)
    call, k1, io = bench.rms_bytes(4096, 5120, False, False)
    assert io == 4096 * 5120 * 2 * 3 + 5120 * 2 + 4096 * 4 + 5120 * 4
    assert call == io + 2 * S * 5120 * 4


def test_roofline_refuses_events_that_do_not_fit_the_call():
    # kernel 1 + kernel 2 beyond the measured time per call: no fraction
    r = bench.roofline("k", 521437184, [114.7] * 20, [4.3] * 20, 101.3, None, None)
    assert r["frac"] is None and r["achieved"] is None and "note" in r
    r = bench.roofline("k", 521437184, [88.0] * 20, [4.0] * 20, 93.0, None, 89.9)
    assert abs(r["frac"] - 521437184 / 88.0e-6 / 1e9 / 8000.0) < 1e-4
    assert abs(r["profile_frac"] - 521437184 / 89.9e-6 / 1e9 / 8000.0) < 1e-4


def test_oracle_row_chunks_cover_every_row_once():
    for rows in (1, 7, 64, 2048, 4095):
        for parts in (1, 3, 16, 128):
            chunks = bench._row_chunks(rows, parts)
            covered = [t for a, b in chunks for t in range(a, b)]
            assert covered == list(range(rows)) and len(chunks) <= parts
