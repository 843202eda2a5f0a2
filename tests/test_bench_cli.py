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
    T, K, S = 4096, 20480, 8
    call, k1 = bench.algorithmic_bytes(T, K, S, False)
    x, dx = T * K * 4, T * K * 2
    small = 24 * K * 4 + 24 * T * 4 + 2 * T * 4   # W, P columns 0..23, grad_r and r
    slabs = S * 24 * K * 4
    assert k1 == x + dx + small + slabs == 521437184
    assert call == k1 + slabs + 24 * K * 4 == 539131904
    call_a, k1_a = bench.algorithmic_bytes(T, K, S, True)
    assert k1_a - k1 == T * K * 2 and call_a - call == T * K * 2   # the BF16 addend


def test_forward_and_rmsnorm_bytes():
    call, k1, io = bench.forward_bytes(4096, 20480)
    assert io == 4096 * 20480 * 4 + 24 * 20480 * 4 + 4096 * 32 * 4 + 4096 * 4
    assert call > k1 > 4096 * 20480 * 4
    S = bench.rms_schedule(4096, 5120)
    call, k1, io = bench.rms_bytes(4096, 5120, False, False)
    assert io == 4096 * 5120 * 2 * 3 + 5120 * 2 + 4096 * 4 + 5120 * 4
    assert call == io + 2 * S * 5120 * 4
