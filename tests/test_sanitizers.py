"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the library's plan and argument validation (mhcpb_plan.cpp, with the
kernel launches replaced by counters: tests/sanitize/plan_checks.cpp) and
the FP64 oracle (oracle/mhcpb_oracle.c, driven by
tests/sanitize/oracle_checks.c).  Both are built with g++/gcc and
-fsanitize=address,undefined (no GPU code is involved) and must run clean."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ROCM_INCLUDE = "/opt/rocm/include"


def _run(cmd, tmp):
    p = subprocess.run(cmd, cwd=tmp, capture_output=True, text=True, timeout=300)
    return p


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def test_plan_validation_under_sanitizers(tmp_path):
    _need("g++")
    if not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("HIP headers not available")
    exe = str(tmp_path / "plan_checks")
    build = _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, *SAN,
                  os.path.join(ROOT, "tests", "sanitize", "plan_checks.cpp"),
                  os.path.join(ROOT, "rms_backward_amd", "csrc", "mhcpb_plan.cpp"),
                  "-o", exe], tmp_path)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("MHCPB_WAIT_POLLS", None)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-3000:]
    assert "plan checks passed" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_checks")
    build = _run(["gcc", "-std=c11", *SAN, "-ffp-contract=off",
                  os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"),
                  os.path.join(ROOT, "oracle", "mhcpb_oracle.c"), "-lm", "-o", exe], tmp_path)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-3000:]
    assert "oracle checks passed" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out
