"""Results do not depend on how many CUs run the kernels: the split count
and every sum's order are functions of the shape alone ("DSv4.1 mHC
projection/RMS backward", introduction: a fixed reduction order; the
FlashInfer RMSNorm page's notes describe the opposite, a dw whose bits change
with the SM count).  A child process runs the stage (tiny and supported
profiles), the forward map and the RMSNorm backward once on the whole GPU and
once with HSA_CU_MASK limiting it to 128 of its 256 CUs; every output bit must
agree.  The masked run must also be visibly slower at the supported profile,
which shows that the mask took effect."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = os.path.join(ROOT, "tests", "cu_mask_child.py")


def _child(mask):
    env = dict(os.environ)
    env.pop("HSA_CU_MASK", None)
    if mask:
        env["HSA_CU_MASK"] = mask
    print(f"child run, HSA_CU_MASK={mask}", flush=True)
    res = subprocess.run([sys.executable, CHILD], env=env, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    return json.loads(res.stdout.strip().splitlines()[-1])


def test_outputs_identical_on_half_the_cus():
    full = _child(None)
    half = _child("0:0-127")
    print(f"kernel 1 at train: {full['train_k1_us']:.1f} us on the whole GPU, "
          f"{half['train_k1_us']:.1f} us on half of it", flush=True)
    assert half["train_k1_us"] > 1.3 * full["train_k1_us"], "the CU mask did not take effect"
    for key in full:
        if key.endswith("_us"):
            continue
        assert half[key] == full[key], key
