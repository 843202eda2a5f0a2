"""Child process of tests/test_cu_mask.py (test infrastructure): runs the
stage (tiny and train workloads), the forward map and the RMSNorm backward
once each on whatever CUs the process may use (the parent sets HSA_CU_MASK
for the masked run), and prints one JSON line with a SHA-256 of every
output's bits and kernel 1's duration at train."""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _digest(t):
    import torch
    raw = t.detach().contiguous().view(-1).view(torch.uint8)
    return hashlib.sha256(raw.cpu().numpy().tobytes()).hexdigest()


def main():
    import torch

    import workloads
    from bench import HipEvents
    from rms_backward_amd import mhcpb_execute_with_events
    from tests import gpu_harness as gh

    out = {}
    for name in ("tiny", "train"):
        wl = workloads.WORKLOADS[name]
        inp = workloads.make(wl, "cuda")
        dx, dw, ws, plan = gh.run(inp)
        out[f"{name}_dx"] = _digest(dx)
        out[f"{name}_dw"] = _digest(dw)
        if name == "train":
            hev = HipEvents()
            times = []
            stream = torch.cuda.current_stream().cuda_stream
            for _ in range(20):
                a, b = hev.create(), hev.create()
                mhcpb_execute_with_events(plan.handle, inp["x"], inp["w"], inp["grad_proj"],
                                          inp["grad_r"], inp["r"], dx, dw, None, ws, ws.numel(),
                                          stream, a, b, None)
                torch.cuda.synchronize()
                times.append(hev.elapsed_ms(a, b) * 1e3)
                hev.destroy(a)
                hev.destroy(b)
            out["train_k1_us"] = sorted(times)[len(times) // 2]
    wl = workloads.custom(4096, 4, 5120, seed=31)
    inp = workloads.forward_inputs(wl, "cuda")
    proj, r, _ = gh.run_forward(inp["x"], inp["w"])
    out["fwd_proj"] = _digest(proj)
    out["fwd_r"] = _digest(r)
    rinp = workloads.rms_inputs(workloads.RMS_WORKLOADS["rms_train"], "cuda")
    rdx, rdw = gh.run_rmsnorm(rinp)
    out["rms_dx"] = _digest(rdx)
    out["rms_dw"] = _digest(rdw)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
