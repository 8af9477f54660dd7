"""Time the 8-GEMM MLIP layer stacks under each dispatch policy.

The policies of "Unlocking Tensor Core Performance for Machine Learning
Interatomic Potentials" (section "BF16x9 on NVIDIA Blackwell GPUs"):
"performant" uses the emulation only where it is predicted to be faster
(EMU_MODE_AUTO), "eager" uses it wherever it applies (EMU_MODE_BF16X9);
"native" never does (EMU_MODE_NATIVE_F32).  BF16X6 is timed beside them.

Per stack and policy it reports the step time two ways:
  wall   - HIP events around the 8 calls issued back to back, what a caller
           that launches eagerly from Python sees (host launch cost included);
  device - the same 8 calls queued behind a GPU spin, so the events time the
           device work alone (what a captured graph or a busy stream sees).

    python3 -m emulated_fp32_matrix_amd.policies [--stacks 2 3 4] [--json out.json]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

POLICIES = {"performant": "AUTO", "eager": "BF16X9", "native": "NATIVE_F32", "bf16x6": "BF16X6"}


def _synth():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import synth

    return synth


def time_stack(stack, reps=5):
    import torch

    import emulated_fp32_matrix_amd as emu

    synth = _synth()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    gemms = synth.gemms(stack)
    tensors = []
    for g in gemms:
        a = torch.from_numpy(synth.make_a(g)).to(dev)
        b = torch.from_numpy(synth.make_b(g)).to(dev)
        tensors.append((g, a, b, torch.empty((g.M, g.N), dtype=torch.float32, device=dev)))
    flops = sum(g.flops for g in gemms)
    choice = {g.name: emu.select_mode(g.M, g.N, g.K, g.trans_a, g.trans_b) for g in gemms}

    def step(mode):
        for g, a, b, c in tensors:
            emu.sgemm(a, b, mode=mode, trans_a=g.trans_a, trans_b=g.trans_b, c=c)

    out = {"stack": stack, "name": synth.CONFIG_NAMES[stack], "gflop": flops / 1e9,
           "auto_choice": choice, "policies": {}}
    for pol, mode in POLICIES.items():
        for _ in range(3):
            step(mode)
        torch.cuda.synchronize()
        walls, devs = [], []
        for r in range(reps):
            for gated in (False, True):
                if gated:
                    torch.cuda._sleep(20_000_000)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                step(mode)
                e1.record(stream)
                torch.cuda.synchronize()
                (devs if gated else walls).append(e0.elapsed_time(e1) * 1e3)
        w, d = statistics.median(walls), statistics.median(devs)
        out["policies"][pol] = {"mode": mode, "wall_us": round(w, 1), "device_us": round(d, 1),
                                "wall_tflops": round(flops / w / 1e6, 2),
                                "device_tflops": round(flops / d / 1e6, 2)}
        print(f"stack {stack} {pol:10s} ({mode:10s}): wall {w:9.1f} us ({flops / w / 1e6:6.1f} TFLOP/s)  "
              f"device {d:9.1f} us ({flops / d / 1e6:6.1f} TFLOP/s)", flush=True)
    del tensors
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stacks", type=int, nargs="+", default=[2, 4, 3])
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--json", default=None)
    args = ap.parse_args()
    res = [time_stack(s, args.reps) for s in args.stacks]
    if args.json:
        json.dump(res, open(args.json, "w"), indent=1)


if __name__ == "__main__":
    main()
