"""Measure the device time of NATIVE_F32 and BF16X9 calls over a set of GEMM
shapes, and fit the cost model that EMU_MODE_AUTO uses to choose between
them (the "performant" policy of "Unlocking Tensor Core Performance for
Machine Learning Interatomic Potentials", section "BF16x9 on NVIDIA
Blackwell GPUs").

Device time, not wall time: each batch of calls is queued behind a GPU spin
(torch.cuda._sleep), so the calls run back to back whatever the host-side
launch cost, and a pair of HIP events around the batch times the device
work of one call (for BF16X9: the B pre-split and the main kernel).

    python3 -m emulated_fp32_matrix_amd.calibrate [--fit] [--out table.json]

Prints one line per shape; with --fit also the least-squares constants of
the model in csrc/emu_api.hip and how often the model picks the faster mode.
"""
from __future__ import annotations

import argparse
import json
import math
import statistics
import sys


def shapes():
    """(M, N, K, trans_b, label): the MLIP layer stacks at 6,144 rows (d = 256
    and 1,024) and 552,960 rows (d = 256), plus squares, skinny shapes and a
    K sweep."""
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import synth

    out = []
    for cfg in (2, 4, 3):
        for g in synth.gemms(cfg):
            out.append((g.M, g.N, g.K, g.trans_b, f"stack{cfg}:{g.name}"))
    for n in (128, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 8192):
        out.append((n, n, n, False, f"square{n}"))
    for M in (1024, 4096, 16384, 65536):
        for N, K in ((64, 64), (128, 128), (256, 64), (64, 256), (512, 512), (2048, 256), (256, 2048)):
            out.append((M, N, K, False, "skinny"))
    for K in (32, 1024, 4096, 16384):
        out.append((2048, 2048, K, False, "k-sweep"))
    return out


def measure(modes=("NATIVE_F32", "BF16X9")):
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    rows = []
    for (M, N, K, tb, label) in shapes():
        a = torch.randn(M, K, device=dev)
        b = torch.randn((N, K) if tb else (K, N), device=dev)
        c = torch.empty(M, N, device=dev)
        reps = max(3, min(50, int(2e11 / (2 * M * N * K))))
        res = {}
        for m in modes:
            for _ in range(2):
                emu.sgemm(a, b, mode=m, trans_b=tb, c=c)
            ts = []
            for _ in range(3):
                torch.cuda._sleep(8_000_000)   # a few ms: the batch below queues behind it
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    emu.sgemm(a, b, mode=m, trans_b=tb, c=c)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) / reps * 1e3)
            res[m] = statistics.median(ts)
        rows.append({"label": label, "M": M, "N": N, "K": K, "trans_b": tb,
                     **{f"us_{m}": round(res[m], 2) for m in modes}})
        print(f"{label:16s} {M:7d} {N:6d} {K:6d} " +
              " ".join(f"{m} {res[m]:9.2f} us" for m in modes), flush=True)
        del a, b, c
    return rows


# ---- the cost model (same form as select_mode in csrc/emu_api.hip) ----
PARAMS = ("x9_fixed", "x9_b", "x9_step", "x9_step_load", "f32_fixed", "f32_step1", "f32_step2")


def predict(M, N, K, p):
    tiles = math.ceil(M / 128) * math.ceil(N / 128)
    nk = math.ceil(K / 32)
    load = min(1.0, tiles / 256)
    x9 = (p["x9_fixed"] + p["x9_b"] * (nk * 32) * (math.ceil(N / 128) * 128) / 1e6 +
          math.ceil(tiles / 256) * nk * (p["x9_step"] + p["x9_step_load"] * load))
    if tiles <= 256:
        f32 = p["f32_fixed"] + nk * p["f32_step1"]
    else:
        f32 = p["f32_fixed"] + math.ceil(tiles / 512) * nk * p["f32_step2"]
    return f32, x9


def fit(rows):
    from scipy.optimize import minimize

    start = dict(x9_fixed=12.0, x9_b=0.3, x9_step=1.3, x9_step_load=0.7, f32_fixed=6.0,
                 f32_step1=2.9, f32_step2=5.1)

    def loss(v):
        p = dict(zip(PARAMS, v))
        e = 0.0
        for r in rows:
            f32, x9 = predict(r["M"], r["N"], r["K"], p)
            if f32 <= 0 or x9 <= 0:
                return 1e9
            e += math.log(f32 / r["us_NATIVE_F32"]) ** 2 + math.log(x9 / r["us_BF16X9"]) ** 2
        return e

    res = minimize(loss, [start[k] for k in PARAMS], method="Nelder-Mead",
                   options=dict(maxiter=40000, xatol=1e-5, fatol=1e-8))
    p = dict(zip(PARAMS, res.x))
    wrong, worst = 0, 1.0
    for r in rows:
        f32, x9 = predict(r["M"], r["N"], r["K"], p)
        best = min(r["us_NATIVE_F32"], r["us_BF16X9"])
        got = r["us_BF16X9"] if x9 < f32 else r["us_NATIVE_F32"]
        wrong += got > best
        worst = max(worst, got / best)
    return p, wrong, worst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fit", action="store_true")
    ap.add_argument("--out", default=None, help="write the measured table as JSON")
    ap.add_argument("--table", default=None, help="fit a table written earlier instead of measuring")
    args = ap.parse_args()
    rows = json.load(open(args.table)) if args.table else measure()
    if args.out:
        json.dump(rows, open(args.out, "w"), indent=1)
    if args.fit:
        p, wrong, worst = fit(rows)
        print("fitted (microseconds): " + ", ".join(f"{k}={v:.4f}" for k, v in p.items()))
        print(f"model picks the slower mode on {wrong} of {len(rows)} shapes; worst ratio to the "
              f"faster mode {worst:.3f}")


if __name__ == "__main__":
    main()
