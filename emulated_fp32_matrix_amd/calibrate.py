"""Measure the device time of NATIVE_F32 and BF16X9 calls over a set of GEMM
shapes, and fit the cost model that EMU_MODE_AUTO uses to choose between
them (the "performant" policy of "Unlocking Tensor Core Performance for
Machine Learning Interatomic Potentials", section "BF16x9 on NVIDIA
Blackwell GPUs").

Device time, not wall time: each batch of calls is queued behind a GPU spin
(torch.cuda._sleep), so the calls run back to back whatever the host-side
launch cost, and a pair of HIP events around the batch times the device
work of one call (for BF16X9: the B pre-split and the main kernel).

    python3 -m emulated_fp32_matrix_amd.calibrate [--fit [--markdown]] [--out table.json]
    python3 -m emulated_fp32_matrix_amd.calibrate --table table.json --fit --markdown

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


# ---- the cost model (same form as predict_x9_us / predict_us in csrc/emu_api.hip) ----
PARAMS = ("x9_fixed", "x9_step_part", "x9_step_full", "f32_fixed", "f32_step_part", "f32_step_full")
# A k-step of the emulated kernel's 64-row tiles against a 128-row one
# (kX9Step64): measured separately, with the tile height forced, on the
# 552,960-row stack where every CU is busy either way; not fitted here.
X9_STEP64 = 0.59


def predict_x9(M, N, K, p, tile_m):
    tiles = math.ceil(M / tile_m) * math.ceil(N / 128)
    nk = math.ceil(K / 32)
    step = (p["x9_step_full"] if tiles >= 256 else p["x9_step_part"]) * (X9_STEP64 if tile_m == 64 else 1.0)
    return p["x9_fixed"] + math.ceil(tiles / 256) * nk * step


def predict(M, N, K, p):
    """(native, BF16X9 unsplit) predicted device time in microseconds: both
    kernels run ceil(tiles / 256) rounds of nk k-steps, each step costing
    *_step_full once every CU has a tile and *_step_part before; the
    emulated kernel's tiles have 128 rows, or 64 where that is predicted at
    least 3 % faster (the library's choose_tile_m), a 64-row step costing
    X9_STEP64 of a 128-row one."""
    tiles = math.ceil(M / 128) * math.ceil(N / 128)
    nk = math.ceil(K / 32)
    full = tiles >= 256
    x9_128, x9_64 = predict_x9(M, N, K, p, 128), predict_x9(M, N, K, p, 64)
    x9 = x9_64 if x9_64 < 0.97 * x9_128 else x9_128
    f32 = p["f32_fixed"] + math.ceil(tiles / 256) * nk * (p["f32_step_full"] if full else p["f32_step_part"])
    return f32, x9


def fit(rows):
    from scipy.optimize import minimize

    start = dict(x9_fixed=12.0, x9_step_part=1.4, x9_step_full=2.0, f32_fixed=12.0,
                 f32_step_part=2.2, f32_step_full=2.3)

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
                   options=dict(maxiter=80000, xatol=1e-7, fatol=1e-10))
    p = dict(zip(PARAMS, res.x))
    wrong, worst = 0, 1.0
    for r in rows:
        f32, x9 = predict(r["M"], r["N"], r["K"], p)
        best = min(r["us_NATIVE_F32"], r["us_BF16X9"])
        got = r["us_BF16X9"] if x9 < f32 else r["us_NATIVE_F32"]
        wrong += got > best
        worst = max(worst, got / best)
    return p, wrong, worst


def markdown(rows, p):
    """The measured table with the model's predictions and choices."""
    out = ["| shape | M | N | K | NATIVE_F32 us | BF16X9 us | native / X9 | model native | model X9 "
           "| AUTO picks | picks the faster |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        f32, x9 = predict(r["M"], r["N"], r["K"], p)
        nat, emu = r["us_NATIVE_F32"], r["us_BF16X9"]
        pick = "BF16X9" if x9 < f32 else "NATIVE_F32"
        got = emu if pick == "BF16X9" else nat
        ok = "yes" if got <= min(nat, emu) else f"no ({got / min(nat, emu):.3f}x)"
        out.append(f"| {r['label']} | {r['M']} | {r['N']} | {r['K']} | {nat:.1f} | {emu:.1f} | "
                   f"{nat / emu:.2f} | {f32:.1f} | {x9:.1f} | {pick} | {ok} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fit", action="store_true")
    ap.add_argument("--out", default=None, help="write the measured table as JSON")
    ap.add_argument("--table", default=None, help="fit a table written earlier instead of measuring")
    ap.add_argument("--markdown", action="store_true", help="with --fit: print the table with the "
                    "model's predictions and choices")
    args = ap.parse_args()
    rows = json.load(open(args.table)) if args.table else measure()
    if args.out:
        json.dump(rows, open(args.out, "w"), indent=1)
    if args.fit:
        p, wrong, worst = fit(rows)
        print("fitted (microseconds): " + ", ".join(f"{k}={v:.4f}" for k, v in p.items()))
        print(f"model picks the slower mode on {wrong} of {len(rows)} shapes; worst ratio to the "
              f"faster mode {worst:.3f}")
        if args.markdown:
            print(markdown(rows, p))


if __name__ == "__main__":
    main()
