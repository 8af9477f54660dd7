"""Time the 8-GEMM MLIP layer stacks under each dispatch policy.

The policies of "Unlocking Tensor Core Performance for Machine Learning
Interatomic Potentials" (section "BF16x9 on NVIDIA Blackwell GPUs"):
"performant" uses the emulation only where it is predicted to be faster
(EMU_MODE_AUTO), "eager" uses it wherever it applies (EMU_MODE_BF16X9);
"native" never does (EMU_MODE_NATIVE_F32).  BF16X6 is timed beside them, and
"performant_cached": AUTO's choices with every emulated GEMM's weights split
once beforehand (emu_presplit_b) and used by emu_sgemm_presplit, as a fixed
model in inference or molecular dynamics allows.

Per stack and policy it reports the step time three ways:
  wall   - HIP events around the 8 calls issued back to back, what a caller
           that launches eagerly from Python sees (host launch cost included);
  device - the same 8 calls queued behind a GPU spin, so the events time the
           device work alone (what a captured graph or a busy stream sees);
  steady - the 8 calls repeated back to back for about half a second, timed
           over the second half: the sustained rate of a training or
           molecular-dynamics loop.  The two one-shot figures start from a
           GPU that was idle or spinning, whose clock has not settled under
           the load yet (it first comes up, and on the power-limited shapes
           then falls back to what the power limit allows); the native path,
           which runs near the spec clock once settled, loses most there.

With --ksplit-sweep it instead times every GEMM of the stacks in BF16X9
with each K split S of every tile (a divisor of ceil(K/32), S <= 8;
emu_sgemm_ex), beside the plan the AUTO policy picks (emu_sgemm_plan: a split
of every tile, of the last round of tiles only, or none; run in BF16X9 with
EMU_KSPLIT_AUTO) and native FP32 (device time, calls queued behind a GPU
spin, median of 5 runs of 20 calls).

    python3 -m emulated_fp32_matrix_amd.policies [--stacks 2 3 4] [--json out.json]
    python3 -m emulated_fp32_matrix_amd.policies --ksplit-sweep --stacks 2 4 [--json out.json]
    python3 -m emulated_fp32_matrix_amd.policies --markdown out.json   # tables of a saved run

With --launches it runs each stack's 8 GEMMs in AUTO and in NATIVE_F32,
queued behind a GPU spin (so that the kernels run back to back), five times:
the run to profile with `rocprofv3 --kernel-trace`.  --launch-table
summarises that trace per kind of kernel and per stack.

    rocprofv3 --kernel-trace -d DIR -o kt --output-format csv -- \
        python3 -m emulated_fp32_matrix_amd.policies --launches --stacks 2 4
    python3 -m emulated_fp32_matrix_amd.policies --launch-table DIR/kt_kernel_trace.csv --stacks 2 4
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

POLICIES = {"performant": "AUTO", "eager": "BF16X9", "native": "NATIVE_F32", "bf16x6": "BF16X6",
            "performant_cached": "AUTO+planes"}


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

    plans = {g.name: emu.select_plan(g.M, g.N, g.K) for g in gemms}
    # "AUTO+planes": AUTO's choices with the weights split once beforehand
    # (emu_presplit_b, outside the timed region) and emu_sgemm_presplit
    planes = {g.name: emu.presplit_b(b, mode="BF16X9", trans_b=g.trans_b)
              for g, a, b, c in tensors if choice[g.name] == "BF16X9"}

    def step(mode):
        for g, a, b, c in tensors:
            if mode == "AUTO+planes" and g.name in planes:
                emu.sgemm_presplit(a, planes[g.name], trans_a=g.trans_a, c=c, ksplit=emu.KSPLIT_AUTO)
            else:
                emu.sgemm(a, b, mode="AUTO" if mode == "AUTO+planes" else mode, trans_a=g.trans_a,
                          trans_b=g.trans_b, c=c)

    out = {"stack": stack, "name": synth.CONFIG_NAMES[stack], "gflop": flops / 1e9,
           "auto_choice": choice, "auto_plan": plans, "policies": {}}
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
        # steady: about half a second of steps back to back, the second half timed
        n = max(20, int(0.5e6 / d))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for i in range(n):
            step(mode)
            if i == n // 2:
                ev[0].record(stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        st = ev[0].elapsed_time(ev[1]) * 1e3 / (n - n // 2 - 1)
        out["policies"][pol] = {"mode": mode, "wall_us": round(w, 1), "device_us": round(d, 1),
                                "steady_us": round(st, 1),
                                "wall_tflops": round(flops / w / 1e6, 2),
                                "device_tflops": round(flops / d / 1e6, 2),
                                "steady_tflops": round(flops / st / 1e6, 2)}
        print(f"stack {stack} {pol:10s} ({mode:10s}): wall {w:9.1f} us ({flops / w / 1e6:6.1f} TFLOP/s)  "
              f"device {d:9.1f} us ({flops / d / 1e6:6.1f} TFLOP/s)  steady {st:9.1f} us "
              f"({flops / st / 1e6:6.1f} TFLOP/s)", flush=True)
    del tensors
    torch.cuda.empty_cache()
    return out


def _device_us(fn, calls=20, reps=5):
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        torch.cuda._sleep(20_000_000)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / calls)
    return statistics.median(ts)


def ksplit_sweep(stack):
    import torch

    import emulated_fp32_matrix_amd as emu

    synth = _synth()
    dev = torch.device("cuda:0")
    rows = []
    for g in synth.gemms(stack):
        a = torch.from_numpy(synth.make_a(g)).to(dev)
        b = torch.from_numpy(synth.make_b(g)).to(dev)
        c = torch.empty((g.M, g.N), dtype=torch.float32, device=dev)
        nk = -(-g.K // 32)
        times = {}
        for S in [s for s in range(1, 9) if nk % s == 0]:
            times[S] = _device_us(lambda: emu.sgemm(a, b, mode="BF16X9", trans_a=g.trans_a,
                                                    trans_b=g.trans_b, c=c, ksplit=S))
        native = _device_us(lambda: emu.sgemm(a, b, mode="NATIVE_F32", trans_a=g.trans_a,
                                              trans_b=g.trans_b, c=c))
        plan = emu.select_plan(g.M, g.N, g.K)
        auto_us = _device_us(lambda: emu.sgemm(a, b, mode="BF16X9", trans_a=g.trans_a,
                                               trans_b=g.trans_b, c=c, ksplit=emu.KSPLIT_AUTO))
        best = min(times, key=times.get)
        rows.append({"gemm": g.name, "M": g.M, "N": g.N, "K": g.K, "auto_plan": list(plan),
                     "auto_us": round(auto_us, 1), "best_ksplit": best,
                     "x9_us": {str(k): round(v, 1) for k, v in times.items()},
                     "native_us": round(native, 1)})
        print(f"stack {stack} {g.name:8s} {g.M}x{g.N}x{g.K}: auto plan {plan} {auto_us:6.1f} us, "
              f"best full split S={best}  " +
              "  ".join(f"S{k} {v:6.1f}" for k, v in times.items()) + f"  native {native:6.1f} us",
              flush=True)
        del a, b, c
    torch.cuda.empty_cache()
    return {"stack": stack, "name": synth.CONFIG_NAMES[stack], "gemms": rows}


LAUNCH_REPS = 5


def launches(stacks):
    """The kernel sequence --launch-table reads: per stack and mode
    (AUTO, NATIVE_F32), LAUNCH_REPS repetitions of the 8 GEMMs, each queued
    behind a GPU spin."""
    import torch

    import emulated_fp32_matrix_amd as emu

    synth = _synth()
    dev = torch.device("cuda:0")
    for stack in stacks:
        gemms = synth.gemms(stack)
        tensors = [(g, torch.from_numpy(synth.make_a(g)).to(dev), torch.from_numpy(synth.make_b(g)).to(dev),
                    torch.empty((g.M, g.N), dtype=torch.float32, device=dev)) for g in gemms]
        for mode in ("AUTO", "NATIVE_F32"):
            for _ in range(LAUNCH_REPS):
                torch.cuda.synchronize()
                torch.cuda._sleep(20_000_000)
                for g, a, b, c in tensors:
                    emu.sgemm(a, b, mode=mode, trans_a=g.trans_a, trans_b=g.trans_b, c=c)
            torch.cuda.synchronize()
            print(f"stack {stack} {mode}: {LAUNCH_REPS} queued runs", flush=True)
        del tensors
        torch.cuda.empty_cache()


def _kernel_kind(name):
    for key, kind in (("presplit_kernel", "B pre-split"), ("pack_b_f32", "B pack (native)"),
                      ("ksplit_reduce", "K-split reduction"), ("gemm_bf16", "emulated GEMM"),
                      ("gemm_f32", "native GEMM")):
        if key in name:
            return kind
    return None


def launch_table(trace_csv, stacks):
    """Markdown summary of a kernel trace of launches(): per stack and mode,
    the median over the repetitions of the summed device time of each kind
    of kernel (start to end of each launch), the number of launches, and the
    span of the 8 GEMMs from the first launch's start to the last one's
    end."""
    import csv

    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    runs, cur = [], None
    for r in rows:
        name = r["Kernel_Name"]
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if "spin_kernel" in name:
            cur = []
            runs.append(cur)
        elif cur is not None:
            cur.append((name, t0, t1))
    expect = len(stacks) * 2 * LAUNCH_REPS
    assert len(runs) == expect, f"{len(runs)} queued runs in the trace, expected {expect}"
    synth = _synth()
    out = ["| stack | mode | launches per step | " + " | ".join(
        ["B pre-split us", "B pack us", "K-split reduction us", "GEMM kernels us"]) +
        " | step span us |", "|---|---|---|---|---|---|---|---|"]
    i = 0
    for stack in stacks:
        for mode in ("AUTO", "NATIVE_F32"):
            sums = {}
            spans, counts = [], []
            for run in runs[i:i + LAUNCH_REPS]:
                per = {}
                for name, t0, t1 in run:
                    kind = _kernel_kind(name)
                    if kind in ("emulated GEMM", "native GEMM"):
                        kind = "GEMM kernels"
                    if kind is not None:
                        per[kind] = per.get(kind, 0.0) + (t1 - t0) / 1e3
                for k, v in per.items():
                    sums.setdefault(k, []).append(v)
                spans.append((run[-1][2] - run[0][1]) / 1e3)
                counts.append(len(run))
            i += LAUNCH_REPS
            cell = lambda k: f"{statistics.median(sums[k]):.1f}" if k in sums else ""
            out.append(f"| {synth.CONFIG_NAMES[stack]} | {mode} | {statistics.median(counts):.0f} | "
                       f"{cell('B pre-split')} | {cell('B pack (native)')} | {cell('K-split reduction')} | "
                       f"{cell('GEMM kernels')} | {statistics.median(spans):.1f} |")
    return "\n".join(out)


def _policy_markdown(res):
    out = []
    for r in res:
        out.append(f"## Stack: {r['name']} ({r['gflop']:.2f} GFLOP per step)\n")
        choice = ", ".join(f"{k} {v}" + (f" ({_plan_text(r['auto_plan'][k])})"
                                          if v != "NATIVE_F32" and r["auto_plan"][k][0] > 1 else "")
                           for k, v in r["auto_choice"].items())
        out.append(f"AUTO's choices: {choice}\n")
        out.append("| policy | mode | wall us | wall TFLOP/s | wall speedup | device us | device TFLOP/s "
                   "| device speedup | steady us | steady TFLOP/s | steady speedup |\n"
                   "|---|---|---|---|---|---|---|---|---|---|---|")
        nat = r["policies"]["native"]
        for name, p in r["policies"].items():
            out.append(f"| {name} | {p['mode']} | {p['wall_us']:.1f} | {p['wall_tflops']:.1f} | "
                       f"{nat['wall_us'] / p['wall_us']:.2f} | {p['device_us']:.1f} | "
                       f"{p['device_tflops']:.1f} | {nat['device_us'] / p['device_us']:.2f} | "
                       f"{p['steady_us']:.1f} | {p['steady_tflops']:.1f} | {nat['steady_us'] / p['steady_us']:.2f} |")
        out.append("")
    return "\n".join(out)


def _plan_text(plan):
    """'S = 2 on the last round (tiles 256..383 of 384, 128 rows)' and the like."""
    S, th, sf = plan
    if S == 1:
        return f"no split, {th}-row tiles"
    if sf == 0:
        return f"S = {S} on every tile, {th}-row tiles"
    return f"S = {S} on the tiles from {sf} on, {th}-row tiles"


def _ksplit_markdown(res):
    out = []
    for r in res:
        splits = sorted({int(s) for g in r["gemms"] for s in g["x9_us"]})
        out.append(f"## {r['name']}\n")
        out.append("| GEMM | M x N x K | 128-row tiles | " + " | ".join(f"S = {s}" for s in splits) +
                   " | native | AUTO plan | AUTO plan us | best full split | AUTO vs S = 1 |")
        out.append("|---|---|---|" + "---|" * len(splits) + "---|---|---|---|---|")
        tot = {"s1": 0.0, "auto": 0.0, "best": 0.0, "native": 0.0}
        for g in r["gemms"]:
            t = {int(k): v for k, v in g["x9_us"].items()}
            tiles = -(-g["M"] // 128) * -(-g["N"] // 128)
            cells = " | ".join(f"{t[s]:.1f}" if s in t else "" for s in splits)
            auto = g["auto_us"]
            out.append(f"| {g['gemm']} | {g['M']} x {g['N']} x {g['K']} | {tiles} | {cells} | "
                       f"{g['native_us']:.1f} | {_plan_text(g['auto_plan'])} | {auto:.1f} | "
                       f"S = {g['best_ksplit']} | {t[1] / auto:.2f}x |")
            tot["s1"] += t[1]
            tot["auto"] += auto
            tot["best"] += t[g["best_ksplit"]]
            tot["native"] += g["native_us"]
        out.append(f"\nStack total: S = 1 {tot['s1']:.1f} us, AUTO's plan {tot['auto']:.1f} us "
                   f"({tot['s1'] / tot['auto']:.2f}x), best full split per GEMM {tot['best']:.1f} us, "
                   f"native {tot['native']:.1f} us.\n")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stacks", type=int, nargs="+", default=[2, 4, 3])
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--json", default=None)
    ap.add_argument("--ksplit-sweep", action="store_true")
    ap.add_argument("--markdown", default=None, help="print the tables of a JSON file written earlier")
    ap.add_argument("--launches", action="store_true", help="queued stack runs for a kernel trace")
    ap.add_argument("--launch-table", default=None, help="summarise a kernel trace of --launches")
    args = ap.parse_args()
    if args.launch_table:
        print(launch_table(args.launch_table, args.stacks))
        return
    if args.launches:
        launches(args.stacks)
        return
    if args.markdown:
        res = json.load(open(args.markdown))
        print(_ksplit_markdown(res) if res and "gemms" in res[0] else _policy_markdown(res))
        return
    if args.ksplit_sweep:
        res = [ksplit_sweep(s) for s in args.stacks]
    else:
        res = [time_stack(s, args.reps) for s in args.stacks]
    if args.json:
        json.dump(res, open(args.json, "w"), indent=1)


if __name__ == "__main__":
    main()
