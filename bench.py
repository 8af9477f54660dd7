#!/usr/bin/env python3
"""Benchmark: emulated-FP32 GEMM throughput on the 17,280-atom MLIP layer stack.

One step = the eight GEMMs of one transformer block at 552,960 token rows
(17,280 atoms x 32 neighbours, d = 256): for each linear layer (QKV 256->768,
out 256->256, FFN 256->512->256) the forward GEMM Y = X.W (NN) and the
input-gradient GEMM dX = dY.W^T (NT), all through emu_sgemm in BF16X9 mode.
This is the large-GEMM workload of "Unlocking Tensor Core Performance for
Machine Learning Interatomic Potentials" (section "BF16x9 on NVIDIA
Blackwell GPUs", Figure 3: 17,280-atom water supercell), with seeded
synthetic inputs in place of the model's activations (X, dY ~ N(0,1),
W ~ N(0, 1/fan_in)).

Prints one JSON line (last line of stdout).  value = aggregate FP32-equivalent
TFLOP/s of the step (2MNK per GEMM) with inputs resident in HBM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

_ROOT = os.path.dirname(os.path.abspath(__file__))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, 256 CUs x 4096 flop/clk x 2.4 GHz
F32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 MFMA
HBM_PEAK_GBS = 8000.0
PRODUCTS = {"BF16X9": 9, "BF16X6": 6, "BF16X3": 3, "BF16X1": 1, "NATIVE_F32": 1}
BANDS = {"BF16X9": 5, "BF16X6": 3, "BF16X3": 2, "BF16X1": 1}
WORKLOAD = 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", default="BF16X9", type=str.upper,
                    choices=["BF16X9", "BF16X6", "BF16X3", "BF16X1", "NATIVE_F32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the NATIVE_F32 and torch-fp32 context timings")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock reading and the matrix-unit stream after the timed region")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, copy 1 GiB three times with one elementwise kernel "
                         "(the reference that scales the FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args()


# Source files that determine the code of the emulated GEMM kernels.
KERNEL_SOURCES = ("emulated_fp32_matrix_amd/csrc/emu_gemm_bf16.hip",
                  "emulated_fp32_matrix_amd/csrc/emu_tile.h",
                  "emulated_fp32_matrix_amd/csrc/emu_walk.h",
                  "emulated_fp32_matrix_amd/csrc/emu_device.h")

# HBM traffic per launch of the main BF16X9 GEMM kernel over this workload
# (bytes, mean over the 8 GEMMs), from two rocprofv3 --pmc runs (FETCH_SIZE,
# WRITE_SIZE) scaled by the same counters' reading for a 1 GiB device copy.
# Keyed by the SHA-256 of KERNEL_SOURCES: a changed kernel reports null.
TRAFFIC_BY_SOURCE = {
    "bdcdf111e991602f3f57b8fcd0c2018b43080069b1718fe08138c2bc7f79b813": 1971042530,
}


SPEC_SCLK_GHZ = 2.4         # the clock of the spec peaks


def cpu_model():
    """The host CPU's model name (first 'model name' of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(_ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _smi_handle(amdsmi, torch):
    """The amdsmi handle of torch's current device (matched by PCI address;
    amdsmi lists every GPU of the machine, whatever the visible devices)."""
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
    handles = amdsmi.amdsmi_get_processor_handles()
    for h in handles:
        dom, bus, rest = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")
        if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
            return h
    return handles[0] if len(handles) == 1 else None


def clock_under_load(torch, emu, gemms, tensors, mode, max_s=4.0):
    """Shader clock of the same steps as the timed region, run again right
    after it.  The driver's GPU metrics table (read through amdsmi) refreshes
    about once a second with each XCD's clock, the socket power and the GFX
    activity over the interval since the previous refresh; the steps keep
    the GPU busy until an interval that began after they started has been
    reported fully busy, and that reading is returned (None when amdsmi is
    missing or gives no such interval within max_s seconds)."""
    try:
        import amdsmi
    except ImportError:
        return None
    try:
        amdsmi.amdsmi_init()
    except Exception as e:   # noqa: BLE001 - the reading is optional
        log(f"clock reading: amdsmi_init failed ({e})")
        return None
    try:
        handle = _smi_handle(amdsmi, torch)
        if handle is None:
            return None

        def read():
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            return (m.get("accumulation_counter"), m.get("current_gfxclks"), m.get("current_socket_power"),
                    m.get("average_gfx_activity"))

        stream = torch.cuda.current_stream()
        last = read()[0]
        refreshes = 0
        done = None
        prev = None
        t0 = time.perf_counter()
        while done is None and time.perf_counter() - t0 < max_s:
            for _ in range(8):
                for g, (a, b, c) in zip(gemms, tensors):
                    emu.sgemm(a, b, mode=mode, trans_a=g.trans_a, trans_b=g.trans_b, c=c, stream=stream)
            ev = torch.cuda.Event()
            ev.record(stream)
            if prev is not None:
                prev.synchronize()   # one batch of steps stays queued behind the one running
            prev = ev
            acc, clks, power, busy = read()
            if acc == last:
                continue
            last = acc
            refreshes += 1
            # the first refresh's interval began before the steps did
            if refreshes >= 2 and isinstance(busy, (int, float)) and busy >= 95:
                mhz = [float(x) for x in clks if isinstance(x, (int, float))]
                if mhz:
                    done = {"sclk_ghz": round(sum(mhz) / len(mhz) / 1e3, 3),
                            "xcd_ghz": [round(x / 1e3, 3) for x in mhz],
                            "socket_power_w": power, "gfx_activity_pct": busy,
                            "after_s": round(time.perf_counter() - t0, 2)}
        torch.cuda.synchronize()
        return done
    except Exception as e:   # noqa: BLE001
        log(f"clock reading failed ({e})")
        torch.cuda.synchronize()
        return None
    finally:
        amdsmi.amdsmi_shut_down()


def mfma_stream_rate(kind):
    """The matrix units' sustained rate on this device under a dense stream
    of the same matrix instruction (emulated_fp32_matrix_amd.ceiling: every
    SIMD, register operands, about 1 s): the practical roof the kernel's
    rate is set against.  None when the probe library is not built."""
    try:
        from emulated_fp32_matrix_amd import ceiling

        r = ceiling.run(kind, 1.0)
    except Exception as e:   # noqa: BLE001 - the reading is optional
        log(f"matrix-unit stream: not measured ({e})")
        return None
    return {"instruction": r["instruction"], "tflops": r["tflops"], "sclk_ghz": r["sclk_ghz"],
            "frac_of_spec": r["frac_of_spec"]}


def make_inputs(torch, dev, gemms):
    import synth

    tensors = []
    for g in gemms:
        t0 = time.time()
        a = torch.from_numpy(synth.make_a(g)).to(dev)
        b = torch.from_numpy(synth.make_b(g)).to(dev)
        c = torch.empty((g.M, g.N), dtype=torch.float32, device=dev)
        tensors.append((a, b, c))
        log(f"  inputs {g.name}: A {tuple(a.shape)} B {tuple(b.shape)} ({time.time() - t0:.1f}s)")
    return tensors


def time_stack(torch, emu, gemms, tensors, mode, steps, warmup):
    """Returns (ms per step, per-GEMM mean ms) timed with HIP events on the
    stream the kernels are launched on (torch's current stream)."""
    stream = torch.cuda.current_stream()

    def step(events=None):
        for gi, (g, (a, b, c)) in enumerate(zip(gemms, tensors)):
            if events is not None:
                events[gi][0].record(stream)
            emu.sgemm(a, b, mode=mode, trans_a=g.trans_a, trans_b=g.trans_b, c=c, stream=stream)
            if events is not None:
                events[gi][1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    per = np.zeros(len(gemms))
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in gemms] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(steps):
        step(ev[s])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    for s in range(steps):
        for gi in range(len(gemms)):
            per[gi] += ev[s][gi][0].elapsed_time(ev[s][gi][1])
    return total_ms / steps, per / steps


def time_torch_fp32(torch, gemms, tensors, steps, warmup):
    torch.backends.cuda.matmul.allow_tf32 = False

    def step():
        for g, (a, b, c) in zip(gemms, tensors):
            bb = b.t() if g.trans_b else b
            torch.matmul(a, bb, out=c)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        step()
    s1.record()
    torch.cuda.synchronize()
    return s0.elapsed_time(s1) / steps


def cpu_baseline(gemms, target_s):
    """The CPU oracle's model of the same computation (split + nine band-
    accumulated products, FP32) on a bounded row sample of each GEMM."""
    import oracle
    import synth

    cores = oracle.num_threads()
    # calibrate: 32 rows of the first GEMM
    g0 = gemms[0]
    a = synth.make_a(g0, rows=(0, 32))
    b = synth.make_b(g0)
    t0 = time.time()
    oracle.emu_gemm(a, b, "BF16X9", g0.trans_a, g0.trans_b)
    dt = max(time.time() - t0, 1e-3)
    flops_per_s = 2 * 32 * g0.N * g0.K / dt
    total_row_flops = sum(2 * g.N * g.K for g in gemms)
    rows = int(max(32, min(65536, target_s * flops_per_s / total_row_flops)))
    flops = 0
    t0 = time.time()
    for g in gemms:
        a = synth.make_a(g, rows=(0, rows))
        b = synth.make_b(g)
        oracle.emu_gemm(a, b, "BF16X9", g.trans_a, g.trans_b)
        flops += 2 * rows * g.N * g.K
    el = time.time() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "sample": (f"first {rows} of 552,960 rows of each of the 8 GEMMs "
                       f"({flops / 1e9:.1f} GFLOP, {el:.1f} s, BF16X9 model: exact split + "
                       "FP32 band accumulation, OpenMP over rows)")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the emulated GEMM "
              "shards by token rows with no exchange, so N GPUs would each run this "
              "benchmark on M/N rows.", file=sys.stderr)
        sys.exit(2)

    import torch

    import emulated_fp32_matrix_amd as emu
    import synth

    mode = args.mode.upper()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gemms = synth.gemms(WORKLOAD)
    flops = np.array([g.flops for g in gemms], dtype=np.float64)
    log(f"workload: {synth.CONFIG_NAMES[WORKLOAD]}, {flops.sum() / 1e9:.2f} GFLOP per step")
    tensors = make_inputs(torch, dev, gemms)

    ms, per = time_stack(torch, emu, gemms, tensors, mode, args.steps, args.warmup)
    value = flops.sum() / (ms * 1e-3) / 1e12
    log(f"{mode}: {ms:.3f} ms/step, {value:.1f} TFLOP/s")
    for g, t, f in zip(gemms, per, flops):
        log(f"  {g.name:9s} {g.M}x{g.N}x{g.K} {'NT' if g.trans_b else 'NN'}: {t * 1e3:8.1f} us "
            f"{f / (t * 1e-3) / 1e12:7.1f} TFLOP/s")

    # Dominant kernel: every GEMM of the stack runs the same main kernel
    # instantiation (A row-major and split inside it in both the forward NN
    # and the input-gradient NT GEMM; B pre-split by a small kernel), so its
    # average launch time is the per-GEMM event time averaged over the 8
    # GEMMs.  The event pair around each call also covers the B pre-split
    # (about 1 us), which the rocprofv3 summary lists separately.
    P = PRODUCTS[mode]
    n_launch = len(gemms)
    avg_us = float(per.sum()) / n_launch * 1e3
    peak = BF16_PEAK_TFLOPS if mode in BANDS else F32_PEAK_TFLOPS
    achieved = P * float(flops.sum()) / n_launch / (avg_us * 1e-6) / 1e12
    traffic = None
    if mode == "BF16X9":
        traffic = TRAFFIC_BY_SOURCE.get(kernel_source_hash())
    clock = None if args.no_clock else clock_under_load(torch, emu, gemms, tensors, mode)
    sclk = clock["sclk_ghz"] if clock else None
    if clock:
        log(f"clock under load: {clock}")
    stream = None if args.no_clock else mfma_stream_rate("bf16" if mode in BANDS else "f32")
    if stream:
        log(f"matrix-unit stream: {stream}")
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                # the same fraction against the peak at the clock the steps run at
                "sclk_ghz": sclk,
                "frac_at_measured_clock": (round(achieved / (peak * sclk / SPEC_SCLK_GHZ), 4)
                                           if sclk else None),
                "clock": ({"source": "amdsmi GPU metrics: mean of the XCD clocks over a fully busy "
                                     "1 s interval of the same steps, right after the timed region",
                           **clock} if clock else None),
                # the practical roof: a dense stream of the same matrix
                # instruction alone, on this device, right after
                "mfma_stream": stream,
                "frac_of_mfma_stream": round(achieved / stream["tflops"], 4) if stream else None,
                "kernel": ("gemm_bf16_pp_kernel<%d, false, false, 128>" % BANDS[mode])
                if mode in BANDS else "gemm_f32_pp_kernel",
                "avg_launch_us": round(avg_us, 2),
                "algorithmic_flop_per_launch": round(P * float(flops.sum()) / n_launch)}

    extra = {}
    if not args.no_context and mode != "NATIVE_F32":
        ms_n, per_n = time_stack(torch, emu, gemms, tensors, "NATIVE_F32", max(3, args.steps // 2), 2)
        ms_t = time_torch_fp32(torch, gemms, tensors, max(3, args.steps // 2), 2)
        extra = {"native_f32_tflops": round(flops.sum() / (ms_n * 1e-3) / 1e12, 2),
                 "speedup_vs_native_f32": round(ms_n / ms, 3),
                 "torch_fp32_matmul_tflops": round(flops.sum() / (ms_t * 1e-3) / 1e12, 2),
                 "speedup_vs_torch_fp32": round(ms_t / ms, 3)}
        log(f"NATIVE_F32: {ms_n:.3f} ms/step; torch fp32 matmul: {ms_t:.3f} ms/step")
    per_gemm = {g.name: round(f / (t * 1e-3) / 1e12, 2) for g, t, f in zip(gemms, per, flops)}
    del tensors
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # one elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copy done")
        del src, dst
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(gemms, args.cpu_seconds)
        log(f"  {cpu}")

    out = {
        "metric": "emulated-FP32 GEMM TFLOP/s at 17,280-atom shapes; fraction of bf16 MFMA peak/9",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "mlip-stack 17,280 atoms x 32 nbrs = 552,960 rows, d=256, "
                               "8 GEMMs (QKV/out/FFN1/FFN2 fwd NN + dX NT)",
                   "mode": mode, "compute": f"{P} bf16 MFMA products, FP32 band accumulation"
                   if P > 1 else "fp32 MFMA",
                   "gflop_per_step": round(flops.sum() / 1e9, 3),
                   "frac_of_bf16_peak_over_9": round(value / (BF16_PEAK_TFLOPS / 9), 4),
                   "frac_of_fp32_mfma_peak": round(value / F32_PEAK_TFLOPS, 4),
                   "per_gemm_tflops": per_gemm, **extra},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
