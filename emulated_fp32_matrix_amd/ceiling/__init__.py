"""The matrix units' sustained rate on this MI355X, under a dense stream of
matrix instructions (``mfma_stream.hip``): the practical roof of every GEMM
here, the emulated one included.

    python3 -m emulated_fp32_matrix_amd.ceiling [--seconds 2.5]

prints one JSON line per instruction (bf16 32x32x16, FP32 32x32x2): the
sustained TFLOP/s, its fraction of the spec peak, the shader clock measured
inside the kernel, and the socket power and GFX activity that the driver's
GPU metrics table reports for a one-second interval inside the run (amdsmi;
null where it is not importable or sees more than one GPU).  ``build()`` compiles the library next to
this file (``__graft_entry__.build()`` calls it).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import subprocess
import threading
import time

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_stream.hip")
LIB = os.path.join(HERE, "libemu_ceiling.so")
SPEC = {"bf16": 2516.6, "f32": 157.3}   # dense MFMA peaks at 2.4 GHz, TFLOP/s

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc"
    cmd = [hipcc, *FLAGS, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {SRC}:\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (run build())")
    lib = ctypes.CDLL(LIB)
    d = ctypes.POINTER(ctypes.c_double)
    lib.emu_ceiling_run.argtypes = [ctypes.c_int, ctypes.c_double, d, d, d]
    lib.emu_ceiling_run.restype = ctypes.c_int
    return lib


class _Power:
    """Polls the GPU metrics table while the stream runs and keeps the
    first refresh whose interval began after the polling started.  Only on
    a machine where amdsmi sees one GPU (the one the stream runs on);
    elsewhere the reading is left out."""

    def __init__(self):
        self.reading = None
        self._stop = False
        self._smi = None
        try:
            import amdsmi
        except ImportError:
            return
        try:
            amdsmi.amdsmi_init()
        except Exception:   # noqa: BLE001 - the reading is optional
            return
        try:
            handles = amdsmi.amdsmi_get_processor_handles()
        except Exception:   # noqa: BLE001
            handles = []
        if len(handles) != 1:
            amdsmi.amdsmi_shut_down()
            return
        self._smi, self._h = amdsmi, handles[0]

    def _run(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        last, refreshes = m.get("accumulation_counter"), 0
        while not self._stop:
            time.sleep(0.02)
            m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
            if m.get("accumulation_counter") == last:
                continue
            last = m.get("accumulation_counter")
            refreshes += 1
            if refreshes >= 2 and self.reading is None:
                clks = [x for x in m.get("current_gfxclks", []) if isinstance(x, (int, float))]
                self.reading = {"socket_power_w": m.get("current_socket_power"),
                                "gfx_activity_pct": m.get("average_gfx_activity"),
                                "xcd_mean_clock_ghz": round(sum(clks) / len(clks) / 1e3, 3) if clks else None}

    def __enter__(self):
        if self._smi is not None:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop = True
        if self._smi is not None:
            self._t.join(timeout=5)
            self._smi.amdsmi_shut_down()


def run(kind: str, seconds: float) -> dict:
    lib = _lib()
    tf, ghz, dur = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    with _Power() as pw:
        st = lib.emu_ceiling_run(0 if kind == "bf16" else 1, float(seconds), ctypes.byref(tf),
                                 ctypes.byref(ghz), ctypes.byref(dur))
    if st != 0:
        raise RuntimeError(f"emu_ceiling_run failed with HIP error {st}")
    spec = SPEC[kind]
    return {"instruction": "v_mfma_f32_32x32x16_bf16" if kind == "bf16" else "v_mfma_f32_32x32x2_f32",
            "tflops": round(tf.value, 1), "spec_tflops": spec, "frac_of_spec": round(tf.value / spec, 4),
            "sclk_ghz": round(ghz.value, 3),
            "frac_of_peak_at_that_clock": round(tf.value / (spec * ghz.value / 2.4), 4) if ghz.value else None,
            "seconds": round(dur.value, 2), "power": pw.reading}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seconds", type=float, default=2.5)
    args = ap.parse_args()
    for kind in ("bf16", "f32"):
        print(json.dumps(run(kind, args.seconds)), flush=True)


if __name__ == "__main__":
    main()
