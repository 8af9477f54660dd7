"""Shared helpers of the GPU parity tests: run a GEMM through the C ABI and
check it against the CPU oracle.

Pass rules (the emulation's accuracy contract):
  * normwise: err_F = ||C - C_ref||_F / ||C_ref||_F against the FP64 oracle,
    over entries with |C_ref| <= FLT_MAX; BF16X9 needs err_F <= 2e-6 and
    err_F <= 1.5 x the NATIVE_F32 path's err_F on the same inputs ("matches
    or exceeds native FP32", section "Limitations and decision criteria" of
    "Unlocking Tensor Core Performance for Machine Learning Interatomic
    Potentials");
  * element by element: |C - C_ref| <= ((2K + 10) 2^-24 + d_P) (|A||B|)_ij
    with d = 0 for NATIVE_F32 and BF16X9, 2^-22 for BF16X6, 2^-14 for
    BF16X3 (a-priori bound of FP32 accumulation allowing 2u per addition,
    plus the dropped bands' size);
  * entries whose FP64 value overflows FP32 must be non-finite in every mode.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

FLT_MAX = float(np.finfo(np.float32).max)
DELTA = {"NATIVE_F32": 0.0, "BF16X9": 0.0, "BF16X6": 2.0**-22, "BF16X3": 2.0**-14, "BF16X1": 2.0**-7}
MODES = ("NATIVE_F32", "BF16X9", "BF16X6", "BF16X3")


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch

    return torch.device("cuda:0")


def run(a_np, b_np, mode, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, c_np=None):
    """emu_sgemm on the GPU; returns the float32 result on the host."""
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch_dev()
    a = torch.from_numpy(np.ascontiguousarray(a_np)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(b_np)).to(dev)
    c = None if c_np is None else torch.from_numpy(np.ascontiguousarray(c_np)).to(dev)
    out = emu.sgemm(a, b, mode=mode, trans_a=trans_a, trans_b=trans_b, alpha=alpha, beta=beta,
                    c=c)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def op(x, t):
    return x.T if t else x


def err_f(out, ref):
    fin = np.abs(ref) <= FLT_MAX
    d = out.astype(np.float64)[fin] - ref[fin]
    return float(np.linalg.norm(d) / np.linalg.norm(ref[fin]))


def bound_ratio(out, ref, a_op, b_op, mode, alpha=1.0, beta=0.0, c=None):
    """max |C - C_ref| / bound over entries whose reference is finite in FP32."""
    K = a_op.shape[1]
    scale = abs(alpha) * (np.abs(a_op).astype(np.float64) @ np.abs(b_op).astype(np.float64))
    if beta != 0.0:
        scale = scale + abs(beta) * np.abs(c.astype(np.float64))
    bound = ((2 * K + 10) * 2.0**-24 + DELTA[mode]) * scale
    fin = np.abs(ref) <= FLT_MAX
    diff = np.abs(out.astype(np.float64) - ref)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(bound > 0, diff / bound, np.where(diff > 0, np.inf, 0.0))
    r = r[fin]
    return float(np.max(r)) if r.size else 0.0


def check_result(out, ref, a_op, b_op, mode, alpha=1.0, beta=0.0, c=None, label=""):
    assert out.shape == ref.shape
    over = np.abs(ref) > FLT_MAX
    assert np.all(~np.isfinite(out[over])), f"{label} {mode}: overflowed entries must be non-finite"
    assert np.all(np.isfinite(out[~over])), f"{label} {mode}: non-finite result for a finite reference"
    ratio = bound_ratio(out, ref, a_op, b_op, mode, alpha, beta, c)
    assert ratio <= 1.0, f"{label} {mode}: componentwise bound exceeded (ratio {ratio:.3g})"
    return err_f(out, ref), ratio
