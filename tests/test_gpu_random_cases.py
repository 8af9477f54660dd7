"""Random calls through the C ABI, each bit for bit against the oracle's model
of the path it takes.

A seeded sample of the argument space: shapes from 1 to a few hundred in
each dimension (ragged against the 128 x 128 tiles and the 32-wide k-steps),
every transpose pair, every mode including AUTO, alpha / beta / bias,
leading dimensions with padding, pointers 4 bytes past a 16-byte boundary
(the pre-split and register-staged paths), and the K split: none, an
explicit one on every tile, or EMU_KSPLIT_AUTO (the AUTO plan, possibly only
the last round of tiles).  The model is oracle.native_gemm_mfma for
NATIVE_F32 and oracle.emu_gemm_mfma for the emulated modes (with the split
on the tiles the plan splits), so every case is an exact comparison.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import say

pytestmark = pytest.mark.gpu

MODES = ["NATIVE_F32", "BF16X9", "BF16X6", "BF16X3", "BF16X1", "AUTO"]
N_CASES = 120


def _case(rng):
    M, N, K = (int(x) for x in rng.integers(1, 400, 3))
    if rng.random() < 0.3:
        K = int(rng.integers(200, 1200))
    ta, tb = bool(rng.random() < 0.3), bool(rng.random() < 0.5)
    mode = MODES[int(rng.integers(0, len(MODES)))]
    alpha = float(rng.choice([1.0, 0.5, -1.75]))
    beta = float(rng.choice([0.0, 0.0, 1.0, -0.5]))
    with_bias = bool(rng.random() < 0.4)
    pad = [int(rng.choice([0, 0, 4, 7])) for _ in range(3)]
    off = [int(rng.choice([0, 0, 0, 1])) for _ in range(3)]
    split = "none"
    if mode not in ("NATIVE_F32", "AUTO"):
        split = str(rng.choice(["none", "auto", "explicit"]))
    return dict(M=M, N=N, K=K, ta=ta, tb=tb, mode=mode, alpha=alpha, beta=beta, bias=with_bias,
                pad=pad, off=off, split=split)


def _device_matrix(torch, dev, x, pad, off):
    """x (rows x cols, float32) on the device with leading dimension cols +
    pad, starting `off` floats into its allocation."""
    rows, cols = x.shape
    ld = cols + pad
    buf = torch.zeros(off + rows * ld + 1, device=dev)
    view = buf[off:off + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(torch.from_numpy(np.ascontiguousarray(x)).to(dev))
    return view


def _fused(c):
    """The emulated kernel splits A itself (and may split K) only for a
    k-contiguous, 16-byte addressable A."""
    lda = c["K"] + c["pad"][0]
    return not c["ta"] and c["off"][0] == 0 and lda % 4 == 0 and c["K"] % 4 == 0


def _split_mask(M, N, plan):
    S, th, sf = plan
    tiles_n = -(-N // 128)
    tile = (np.arange(M)[:, None] // th) * tiles_n + np.arange(N)[None, :] // 128
    return tile >= sf


def test_random_calls_bitwise():
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(2026)
    for n in range(N_CASES):
        c = _case(rng)
        M, N, K = c["M"], c["N"], c["K"]
        a = (rng.standard_normal((M, K)) * 2.0 ** rng.integers(-6, 6, (M, K))).astype(np.float32)
        b = rng.standard_normal((K, N)).astype(np.float32)
        cin = rng.standard_normal((M, N)).astype(np.float32)
        bias = rng.standard_normal(N).astype(np.float32) if c["bias"] else None
        mode = c["mode"]
        run_mode = emu.select_mode(M, N, K, c["ta"], c["tb"]) if mode == "AUTO" else mode
        # the K split the call asks for, and the plan the library runs
        ksplit, plan = None, (1, 128, 0)
        if c["split"] == "auto":
            ksplit = emu.KSPLIT_AUTO
        elif c["split"] == "explicit":
            nk = -(-K // 32)
            divs = [s for s in range(2, 9) if nk % s == 0]
            if divs and _fused(c):
                ksplit = int(rng.choice(divs))
        if run_mode != "NATIVE_F32" and _fused(c):
            if ksplit == emu.KSPLIT_AUTO or mode == "AUTO":
                plan = emu.select_plan(M, N, K)
            elif ksplit is not None:
                plan = (ksplit, 128, 0)
        label = (f"case {n}: {M}x{N}x{K} t{int(c['ta'])}{int(c['tb'])} {mode}->{run_mode} "
                 f"alpha {c['alpha']} beta {c['beta']} bias {c['bias']} pad {c['pad']} off {c['off']} "
                 f"split {c['split']} plan {plan}")
        say(label)
        ga = _device_matrix(torch, dev, a.T if c["ta"] else a, c["pad"][0], c["off"][0])
        gb = _device_matrix(torch, dev, b.T if c["tb"] else b, c["pad"][1], c["off"][1])
        gc = _device_matrix(torch, dev, cin, c["pad"][2], c["off"][2])
        gbias = torch.from_numpy(bias).to(dev) if bias is not None else None
        out = emu.sgemm(ga, gb, mode=mode, trans_a=c["ta"], trans_b=c["tb"], alpha=c["alpha"],
                        beta=c["beta"], c=gc, bias=gbias, ksplit=ksplit)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        kw = dict(alpha=c["alpha"], beta=c["beta"], c=cin, bias=bias)
        if run_mode == "NATIVE_F32":
            want = oracle.native_gemm_mfma(a, b, **kw)
        else:
            want = oracle.emu_gemm_mfma(a, b, run_mode, **kw)
            if plan[0] > 1:
                split = oracle.emu_gemm_mfma(a, b, run_mode, ksplit=plan[0], **kw)
                want = np.where(_split_mask(M, N, plan), split, want)
        diff = got.view(np.uint32) != want.view(np.uint32)
        assert not diff.any(), (f"{label}: {int(diff.sum())} of {diff.size} differ, "
                                f"e.g. gpu {got[diff][:3]} model {want[diff][:3]}")


N_LARGE = 16


def _large_case(rng, n):
    if n % 4 == 3:
        # shapes of a few rounds of tiles and a long K, where the AUTO plan
        # tends to split the last round: an explicit emulated mode with
        # EMU_KSPLIT_AUTO on a k-contiguous A
        tiles_n = int(rng.integers(7, 12))
        tiles_m = -(-int(rng.integers(280, 400)) // tiles_n)     # 1.1-1.6 rounds of 256 tiles
        M = tiles_m * 128 - int(rng.integers(0, 128))
        N = tiles_n * 128 - int(rng.integers(0, 128))
        K = int(rng.integers(128, 384)) * 4
        return dict(M=M, N=N, K=K, ta=False, tb=bool(rng.random() < 0.5),
                    mode=MODES[int(rng.integers(1, 5))], alpha=float(rng.choice([1.0, -0.5])),
                    beta=float(rng.choice([0.0, 1.0])), bias=bool(rng.random() < 0.5),
                    pad=[int(rng.choice([0, 4])) for _ in range(3)], off=[0, 0, 0], split="auto")
    M = int(rng.integers(2000, 40000))
    N = int(rng.choice([int(rng.integers(64, 700)), int(rng.integers(700, 5000))]))
    K = int(rng.choice([int(rng.integers(32, 300)), int(rng.integers(300, 1500))]))
    if rng.random() < 0.5:
        K -= K % 4                     # k-contiguous A that the kernel splits itself
    return dict(M=M, N=N, K=max(K, 4), ta=bool(rng.random() < 0.2), tb=bool(rng.random() < 0.5),
                mode=MODES[int(rng.integers(0, len(MODES)))], alpha=float(rng.choice([1.0, -0.5])),
                beta=float(rng.choice([0.0, 1.0])), bias=bool(rng.random() < 0.4),
                pad=[int(rng.choice([0, 4])) for _ in range(3)], off=[0, 0, 0],
                split=str(rng.choice(["none", "auto"])))


def test_random_large_calls_sampled_rows():
    """16 seeded calls of up to 40,000 x 5,000 x 1,500: many rounds of tiles
    per workgroup, the tile heights AUTO picks and, on every fourth call
    (a few rounds of tiles, K >= 512, EMU_KSPLIT_AUTO), the plan's split of
    the last round of tiles.  Sampled rows (the first and last, both sides of tile-row
    boundaries, random ones) are compared bit for bit with the oracle's
    model of those rows."""
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7)
    for n in range(N_LARGE):
        c = _large_case(rng, n)
        M, N, K = c["M"], c["N"], c["K"]
        mode = c["mode"]
        if mode == "NATIVE_F32" or mode == "AUTO":
            c["split"] = "none"
        a = rng.standard_normal((M, K)).astype(np.float32)
        b = rng.standard_normal((K, N)).astype(np.float32)
        cin = rng.standard_normal((M, N)).astype(np.float32)
        bias = rng.standard_normal(N).astype(np.float32) if c["bias"] else None
        run_mode = emu.select_mode(M, N, K, c["ta"], c["tb"]) if mode == "AUTO" else mode
        ksplit = emu.KSPLIT_AUTO if c["split"] == "auto" else None
        plan = (1, 128, 0)
        if run_mode != "NATIVE_F32" and _fused(c) and (ksplit == emu.KSPLIT_AUTO or mode == "AUTO"):
            plan = emu.select_plan(M, N, K)
        rows = np.unique(np.r_[0, M - 1, np.arange(63, M, 64)[::max(1, M // 64 // 12)],
                               np.arange(64, M, 64)[::max(1, M // 64 // 12)], rng.integers(0, M, 8)])
        label = (f"large case {n}: {M}x{N}x{K} t{int(c['ta'])}{int(c['tb'])} {mode}->{run_mode} "
                 f"alpha {c['alpha']} beta {c['beta']} bias {c['bias']} pad {c['pad']} split {c['split']} "
                 f"plan {plan} rows {rows.size}")
        say(label)
        ga = _device_matrix(torch, dev, a.T if c["ta"] else a, c["pad"][0], 0)
        gb = _device_matrix(torch, dev, b.T if c["tb"] else b, c["pad"][1], 0)
        gc = _device_matrix(torch, dev, cin, c["pad"][2], 0)
        gbias = torch.from_numpy(bias).to(dev) if bias is not None else None
        out = emu.sgemm(ga, gb, mode=mode, trans_a=c["ta"], trans_b=c["tb"], alpha=c["alpha"],
                        beta=c["beta"], c=gc, bias=gbias, ksplit=ksplit)
        torch.cuda.synchronize()
        got = out.cpu().numpy()[rows]
        del ga, gb, gc, out
        kw = dict(alpha=c["alpha"], beta=c["beta"], c=cin[rows], bias=bias)
        if run_mode == "NATIVE_F32":
            want = oracle.native_gemm_mfma(a[rows], b, **kw)
        else:
            want = oracle.emu_gemm_mfma(a[rows], b, run_mode, **kw)
            if plan[0] > 1:
                split = oracle.emu_gemm_mfma(a[rows], b, run_mode, ksplit=plan[0], **kw)
                S, th, sf = plan
                tiles_n = -(-N // 128)
                mask = (rows[:, None] // th) * tiles_n + np.arange(N)[None, :] // 128 >= sf
                want = np.where(mask, split, want)
        diff = got.view(np.uint32) != want.view(np.uint32)
        assert not diff.any(), (f"{label}: {int(diff.sum())} of {diff.size} differ, "
                                f"e.g. gpu {got[diff][:3]} model {want[diff][:3]}")
