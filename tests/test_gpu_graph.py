"""Library calls captured in a HIP graph replay the eager results bit for bit.

A call allocates only when its stream's workspace is smaller than the call
needs, so calls on a stream whose workspace has already grown to their need
can be captured (emu_sgemm, emu_sgemm_bias, emu_sgemm_ex; emu_sgemm_noalloc
never allocates).  Each test captures a step of several calls (every mode,
K-split plans whose last round of tiles is split, the native path, bias and
beta != 0), then replays the graph four times.  Every output is cleared to
NaN (or C restored, where beta != 0) before a replay, and eager calls on
the same stream plus a synchronisation run between replays.  Every replay
must equal the eager results bit for bit.
"""
import numpy as np
import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu

# (M, N, K, transB, mode, ksplit, bias, alpha, beta)
STEP = [
    (6144, 768, 256, False, "AUTO", None, False, 1.0, 0.0),
    (6144, 256, 768, True, "AUTO", None, True, 1.0, 0.0),
    (6144, 1024, 1024, False, "AUTO", None, False, 1.0, 0.0),       # last round of tiles split
    (3300, 1200, 512, False, "BF16X9", -1, True, 0.75, -1.25),      # EMU_KSPLIT_AUTO, beta != 0
    (2048, 512, 512, False, "BF16X6", 4, False, 1.0, 0.0),          # every tile split
    (1500, 1024, 512, True, "NATIVE_F32", None, False, 1.0, 0.0),   # packed op(B)
    (700, 300, 129, False, "BF16X3", None, True, 1.0, 0.5),         # A pre-split (K % 4 != 0)
]


def _setup(torch, dev, rng):
    calls = []
    for (M, N, K, tb, mode, ksplit, with_bias, alpha, beta) in STEP:
        a = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(dev)
        b = torch.from_numpy(rng.standard_normal((N, K) if tb else (K, N)).astype(np.float32)).to(dev)
        c0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(dev)
        bias = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).to(dev) if with_bias else None
        calls.append(dict(M=M, N=N, K=K, tb=tb, mode=mode, ksplit=ksplit, a=a, b=b, c0=c0, c=c0.clone(),
                          bias=bias, alpha=alpha, beta=beta))
    return calls


def _reset(calls):
    for x in calls:
        if x["beta"] != 0.0:
            x["c"].copy_(x["c0"])
        else:
            x["c"].fill_(float("nan"))


def _check_replays(torch, s, calls, step, label):
    with torch.cuda.stream(s):
        _reset(calls)
        step()
    s.synchronize()
    ref = [x["c"].clone() for x in calls]
    assert all(bool(torch.isfinite(r).all()) for r in ref), f"{label}: eager outputs not finite"
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        _reset(calls)
    s.synchronize()
    with torch.cuda.graph(graph, stream=s):
        step()
    s.synchronize()
    for rep in range(4):
        with torch.cuda.stream(s):
            _reset(calls)
        s.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (x, r) in enumerate(zip(calls, ref)):
            same = torch.equal(x["c"].view(torch.int32), r.view(torch.int32))
            assert same, f"{label}: replay {rep}, call {i} ({x['M']}x{x['N']}x{x['K']} {x['mode']}) differs from eager"
        # eager work on the same stream between replays
        with torch.cuda.stream(s):
            _reset(calls)
            step()
        s.synchronize()
        for i, (x, r) in enumerate(zip(calls, ref)):
            assert torch.equal(x["c"].view(torch.int32), r.view(torch.int32)), f"{label}: eager call {i} after replay {rep}"
    say(f"{label}: 4 replays of {len(calls)} calls bitwise equal to eager")
    del graph


def test_captured_calls_replay_bitwise():
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    calls = _setup(torch, dev, np.random.default_rng(11))
    s = torch.cuda.Stream()

    def step():
        for x in calls:
            emu.sgemm(x["a"], x["b"], mode=x["mode"], trans_b=x["tb"], alpha=x["alpha"], beta=x["beta"],
                      c=x["c"], bias=x["bias"], stream=s, ksplit=x["ksplit"])

    # grow the stream's workspace to the step's need before the capture
    with torch.cuda.stream(s):
        for _ in range(2):
            step()
    s.synchronize()
    _check_replays(torch, s, calls, step, "emu_sgemm/_bias/_ex")


def test_captured_noalloc_calls_replay_bitwise():
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    calls = _setup(torch, dev, np.random.default_rng(12))
    s = torch.cuda.Stream()

    def step():
        for x in calls:
            st = emu.emu_sgemm_noalloc(
                emu.OP_N, emu.OP_T if x["tb"] else emu.OP_N, x["M"], x["N"], x["K"], x["alpha"],
                x["a"].data_ptr(), x["a"].stride(0), x["b"].data_ptr(), x["b"].stride(0), x["beta"],
                x["c"].data_ptr(), x["c"].stride(0), x["bias"].data_ptr() if x["bias"] is not None else 0,
                x["mode"], 0 if x["ksplit"] is None else x["ksplit"], s.cuda_stream)
            assert st == emu.STATUS_SUCCESS, emu.emu_status_string(st)

    _check_replays(torch, s, calls, step, "emu_sgemm_noalloc")
