"""Weights split once (emu_presplit_b + emu_sgemm_presplit): the GEMM equals
the same call with op(B) split inside it (emu_sgemm_ex, same mode and K
split) bit for bit, and the oracle's model of the evaluation
(oracle.emu_gemm_mfma), for every emulated mode, ragged shapes, NN and NT
weights, the fused and pre-split A paths, alpha/beta/bias, explicit K
splits, and planes reused across many inputs.

The method's split of each operand into three scaled BF16 pieces:
"Unlocking Tensor Core Performance for Machine Learning Interatomic
Potentials", section "How Tensor Core FP32 bridges the hardware gap",
Figure 1.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _gpu(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _bits_equal(x, y, label):
    x, y = np.asarray(x), np.asarray(y)
    diff = x.view(np.uint32) != y.view(np.uint32)
    n = int(diff.sum())
    assert n == 0, f"{label}: {n} of {x.size} differ, e.g. {x[diff][:3]} vs {y[diff][:3]}"
    say(f"{label}: {x.size} entries bitwise equal")


@pytest.mark.parametrize("mode", ["BF16X9", "BF16X6", "BF16X3", "BF16X1"])
@pytest.mark.parametrize("M,N,K,tb", [(256, 256, 256, False), (300, 200, 96, True), (129, 131, 40, False),
                                      (64, 520, 1000, True), (1, 1, 1, False)])
def test_presplit_equals_split_in_call_and_model(mode, M, N, K, tb):
    import torch

    import emulated_fp32_matrix_amd as emu

    rng = np.random.default_rng(M * 7 + N * 3 + K + (5 if tb else 0))
    a = rng.standard_normal((M, K)).astype(np.float32)
    bop = rng.standard_normal((K, N)).astype(np.float32)
    b = np.ascontiguousarray(bop.T) if tb else bop
    da, db = _gpu(a), _gpu(b)
    pb = emu.presplit_b(db, mode=mode, trans_b=tb)
    out = emu.sgemm_presplit(da, pb)
    ref = emu.sgemm(da, db, mode=mode, trans_b=tb, ksplit=1)
    torch.cuda.synchronize()
    out, ref = out.cpu().numpy(), ref.cpu().numpy()
    _bits_equal(out, ref, f"{mode} {M}x{N}x{K} t0{int(tb)} presplit vs in-call split")
    _bits_equal(out, oracle.emu_gemm_mfma(a, bop, mode), f"{mode} {M}x{N}x{K} presplit vs model")


@pytest.mark.parametrize("mode", ["BF16X9", "BF16X3"])
def test_presplit_epilogue_split_and_prepacked_a(mode):
    """alpha/beta/bias; K split S = 2 and 4 (fused A); op(A) transposed (the
    pre-split A path, no K split) — each equal to the in-call split."""
    import torch

    import emulated_fp32_matrix_amd as emu

    rng = np.random.default_rng(11)
    M, N, K = 260, 384, 256
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((K, N)).astype(np.float32)
    c = rng.standard_normal((M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    da, db, dbias = _gpu(a), _gpu(b), _gpu(bias)
    pb = emu.presplit_b(db, mode=mode)
    for S in (1, 2, 4):
        out = emu.sgemm_presplit(da, pb, alpha=0.75, beta=-1.25, c=_gpu(c), bias=dbias, ksplit=S)
        ref = emu.sgemm(da, db, mode=mode, alpha=0.75, beta=-1.25, c=_gpu(c), bias=dbias, ksplit=S)
        torch.cuda.synchronize()
        _bits_equal(out.cpu().numpy(), ref.cpu().numpy(), f"{mode} alpha/beta/bias ksplit {S}")
    model = oracle.emu_gemm_mfma(a, b, mode, alpha=0.75, beta=-1.25, c=c, bias=bias, ksplit=4)
    _bits_equal(out.cpu().numpy(), model, f"{mode} alpha/beta/bias ksplit 4 vs model")
    at = _gpu(np.ascontiguousarray(a.T))
    out = emu.sgemm_presplit(at, pb, trans_a=True, bias=dbias)
    ref = emu.sgemm(at, db, mode=mode, trans_a=True, bias=dbias, ksplit=1)
    torch.cuda.synchronize()
    _bits_equal(out.cpu().numpy(), ref.cpu().numpy(), f"{mode} op(A) transposed")
    with pytest.raises(emu.EmuError) as e:   # the pre-split A path does not split K
        emu.sgemm_presplit(at, pb, trans_a=True, ksplit=2)
    assert e.value.status == emu.STATUS_NOT_SUPPORTED


def test_planes_reused_across_inputs():
    """One set of planes, many activations of different row counts, on two
    streams: every result equals the in-call split."""
    import torch

    import emulated_fp32_matrix_amd as emu

    rng = np.random.default_rng(2)
    K, N = 256, 768
    db = _gpu(rng.standard_normal((N, K)).astype(np.float32))   # NT: a weight stored out x in
    pb = emu.presplit_b(db, trans_b=True)
    s2 = torch.cuda.Stream()
    torch.cuda.synchronize()
    for i, M in enumerate((6144, 100, 4096, 257, 6144)):
        da = _gpu(rng.standard_normal((M, K)).astype(np.float32))
        with torch.cuda.stream(s2 if i % 2 else torch.cuda.current_stream()):
            out = emu.sgemm_presplit(da, pb)
            ref = emu.sgemm(da, db, trans_b=True, ksplit=1)
        torch.cuda.synchronize()
        _bits_equal(out.cpu().numpy(), ref.cpu().numpy(), f"reuse {i}: {M} rows")


def test_full_size_layer_gemm():
    """The 552,960-row qkv.fwd GEMM of the 17,280-atom stack: equal to the
    in-call split over the whole output."""
    import torch

    import emulated_fp32_matrix_amd as emu

    g = synth.gemms(3)[0]
    da, db = _gpu(synth.make_a(g)), _gpu(synth.make_b(g))
    pb = emu.presplit_b(db, trans_b=g.trans_b)
    out = emu.sgemm_presplit(da, pb)
    ref = emu.sgemm(da, db, trans_b=g.trans_b, ksplit=1)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    say(f"{g.name} {g.M}x{g.N}x{g.K}: presplit equals the in-call split on all {g.M * g.N} entries")
