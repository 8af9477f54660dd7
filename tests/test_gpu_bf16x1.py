"""GPU parity of the one-product mode BF16X1 (hi*hi only: both operands
rounded once to BF16, FP32 accumulation) against the oracle's one-band
model, and its place in the error ordering of the modes.

The one-pass analog of "Unlocking Tensor Core Performance for Machine
Learning Interatomic Potentials", section "TF32x3 on Ampere GPUs" (single
TF32 pass versus TF32x3).  Not FP32-accurate: its componentwise bound adds
2^-7 |A||B| for the dropped bands (each product loses at most about 2^-8 of
its size).
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_result, err_f, op, run, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ta,tb", list(itertools.product([False, True], [False, True])))
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (31, 33, 17), (129, 127, 33), (300, 260, 100),
                                   (256, 512, 256)])
def test_bf16x1_against_oracle(M, N, K, ta, tb):
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    out = run(np.ascontiguousarray(a.T) if ta else a, np.ascontiguousarray(b.T) if tb else b,
              "BF16X1", trans_a=ta, trans_b=tb)
    ref = oracle.gemm_f64(a, b)
    e, r = check_result(out, ref, a, b, "BF16X1", label=f"{M}x{N}x{K}")
    # the GPU sits at the one-band model's error level
    model = oracle.emu_gemm(a, b, "BF16X1")
    say(f"BF16X1 {M}x{N}x{K} t{int(ta)}{int(tb)}: err_F {e:.3e} (model {err_f(model, ref):.3e}), "
        f"bound ratio {r:.3f}")
    assert e <= 2.0 * err_f(model, ref) + 1e-7


def test_bf16x1_identity_is_bf16_rounding_bitwise():
    """B = I: every output is one product hi(a)*1 summed with zeros, i.e. the
    BF16 rounding of A (saturating, nearest even), bit for bit; the same
    holds on the pre-split path (A transposed)."""
    rng = np.random.default_rng(2)
    a = np.concatenate([rng.standard_normal((150, 96)),
                        rng.uniform(-1, 1, (150, 96)) * 2.0**rng.uniform(-30, 30, (150, 96))]
                       ).astype(np.float32)
    eye = np.eye(96, dtype=np.float32)
    hi = oracle.bf16_bits_to_f64(oracle.split_bf16x3(a)[0]).astype(np.float32)
    for ta in (False, True):
        out = run(np.ascontiguousarray(a.T) if ta else a, eye, "BF16X1", trans_a=ta)
        assert np.array_equal(out, hi), f"trans_a={ta}: {np.sum(out != hi)} mismatches"


def test_bf16x1_integers_exact():
    """Integers of magnitude <= 128 are BF16 numbers: one product is exact."""
    rng = np.random.default_rng(4)
    a = rng.integers(-128, 129, (200, 300)).astype(np.float32)
    b = rng.integers(-128, 129, (300, 130)).astype(np.float32)
    out = run(a, b, "BF16X1")
    assert np.array_equal(out.astype(np.int64), a.astype(np.int64) @ b.astype(np.int64))


@pytest.mark.parametrize("cfg", [0, 1])
def test_error_ordering_with_bf16x1(cfg):
    g = synth.gemms(cfg)[0]
    a, b = synth.make_a(g), synth.make_b(g)
    ref = oracle.gemm_f64(a, b)
    errs = {m: err_f(run(a, b, m), ref) for m in ("BF16X1", "BF16X3", "BF16X6", "BF16X9")}
    say(f"workload {cfg} err_F: " + ", ".join(f"{m} {e:.3e}" for m, e in errs.items()))
    assert errs["BF16X1"] > errs["BF16X3"] > errs["BF16X6"]
    assert errs["BF16X6"] >= 0.99 * errs["BF16X9"]
