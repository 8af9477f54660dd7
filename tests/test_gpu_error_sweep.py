"""Normwise error of every mode against the FP64 oracle as K grows.

The pages observe that the accuracy of multi-word emulation depends on the
matrix unit's internal arithmetic and shows at large inner dimensions
("Accurate Models of NVIDIA Tensor Cores", section "Results"), and the
emulation's claim is to match or beat native FP32 ("Unlocking Tensor Core
Performance for Machine Learning Interatomic Potentials", section
"Limitations and decision criteria").  This sweep checks, at every K from 64
to 16,384 and for two input distributions, that BF16X9 stays within the pass
rule (err_F <= 2e-6 and <= 1.5 x NATIVE_F32) and that the modes keep their
order (BF16X1 > BF16X3 > BF16X6 >= 0.99 BF16X9).  Run with -s to see the
table.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import err_f, run, say

pytestmark = pytest.mark.gpu

MODES = ("NATIVE_F32", "BF16X9", "BF16X6", "BF16X3", "BF16X1")
KS = (64, 256, 1024, 4096, 16384)


@pytest.mark.parametrize("dist", ["uniform", "normal"])
def test_error_versus_k(dist):
    rng = np.random.default_rng(21 if dist == "uniform" else 22)
    M = N = 128
    say(f"\nerr_F vs K, {dist} inputs, M = N = {M}")
    say("| K | " + " | ".join(MODES) + " | X9 / native |")
    say("|---|" + "---|" * (len(MODES) + 1))
    for K in KS:
        if dist == "uniform":
            a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
            b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        else:
            a = rng.standard_normal((M, K)).astype(np.float32)
            b = rng.standard_normal((K, N)).astype(np.float32)
        ref = oracle.gemm_f64(a, b)
        e = {m: err_f(run(a, b, m), ref) for m in MODES}
        say(f"| {K} | " + " | ".join(f"{e[m]:.3e}" for m in MODES) +
            f" | {e['BF16X9'] / e['NATIVE_F32']:.3f} |")
        assert e["BF16X9"] <= 2e-6 and e["BF16X9"] <= 1.5 * e["NATIVE_F32"], (K, e)
        assert e["BF16X1"] > e["BF16X3"] > e["BF16X6"] >= 0.99 * e["BF16X9"], (K, e)
