"""Randomised argument validation of the GEMM entry points, on the host.

Every entry point validates its arguments before any HIP call (the contract
of include/emu_sgemm.h).  This test restates the header's rules as a small
Python model, draws argument sets with zero to three faults, and calls the
library only where the model says the call returns before touching a
device: an invalid set must give EMU_STATUS_INVALID_VALUE, a valid set with
an empty output (M or N zero) EMU_STATUS_SUCCESS.  Valid sets with work to
do are never called (their pointers are fake), so the test is safe on a
machine with a GPU as well.
"""
import numpy as np
import pytest

import emulated_fp32_matrix_amd as emu

FAKE = 0x1000
EMULATED = (1, 2, 3, 5)        # BF16X9, BF16X6, BF16X3, BF16X1
KSPLIT_AUTO = -1


def _valid(c, with_split):
    """The header's rules (Conventions, emu_sgemm_ex's ksplit)."""
    M, N, K = c["M"], c["N"], c["K"]
    if c["transA"] not in (0, 1) or c["transB"] not in (0, 1):
        return False
    if not 0 <= c["mode"] <= 5:
        return False
    if with_split:
        s = c["ksplit"]
        if s < KSPLIT_AUTO or (s != 0 and c["mode"] not in EMULATED):
            return False
        if s > 1 and (K == 0 or (-(-K // 32)) % s != 0):
            return False
    if M < 0 or N < 0 or K < 0:
        return False
    if c["lda"] < max(1, K if c["transA"] == 0 else M):
        return False
    if c["ldb"] < max(1, N if c["transB"] == 0 else K):
        return False
    if c["ldc"] < max(1, N):
        return False
    if M > 0 and N > 0:
        if c["C"] == 0:
            return False
        if K > 0 and (c["A"] == 0 or c["B"] == 0):
            return False
    return True


def _draw(rng, with_split):
    M, N, K = (int(x) for x in rng.integers(0, 300, 3))
    tA, tB = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    c = dict(transA=tA, transB=tB, M=M, N=N, K=K, alpha=1.0, beta=0.0,
             A=FAKE, B=FAKE, C=FAKE, lda=max(1, K if tA == 0 else M) + int(rng.integers(0, 3)),
             ldb=max(1, N if tB == 0 else K) + int(rng.integers(0, 3)), ldc=max(1, N) + int(rng.integers(0, 3)),
             mode=int(rng.choice([0, 1, 2, 3, 4, 5])), stream=0)
    if with_split:
        c["ksplit"] = int(rng.choice([0, 0, 1, KSPLIT_AUTO, 2, 3, 4]))
        if c["ksplit"] != 0 and c["mode"] not in EMULATED:
            c["mode"] = int(rng.choice(EMULATED))
    if rng.random() < 0.2:          # empty output
        c["M" if rng.random() < 0.5 else "N"] = 0
    faults = int(rng.choice([0, 1, 1, 2, 3]))
    for _ in range(faults):
        f = int(rng.integers(0, 9 if with_split else 8))
        if f == 0:
            c["transA" if rng.random() < 0.5 else "transB"] = int(rng.choice([-1, 2, 7]))
        elif f == 1:
            c["mode"] = int(rng.choice([-1, 6, 99]))
        elif f == 2:
            c[str(rng.choice(["M", "N", "K"]))] = -int(rng.integers(1, 5))
        elif f == 3:
            c["lda"] = int(rng.integers(0, max(1, c["lda"])))
        elif f == 4:
            c["ldb"] = int(rng.integers(0, max(1, c["ldb"])))
        elif f == 5:
            c["ldc"] = int(rng.integers(0, max(1, c["ldc"])))
        elif f == 6:
            c[str(rng.choice(["A", "B", "C"]))] = 0
        elif f == 7:
            c["alpha"] = float(rng.choice([0.0, -2.0]))   # not a fault: alpha and beta are free
        else:
            c["ksplit"] = int(rng.choice([-2, -5, 5, 6, 7, 8]))
    return c


@pytest.mark.parametrize("entry", ["emu_sgemm", "emu_sgemm_bias", "emu_sgemm_ex", "emu_sgemm_noalloc"])
def test_random_arguments_follow_the_header(entry):
    rng = np.random.default_rng({"emu_sgemm": 1, "emu_sgemm_bias": 2, "emu_sgemm_ex": 3,
                                 "emu_sgemm_noalloc": 4}[entry])
    with_split = entry in ("emu_sgemm_ex", "emu_sgemm_noalloc")
    counts = {"invalid": 0, "empty": 0, "not called": 0}
    for _ in range(3000):
        c = _draw(rng, with_split)
        valid = _valid(c, with_split)
        empty = c["M"] == 0 or c["N"] == 0
        if valid and not empty:
            counts["not called"] += 1
            continue
        args = dict(c)
        if entry != "emu_sgemm":
            args["bias"] = 0 if rng.random() < 0.5 else FAKE
        if not with_split:
            args.pop("ksplit", None)
        st = getattr(emu, entry)(**args)
        want = emu.STATUS_SUCCESS if valid else emu.STATUS_INVALID_VALUE
        assert st == want, (entry, c, emu.emu_status_string(st))
        counts["invalid" if not valid else "empty"] += 1
    # the draw reaches every outcome often
    assert counts["invalid"] > 1000 and counts["empty"] > 100 and counts["not called"] > 300, counts
