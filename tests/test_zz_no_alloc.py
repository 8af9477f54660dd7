"""GPU test of emu_sgemm_noalloc, the allocation-free variant of emu_sgemm_ex
for callers that cannot allocate (graph capture, serving loops): through
the C ABI, its results equal emu_sgemm_ex's bit for bit on two calls in a
row (the second smaller, in the scratch the first left behind), in every
mode and path that uses a workspace (pre-split B, pre-split A, split K,
NATIVE_F32's packed B), and a call that needs more than the scratch holds
is refused before any launch.
"""
import numpy as np
import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _call(fn, a, b, c, bias, M, N, K, ta, tb, mode, ksplit, alpha=1.0, beta=0.0):
    import torch

    lda = a.stride(0)
    ldb = b.stride(0)
    return fn(1 if ta else 0, 1 if tb else 0, M, N, K, alpha, a.data_ptr(), lda, b.data_ptr(), ldb,
              beta, c.data_ptr(), c.stride(0), bias.data_ptr() if bias is not None else 0, mode,
              ksplit, torch.cuda.current_stream().cuda_stream)


# (M, N, K, transA, transB, mode, ksplit, bias, alpha, beta): the second of
# each pair is the smaller call
CASES = [
    ((1000, 768, 256, False, False, "BF16X9", 0, True, 1.0, 0.0),
     (300, 256, 64, False, True, "BF16X9", 0, False, 1.0, 0.0)),
    ((700, 520, 300, True, False, "BF16X6", 0, False, 0.5, 1.5),     # A pre-split into the scratch
     (129, 33, 17, True, True, "BF16X6", 0, True, 1.0, 0.0)),
    ((2048, 512, 512, False, False, "BF16X9", 4, True, 1.0, 0.0),    # split K: partials in the scratch
     (640, 256, 256, False, False, "BF16X3", 2, False, 1.0, 0.0)),
    ((1500, 1024, 512, False, True, "NATIVE_F32", 0, False, 1.0, 0.0),  # packed op(B)
     (200, 100, 36, False, False, "NATIVE_F32", 0, True, 1.0, 0.0)),
    ((6144, 768, 256, False, False, "AUTO", 0, False, 1.0, 0.0),
     (6144, 256, 768, False, True, "AUTO", 0, True, 1.0, 0.0)),
    ((6144, 1024, 1024, False, False, "AUTO", 0, True, 1.0, 0.0),   # last round of tiles split
     (3300, 1200, 512, False, True, "BF16X6", -1, True, 0.5, 2.0)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_emu_sgemm_ex(first, second):
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    for i, (M, N, K, ta, tb, mode, ksplit, with_bias, alpha, beta) in enumerate((first, second)):
        say(f"noalloc call {i + 1}: {M}x{N}x{K} t{int(ta)}{int(tb)} {mode} ksplit={ksplit} "
            f"bias={with_bias} alpha={alpha} beta={beta}")
        g = torch.Generator(device="cpu").manual_seed(M * 31 + N * 7 + K)
        a = torch.randn((K, M) if ta else (M, K), generator=g).to(dev)
        b = torch.randn((N, K) if tb else (K, N), generator=g).to(dev)
        bias = torch.randn(N, generator=g).to(dev) if with_bias else None
        c0 = torch.randn((M, N), generator=g).to(dev)
        c_ref, c_new = c0.clone(), c0.clone()
        st = _call(emu.emu_sgemm_ex, a, b, c_ref, bias, M, N, K, ta, tb, mode, ksplit, alpha, beta)
        assert st == emu.STATUS_SUCCESS, emu.emu_status_string(st)
        st = _call(emu.emu_sgemm_noalloc, a, b, c_new, bias, M, N, K, ta, tb, mode, ksplit, alpha,
                   beta)
        assert st == emu.STATUS_SUCCESS, emu.emu_status_string(st)
        torch.cuda.synchronize()
        assert torch.isfinite(c_new).all()
        same = torch.equal(c_new.view(torch.int32), c_ref.view(torch.int32))
        assert same, f"call {i + 1}: {int((c_new != c_ref).sum())} entries differ from emu_sgemm_ex"


def test_noalloc_refuses_more_than_the_scratch():
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    # a split K of 4 segments needs 4 * M * N * 4 bytes = 96 MiB > 64 MiB
    M, N, K = 8192, 768, 256
    assert 4 * M * N * 4 > emu.NOALLOC_SCRATCH_BYTES
    a = torch.randn(M, K, device=dev)
    b = torch.randn(K, N, device=dev)
    c = torch.full((M, N), 7.0, device=dev)
    st = _call(emu.emu_sgemm_noalloc, a, b, c, None, M, N, K, False, False, "BF16X9", 4)
    assert st == emu.STATUS_SCRATCH_TOO_SMALL, emu.emu_status_string(st)
    assert emu.emu_status_string(st) == "EMU_STATUS_SCRATCH_TOO_SMALL"
    torch.cuda.synchronize()
    assert bool((c == 7.0).all()), "nothing may be launched"
    # the same shape without a split fits (B planes only) and matches emu_sgemm_ex
    c_ref = torch.empty_like(c)
    assert _call(emu.emu_sgemm_noalloc, a, b, c, None, M, N, K, False, False, "BF16X9", 0) == 0
    assert _call(emu.emu_sgemm_ex, a, b, c_ref, None, M, N, K, False, False, "BF16X9", 0) == 0
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), c_ref.view(torch.int32))
