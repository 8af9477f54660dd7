"""GPU parity of the stand-alone split kernel (emu_split_bf16x3) against the
oracle: bit-exact on every input.

The split is Figure 1's three scaled BF16 pieces ("Unlocking Tensor Core
Performance for Machine Learning Interatomic Potentials", section "How Tensor
Core FP32 bridges the hardware gap"); the GEMM kernels stage their operands
with the same device routine, so this also checks the fused split.
"""
import numpy as np
import pytest

import oracle
import split_check
import synth
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _gpu_split(x_np, offset=0):
    """Split x on the GPU; `offset` elements of padding shift every pointer
    off 16-byte alignment."""
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    n = x_np.size
    xb = torch.zeros(n + offset, dtype=torch.float32, device=dev)
    xb[offset:] = torch.from_numpy(np.ascontiguousarray(x_np).ravel()).to(dev)
    planes = [torch.zeros(n + offset, dtype=torch.int16, device=dev) for _ in range(3)]
    x = xb[offset:]
    hi, mid, lo = (p[offset:] for p in planes)
    st = emu.emu_split_bf16x3(x.data_ptr(), n, hi.data_ptr(), mid.data_ptr(), lo.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    assert st == emu.STATUS_SUCCESS, emu.emu_status_string(st)
    torch.cuda.synchronize()
    return tuple(p.cpu().numpy().view(np.uint16) for p in (hi, mid, lo))


def _check(x_np, offset=0, label=""):
    say(f"split {label}: n={x_np.size} offset={offset}")
    got = _gpu_split(x_np, offset)
    want = oracle.split_bf16x3(np.ascontiguousarray(x_np).ravel())
    for name, g, w in zip(("hi", "mid", "lo"), got, want):
        bad = np.nonzero(g != w)[0]
        assert bad.size == 0, (f"{label} {name}: {bad.size} mismatches, first at input bits "
                               f"{hex(int(np.ascontiguousarray(x_np).ravel().view(np.uint32)[bad[0]]))}: "
                               f"gpu {hex(int(g[bad[0]]))} oracle {hex(int(w[bad[0]]))}")


def test_split_config0_inputs():
    g = synth.gemms(0)[0]
    _check(np.concatenate([synth.make_a(g).ravel(), synth.make_b(g).ravel()]), label="256^3 A,B")


def test_split_config1_inputs():
    g = synth.gemms(1)[0]
    _check(np.concatenate([synth.make_a(g).ravel(), synth.make_b(g).ravel()]), label="stress A,B")


def test_split_structured_patterns_and_specials():
    tops = np.arange(0, 2**16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x0080, 0x7F80, 0x4000, 0xC000,
                     0x1234, 0xFEDC], dtype=np.uint32)
    u = (tops[:, None] | lows[None, :]).ravel()  # includes +-0, subnormals, inf, NaNs
    _check(u.view(np.float32), label="structured")


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 15, 16, 17, 1023, 1025, 4099])
@pytest.mark.parametrize("offset", [0, 1, 3])
def test_split_ragged_and_unaligned(n, offset):
    rng = np.random.default_rng(n * 7 + offset)
    u = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    _check(u.view(np.float32), offset, label="ragged")


def test_split_sweep_of_bit_patterns():
    """Every one of the 2^32 FP32 bit patterns, in chunks of 2^26 made on the
    device: the GPU split equals the oracle's bit for bit, and its pieces pass
    the C range checker (exact reconstruction hi + 2^-8 mid' + 2^-16 lo' == a
    in float64, finite pieces, piece bounds, non-finite conventions).  Stops
    at the first failing chunk."""
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    chunk = 2**26
    planes = [torch.empty(chunk, dtype=torch.int16, device=dev) for _ in range(3)]
    stream = torch.cuda.current_stream().cuda_stream
    for c in range(2**32 // chunk):
        first = c * chunk
        bits = torch.arange(first, first + chunk, dtype=torch.int64, device=dev)
        bits = torch.where(bits >= 2**31, bits - 2**32, bits).to(torch.int32)
        x = bits.view(torch.float32)
        st = emu.emu_split_bf16x3(x.data_ptr(), chunk, *(p.data_ptr() for p in planes), stream)
        assert st == emu.STATUS_SUCCESS, emu.emu_status_string(st)
        got = [p.cpu().numpy().view(np.uint16) for p in planes]   # synchronises
        u = np.arange(first, first + chunk, dtype=np.uint64).astype(np.uint32)
        want = oracle.split_bf16x3(u.view(np.float32))
        for name, g, w in zip(("hi", "mid", "lo"), got, want):
            bad = np.nonzero(g != w)[0]
            assert bad.size == 0, (f"chunk {c} {name}: {bad.size} mismatches, first at bits "
                                   f"{hex(first + int(bad[0]))}: gpu {hex(int(g[bad[0]]))} "
                                   f"oracle {hex(int(w[bad[0]]))}")
        nbad, at = split_check.check_range(first, *got)
        assert nbad == 0, f"chunk {c}: {nbad} pieces fail the checker, first at bits {hex(first + at)}"
        if c % 8 == 7:
            say(f"split sweep: {c + 1} of {2**32 // chunk} chunks of 2^26 bit-exact")
