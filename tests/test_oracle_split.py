"""Pins for the oracle's BF16 rounding and three-piece split (CPU only).

The split follows "Unlocking Tensor Core Performance for Machine Learning
Interatomic Potentials", section "How Tensor Core FP32 bridges the hardware
gap", Figure 1 (three scaled BF16 pieces per FP32 operand), under the reading
hi = R(a), mid' = R(2^8 (a - hi)), lo' = 2^8 (2^8 (a - hi) - mid') with R =
round-to-nearest-even, saturating.  The page prints no worked example, so the
oracle is pinned to what the mathematics fixes:

* exact reconstruction a == hi + 2^-8 mid' + 2^-16 lo' (checked in float64,
  independently of the oracle's code) over dense sweeps of bit patterns, and
  over all 2^32 patterns (the C range checker of split_check.c);
* the nearest-piece bounds |2^-8 mid'| <= ulp(hi)/2, |2^-16 lo'| <= ulp(2^-8 mid')/2;
* R itself against torch's FP32 -> BF16 conversion (a library routine, round
  to nearest even) wherever no saturation occurs;
* hand-derived special cases (below, each with its derivation);
* sign symmetry and the non-finite conventions.
"""
import numpy as np
import torch

import oracle
import split_check

F32_TOP = 0x7F7F8000  # |a| >= this rounds to BF16 infinity without saturation


def _bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def _from_bits(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def _ulp_bf16(v):
    """Spacing of BF16 numbers at magnitude |v| (float64 in, float64 out)."""
    v = np.abs(v)
    out = np.full(v.shape, 2.0**-133)
    norm = v >= 2.0**-126
    e = np.floor(np.log2(np.where(norm, v, 1.0)))
    out[norm] = np.exp2(e[norm] - 7)
    return out


def check_split_invariants(x):
    """Reconstruction and piece bounds for the finite entries of ``x``."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    hi, mid, lo = oracle.split_bf16x3(x)
    fin = np.isfinite(x)
    xf = x[fin].astype(np.float64)
    h = oracle.bf16_bits_to_f64(hi[fin])
    m = oracle.bf16_bits_to_f64(mid[fin]) * 2.0**-8
    low = oracle.bf16_bits_to_f64(lo[fin]) * 2.0**-16
    recon = h + m + low
    bad = np.nonzero(recon != xf)[0]
    assert bad.size == 0, f"reconstruction fails for bits {hex(_bits(x[fin][bad[0]])[()])}"
    unsat = np.abs(xf) < float(_from_bits(np.uint32(F32_TOP)))
    assert np.all(np.abs(m[unsat]) <= 0.5 * _ulp_bf16(h[unsat]))
    assert np.all(np.abs(low[unsat]) <= 0.5 * _ulp_bf16(m[unsat]))
    # every piece is finite for finite input
    assert np.all((hi[fin] & 0x7F80) != 0x7F80)
    assert np.all((mid[fin] & 0x7F80) != 0x7F80)
    assert np.all((lo[fin] & 0x7F80) != 0x7F80)
    return hi, mid, lo


# (input bits, hi, mid', lo'), each derived by hand from the definition:
HAND_CASES = [
    # 1.0 is a BF16 number: residual 0.
    (0x3F800000, 0x3F80, 0x0000, 0x0000),
    # 1/3 = 0xAAAAAB*2^-25: low half 0xAAAB > 0x8000 rounds up, hi = 0xAB0000*2^-25;
    # r1 = -21845*2^-25, 2^8 r1 = -0x5555*2^-17 -> 8 bits 0xAB*2^-10 (rounded up),
    # q = 43*2^-17, lo' = 43*2^-9.
    (0x3EAAAAAB, 0x3EAB, 0xBE2B, 0x3DAC),
    # pi: low half 0x0FDB < 0x8000 rounds down; 2^8 r1 = 4059*2^-14 -> 254*2^-10;
    # q = -5*2^-14, lo' = -5*2^-6.
    (0x40490FDB, 0x4049, 0x3E7E, 0xBDA0),
    # 0.1: rounds up; 2^8 r1 = -13107*2^-19 -> -205*2^-13; q = 13*2^-19, lo' = 13*2^-11.
    (0x3DCCCCCD, 0x3DCD, 0xBCCD, 0x3BD0),
    # 1 + 2^-8: exact tie between 1 and 1 + 2^-7, the even one is 1; mid' = 1.
    (0x3F808000, 0x3F80, 0x3F80, 0x0000),
    # 1 + 2^-8 + 2^-16: above the tie, rounds up to 1 + 2^-7; mid' = -(1 - 2^-8).
    (0x3F808080, 0x3F81, 0xBF7F, 0x0000),
    (0xBF808080, 0xBF81, 0x3F7F, 0x0000),
    # 1 - 2^-24 rounds up into the next binade: hi = 1, mid' = -2^-16.
    (0x3F7FFFFF, 0x3F80, 0xB780, 0x0000),
    # -0: hi keeps the sign, residuals are +0.
    (0x80000000, 0x8000, 0x0000, 0x0000),
    # FLT_MAX = (2^24-1)*2^104 would round to infinity: hi saturates to 0x7F7F,
    # 2^8 r1 = (2^16-1)*2^112 saturates too, lo' = 2^128 - 2^120 = 0x7F7F.
    (0x7F7FFFFF, 0x7F7F, 0x7F7F, 0x7F7F),
    # FLT_MIN is a BF16 number.
    (0x00800000, 0x0080, 0x0000, 0x0000),
    # 2^-149: hi = 0, 2^8 r1 = 2^-141 rounds to 0, lo' = 2^-133 (smallest BF16).
    (0x00000001, 0x0000, 0x0000, 0x0001),
]


def test_hand_derived_cases():
    x = _from_bits(np.array([c[0] for c in HAND_CASES], dtype=np.uint32))
    hi, mid, lo = oracle.split_bf16x3(x)
    for i, (xb, h, m, l) in enumerate(HAND_CASES):
        assert (int(hi[i]), int(mid[i]), int(lo[i])) == (h, m, l), hex(xb)


def test_nonfinite_conventions():
    x = _from_bits(np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x7F800001],
                            dtype=np.uint32))
    hi, mid, lo = oracle.split_bf16x3(x)
    assert [int(v) for v in hi] == [0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7FC0]
    assert not mid.any() and not lo.any()


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(123)
    u = rng.integers(0, 2**32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    # dense around ties: low half exactly 0x8000, 0x7FFF, 0x8001
    top = rng.integers(0, 2**16, size=300_000, dtype=np.uint64).astype(np.uint32) << 16
    u = np.concatenate([u, top | 0x8000, top | 0x7FFF, top | 0x8001, top])
    x = _from_bits(u)
    keep = np.isfinite(x) & ((u & 0x7FFFFFFF) < F32_TOP)
    x = x[keep]
    ours = oracle.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_round_saturates():
    u = np.array([F32_TOP, 0x7F7FFFFF, F32_TOP | 0x80000000, 0x7F7F7FFF], dtype=np.uint32)
    out = oracle.bf16_round(_from_bits(u))
    assert [int(v) for v in out] == [0x7F7F, 0x7F7F, 0xFF7F, 0x7F7F]


def test_sign_symmetry():
    """split(-a) is the negation of split(a), piece by piece (as values; a
    piece that rounds to zero keeps the sign of its residual)."""
    rng = np.random.default_rng(5)
    u = rng.integers(1, 0x7F800000, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    pos = _from_bits(u)
    for p, n in zip(oracle.split_bf16x3(pos), oracle.split_bf16x3(-pos)):
        vp, vn = oracle.bf16_bits_to_f64(p), oracle.bf16_bits_to_f64(n)
        assert np.array_equal(vn, -vp)
        nz = vp != 0
        assert np.array_equal(n[nz], p[nz] ^ 0x8000)


def test_reconstruction_structured_sweep():
    """Every (sign, exponent, top-7 mantissa) pattern with 24 low-half
    patterns: ties, near-ties, extremes and random halves."""
    tops = np.arange(0, 2**16, dtype=np.uint32) << 16
    rng = np.random.default_rng(7)
    lows = np.concatenate([np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x0080, 0x7F80],
                                    dtype=np.uint32),
                           rng.integers(0, 2**16, size=16, dtype=np.uint64).astype(np.uint32)])
    u = (tops[:, None] | lows[None, :]).ravel()
    check_split_invariants(_from_bits(u))


def test_reconstruction_random_sweep():
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2**32, size=8_000_000, dtype=np.uint64).astype(np.uint32)
    check_split_invariants(_from_bits(u))


def test_reconstruction_strided_sweep():
    """One bit pattern in 256 of the whole FP32 space (16.7 M values)."""
    u = (np.arange(0, 2**24, dtype=np.uint64) * 256 + 97).astype(np.uint32)
    check_split_invariants(_from_bits(u))


def test_checker_catches_wrong_pieces():
    """The range checker used by the exhaustive sweeps flags pieces that miss
    by one unit in any plane, a piece outside its bound, and wrong
    non-finite conventions."""
    u = np.arange(0x3F800000, 0x3F800000 + 4096, dtype=np.uint32)
    hi, mid, lo = oracle.split_bf16x3(_from_bits(u))
    assert split_check.check_range(0x3F800000, hi, mid, lo) == (0, -1)
    for plane in range(3):
        bad = [p.copy() for p in (hi, mid, lo)]
        bad[plane][100] ^= 1
        assert split_check.check_range(0x3F800000, *bad) == (1, 100), plane
    # a = 1 + 2^-8 + 2^-16: (1, 2^-8 + 2^-15, -2^-16) also reconstructs a, but
    # its hi is not the nearest BF16 (|2^-8 mid'| > ulp(1)/2 = 2^-8); the
    # split is (1 + 2^-7, -(2^-8 - 2^-16), 0)
    assert split_check.check_range(0x3F808080, [0x3F80], [0x3F81], [0xBF80]) == (1, 0)
    assert split_check.check_range(0x3F808080, [0x3F81], [0xBF7F], [0]) == (0, -1)
    assert split_check.check_range(0x7F800000, [0x7F7F], [0x7F7F], [0x7F80]) == (1, 0)
    assert split_check.check_range(0x7FC00000, [0x7FC0], [0], [0]) == (0, -1)


def test_reconstruction_exhaustive():
    """All 2^32 bit patterns, in chunks of 2^26, through the C range checker
    (reconstruction in float64, finite pieces, piece bounds, non-finite
    conventions); stops at the first failing chunk."""
    step = 2**26
    for c in range(2**32 // step):
        first = c * step
        u = np.arange(first, first + step, dtype=np.uint64).astype(np.uint32)
        hi, mid, lo = oracle.split_bf16x3(_from_bits(u))
        bad, at = split_check.check_range(first, hi, mid, lo)
        assert bad == 0, (f"chunk {c}: {bad} failures, first at bits {hex(first + at)}: "
                          f"{hex(int(hi[at]))} {hex(int(mid[at]))} {hex(int(lo[at]))}")
