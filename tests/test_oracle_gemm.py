"""Pins for the oracle's FP64 reference GEMM and its emulated-GEMM model (CPU).

* ``gemm_f64`` is the plain FP64-accumulated definition; it is pinned to
  numpy's float64 matmul (an independent library routine) for every
  transpose pair, ragged shapes and alpha/beta, and to exact rational
  arithmetic on small cases.
* ``emu_gemm`` models the method of "Unlocking Tensor Core Performance for
  Machine Learning Interatomic Potentials", section "How Tensor Core FP32
  bridges the hardware gap", Figure 1 (nine products of three scaled BF16
  pieces, FP32 accumulation along five anti-diagonal bands) and Figure 2's
  three-product rule.  It is pinned by:
    - exact rational arithmetic on 4x4x4 cases: the nine products of the
      pieces, weighted by their band scale 2^-8j, sum exactly to the exact
      product (checked with Python fractions, no oracle code involved);
    - closed forms: B = I returns A exactly (X9, X6) and hi + 2^-8 mid'
      (X3); small-integer matrices return the exact product; negating A
      negates C; scaling A by 2^s scales C by 2^s;
    - a-priori componentwise error bounds against the FP64 reference:
      |C - C_ref| <= ((2K + 10) 2^-24 + d_P) (|A||B|), d_9 = 0,
      d_6 = 2^-22, d_3 = 2^-14;
    - ordering of the exact-band variant: err(X3) > err(X6) > err(X9), and
      the page's accuracy claim (section "Limitations and decision criteria":
      BF16x9 matches or beats native FP32) against numpy's float32 matmul.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

TRANS = list(itertools.product([False, True], [False, True]))
DELTA = {"BF16X9": 0.0, "BF16X6": 2.0**-22, "BF16X3": 2.0**-14, "BF16X1": 2.0**-7}


def _op(x, t):
    return x.T if t else x


def _store(op_x, t):
    """Stored array whose op() is ``op_x``."""
    return np.ascontiguousarray(op_x.T if t else op_x)


def _rand(rng, shape, dist="uniform"):
    if dist == "uniform":
        return rng.uniform(-1, 1, shape).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    return synth.stress_values(rng, shape)


def _frac(x):
    return Fraction(float(x))


@pytest.mark.parametrize("ta,tb", TRANS)
def test_gemm_f64_matches_numpy(ta, tb):
    rng = np.random.default_rng(1)
    for M, N, K in [(1, 1, 1), (7, 5, 3), (33, 65, 17), (130, 70, 129)]:
        a = _rand(rng, (M, K))
        b = _rand(rng, (K, N))
        c = _rand(rng, (M, N))
        A, B = _store(a, ta), _store(b, tb)
        ref = 0.75 * (a.astype(np.float64) @ b.astype(np.float64)) - 1.5 * c.astype(np.float64)
        out = oracle.gemm_f64(A, B, ta, tb, alpha=0.75, beta=-1.5, c=c)
        assert out.shape == (M, N)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        out0 = oracle.gemm_f64(A, B, ta, tb)  # beta = 0: C not read
        np.testing.assert_allclose(out0, a.astype(np.float64) @ b.astype(np.float64),
                                   rtol=1e-12, atol=1e-12)


def test_gemm_f64_exact_rationals():
    rng = np.random.default_rng(2)
    for _ in range(50):
        # dyadic inputs with few bits: every partial sum is exact in float64
        a = (rng.integers(-64, 64, (4, 4)) * 2.0 ** rng.integers(-8, 8, (4, 4))).astype(np.float32)
        b = (rng.integers(-64, 64, (4, 4)) * 2.0 ** rng.integers(-8, 8, (4, 4))).astype(np.float32)
        out = oracle.gemm_f64(a, b)
        for i in range(4):
            for j in range(4):
                exact = sum(_frac(a[i, k]) * _frac(b[k, j]) for k in range(4))
                assert Fraction(out[i, j]) == exact


def _pieces(x):
    h, m, l = oracle.split_bf16x3(x)
    return (oracle.bf16_bits_to_f64(h), oracle.bf16_bits_to_f64(m), oracle.bf16_bits_to_f64(l))


@pytest.mark.parametrize("dist", ["uniform", "normal", "stress", "smallint", "special"])
def test_nine_products_sum_exactly(dist):
    """sum_j 2^-8j sum_{u+v=j} a_u b_v == sum_k a_k b_k in exact arithmetic."""
    rng = np.random.default_rng(3)
    cases = 2000 if dist != "special" else 500
    for _ in range(cases):
        if dist == "smallint":
            a = rng.integers(-300, 300, (4, 4)).astype(np.float32)
            b = rng.integers(-300, 300, (4, 4)).astype(np.float32)
        elif dist == "special":
            pool = np.array([0.0, -0.0, 1.0, 1 / 3, np.pi, 0.1, 1 + 2**-8, 1 - 2**-24,
                             float(np.finfo(np.float32).tiny), 2.0**-149, 2.0**-130, 3.0e38,
                             -1.5e38, 65504.0], dtype=np.float32)
            a = rng.choice(pool, (4, 4)) * rng.choice([-1, 1], (4, 4)).astype(np.float32)
            b = rng.choice(pool, (4, 4)) * rng.choice([-1, 1], (4, 4)).astype(np.float32)
            a, b = a.astype(np.float32), b.astype(np.float32)
        else:
            a = _rand(rng, (4, 4), dist)
            b = _rand(rng, (4, 4), dist)
        pa, pb = _pieces(a), _pieces(b)
        for i, j in [(0, 0), (1, 2), (3, 3)]:
            exact = sum(_frac(a[i, k]) * _frac(b[k, j]) for k in range(4))
            bands = [Fraction(0)] * 5
            for k in range(4):
                for u in range(3):
                    for v in range(3):
                        bands[u + v] += _frac(pa[u][i, k]) * _frac(pb[v][k, j])
            total = sum(Fraction(1, 256**jb) * s for jb, s in enumerate(bands))
            assert total == exact


@pytest.mark.parametrize("ta,tb", TRANS)
def test_emu_exact_band_matches_rationals(ta, tb):
    """The exact-band model (FP64 band sums) equals the rational value of its
    kept bands for small, exactly representable cases."""
    rng = np.random.default_rng(4)
    for _ in range(30):
        a = _rand(rng, (4, 4))
        b = _rand(rng, (4, 4))
        pa, pb = _pieces(a), _pieces(b)
        for mode, nb in oracle.NBANDS.items():
            out = oracle.emu_gemm(_store(a, ta), _store(b, tb), mode, ta, tb, acc_f64=True)
            for i in range(4):
                for j in range(4):
                    exact = sum(_frac(pa[u][i, k]) * _frac(pb[v][k, j]) * Fraction(1, 256**(u + v))
                                for k in range(4) for u in range(3) for v in range(3) if u + v < nb)
                    assert abs(Fraction(out[i, j]) - exact) <= abs(exact) * Fraction(1, 2**50)


def _componentwise_ok(out, a, b, K, mode, alpha=1.0, beta=0.0, c=None):
    ref = oracle.gemm_f64(a, b, alpha=alpha, beta=beta, c=c)
    scale = np.abs(alpha) * (np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64))
    if beta != 0.0:
        scale = scale + np.abs(beta) * np.abs(c.astype(np.float64))
    bound = ((2 * K + 10) * 2.0**-24 + DELTA[mode]) * scale
    diff = np.abs(out.astype(np.float64) - ref)
    return bool(np.all(diff <= bound)), float(np.max(diff / np.where(bound > 0, bound, 1.0)))


@pytest.mark.parametrize("mode", ["BF16X9", "BF16X6", "BF16X3", "BF16X1"])
@pytest.mark.parametrize("ta,tb", TRANS)
def test_emu_componentwise_bound(mode, ta, tb):
    rng = np.random.default_rng(5)
    for M, N, K, dist in [(5, 3, 1, "uniform"), (40, 33, 67, "normal"), (64, 64, 300, "uniform"),
                          (48, 40, 96, "stress")]:
        a = _rand(rng, (M, K), dist)
        b = _rand(rng, (K, N), dist)
        out = oracle.emu_gemm(_store(a, ta), _store(b, tb), mode, ta, tb)
        ok, ratio = _componentwise_ok(out, a, b, K, mode)
        fin = np.isfinite(oracle.gemm_f64(a, b)) & (np.abs(oracle.gemm_f64(a, b)) < 3.4e38)
        assert fin.all() or dist == "stress"
        assert ok, f"{mode} {ta}{tb} {M}x{N}x{K} {dist}: bound ratio {ratio}"


def test_emu_alpha_beta():
    rng = np.random.default_rng(6)
    a, b, c = _rand(rng, (20, 30)), _rand(rng, (30, 25)), _rand(rng, (20, 25))
    for mode in oracle.NBANDS:
        out = oracle.emu_gemm(a, b, mode, alpha=-0.5, beta=2.0, c=c)
        ok, ratio = _componentwise_ok(out, a, b, 30, mode, alpha=-0.5, beta=2.0, c=c)
        assert ok, ratio
        c_nan = np.full_like(c, np.nan)
        out0 = oracle.emu_gemm(a, b, mode, beta=0.0, c=c_nan)  # C must not be read
        assert np.isfinite(out0).all()


@pytest.mark.parametrize("ta,tb", TRANS)
def test_emu_identity_closed_form(ta, tb):
    rng = np.random.default_rng(7)
    a = np.concatenate([_rand(rng, (40, 48), "normal"), _rand(rng, (40, 48), "stress")])
    eye = np.eye(48, dtype=np.float32)
    h, m, _ = _pieces(a)
    for mode in oracle.NBANDS:
        out = oracle.emu_gemm(_store(a, ta), _store(eye, tb), mode, ta, tb)
        if mode == "BF16X3":
            expect = (h + m * 2.0**-8).astype(np.float32)
            assert np.array_equal(expect.astype(np.float64), h + m * 2.0**-8)  # exact in FP32
            assert np.array_equal(out, expect)
        elif mode == "BF16X1":
            assert np.array_equal(out, h.astype(np.float32))   # A rounded once to BF16
        else:
            assert np.array_equal(out.view(np.uint32) & 0x7FFFFFFF, a.view(np.uint32) & 0x7FFFFFFF)
            assert np.array_equal(out, a)


def test_emu_integer_closed_form():
    rng = np.random.default_rng(8)
    for K in (1, 17, 256, 1024):
        a = rng.integers(-128, 129, (16, K)).astype(np.float32)
        b = rng.integers(-128, 129, (K, 12)).astype(np.float32)
        exact = a.astype(np.int64) @ b.astype(np.int64)
        for mode in oracle.NBANDS:
            out = oracle.emu_gemm(a, b, mode)
            assert np.array_equal(out.astype(np.int64), exact)


def test_emu_sign_and_power_of_two_scaling():
    rng = np.random.default_rng(9)
    a, b = _rand(rng, (30, 50), "normal"), _rand(rng, (50, 20), "normal")
    for mode in oracle.NBANDS:
        base = oracle.emu_gemm(a, b, mode)
        assert np.array_equal(oracle.emu_gemm(-a, b, mode), -base)
        for s in (-20, -3, 5, 30):
            sc = oracle.emu_gemm((a * np.float32(2.0**s)).astype(np.float32), b, mode)
            assert np.array_equal(sc, (base * np.float32(2.0**s)).astype(np.float32))


def _err_f(out, ref):
    return float(np.linalg.norm(out.astype(np.float64) - ref) / np.linalg.norm(ref))


def test_exact_band_error_ordering_and_accuracy_claim():
    rng = np.random.default_rng(10)
    for dist, shape in [("uniform", (96, 128, 80)), ("normal", (64, 200, 72)),
                        ("stress", (64, 96, 64))]:
        M, K, N = shape
        a, b = _rand(rng, (M, K), dist), _rand(rng, (K, N), dist)
        ref = oracle.gemm_f64(a, b)
        fin = np.isfinite(ref) & (np.abs(ref) <= float(np.finfo(np.float32).max))
        errs = {}
        for mode in oracle.NBANDS:
            out = oracle.emu_gemm(a, b, mode, acc_f64=True)
            d = (out - ref)[fin]
            errs[mode] = float(np.linalg.norm(d) / np.linalg.norm(ref[fin]))
        assert errs["BF16X1"] > errs["BF16X3"] > errs["BF16X6"] > errs["BF16X9"], (dist, errs)
        # with FP32 band accumulation, X9 is at least as accurate as FP32 matmul
        x9 = oracle.emu_gemm(a, b, "BF16X9")
        f32 = (a @ b).astype(np.float32)
        fin2 = fin & np.isfinite(f32) & np.isfinite(x9)
        e9 = float(np.linalg.norm((x9 - ref)[fin2]) / np.linalg.norm(ref[fin2]))
        e32 = float(np.linalg.norm((f32 - ref)[fin2]) / np.linalg.norm(ref[fin2]))
        assert e9 <= 1.5 * e32, (dist, e9, e32)


def test_emu_matches_fp64_on_config0():
    """Workload 0 through the model: within the pass rule of 2e-6."""
    g = synth.gemms(0)[0]
    a, b = synth.make_a(g), synth.make_b(g)
    ref = oracle.gemm_f64(a, b)
    out = oracle.emu_gemm(a, b, "BF16X9")
    assert _err_f(out, ref) <= 2e-6


# ---------------------------------------------------------------- bias (linear layer)

def test_bias_identity_closed_form():
    """B = I (K = N) makes the GEMM part exactly op(A) in every mode's band
    model (X9, X6) and in FP64; the bias is then one FP32 addition per entry
    (one FP64 addition for the reference), added to column j of every row.
    M != N, so a bias indexed by row instead of column would fail."""
    rng = np.random.default_rng(11)
    M, N = 7, 5
    a = rng.standard_normal((M, N)).astype(np.float32)
    eye = np.eye(N, dtype=np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    expect32 = (a + bias[None, :]).astype(np.float32)
    for mode in ("BF16X9", "BF16X6"):
        out = oracle.emu_gemm(a, eye, mode, bias=bias)
        assert out.dtype == np.float32 and np.array_equal(out, expect32), mode
    ref = oracle.gemm_f64(a, eye, bias=bias)
    assert np.array_equal(ref, a.astype(np.float64) + bias.astype(np.float64)[None, :])


def test_bias_with_zero_k_and_beta():
    """K = 0: the product is empty, so C = beta*C + bias exactly as written."""
    rng = np.random.default_rng(12)
    M, N = 4, 6
    a = np.zeros((M, 0), np.float32)
    b = np.zeros((0, N), np.float32)
    c = rng.standard_normal((M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    ref = oracle.gemm_f64(a, b, beta=0.5, c=c, bias=bias)
    assert np.array_equal(ref, 0.5 * c.astype(np.float64) + bias.astype(np.float64)[None, :])


def test_bias_matches_numpy_float64():
    rng = np.random.default_rng(13)
    a = rng.standard_normal((9, 13)).astype(np.float32)
    b = rng.standard_normal((13, 11)).astype(np.float32)
    bias = rng.standard_normal(11).astype(np.float32)
    ref = oracle.gemm_f64(a, b, bias=bias)
    want = a.astype(np.float64) @ b.astype(np.float64) + bias.astype(np.float64)
    assert np.max(np.abs(ref - want)) <= 1e-13 * np.max(np.abs(want))
