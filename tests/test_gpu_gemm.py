"""GPU parity of emu_sgemm (all modes, all transpose pairs) against the oracle.

Every case compares the HIP result with the FP64 oracle element by element
(componentwise bound) and normwise (err_F rules); closed forms are checked
bit for bit.  See gpu_helpers for the pass rules.  Workloads are the seeded
synthetic stand-ins of the MLIP systems (synth).
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import MODES, FLT_MAX, check_result, err_f, op, run, say

pytestmark = pytest.mark.gpu

TRANS = list(itertools.product([False, True], [False, True]))


def _store(op_x, t):
    return np.ascontiguousarray(op_x.T if t else op_x)


def _x9_rules(errs, label):
    assert errs["BF16X9"] <= 2e-6, f"{label}: err_F(BF16X9) {errs['BF16X9']:.3e} > 2e-6"
    assert errs["BF16X9"] <= 1.5 * errs["NATIVE_F32"], (
        f"{label}: err_F(BF16X9) {errs['BF16X9']:.3e} > 1.5 x native {errs['NATIVE_F32']:.3e}")


# ---------------------------------------------------------------- workloads 0, 1

def test_config0_all_modes():
    g = synth.gemms(0)[0]
    a, b = synth.make_a(g), synth.make_b(g)
    ref = oracle.gemm_f64(a, b)
    errs = {}
    for mode in MODES:
        say(f"config0 256^3 {mode}")
        out = run(a, b, mode)
        errs[mode], _ = check_result(out, ref, a, b, mode, label="config0")
    say("config0 err_F", errs)
    _x9_rules(errs, "config0")
    assert errs["BF16X3"] > errs["BF16X6"]
    assert errs["BF16X6"] >= 0.99 * errs["BF16X9"]
    model = oracle.emu_gemm(a, b, "BF16X9")
    say("config0 oracle model err_F", err_f(model, ref))


def test_config1_stress_all_modes():
    g = synth.gemms(1)[0]
    a, b = synth.make_a(g), synth.make_b(g)
    say("config1 oracle fp64 2048^3")
    ref = oracle.gemm_f64(a, b)
    n_over = int((np.abs(ref) > FLT_MAX).sum())
    errs = {}
    for mode in MODES:
        say(f"config1 stress 2048^3 {mode}")
        out = run(a, b, mode)
        errs[mode], _ = check_result(out, ref, a, b, mode, label="config1")
    say("config1 err_F", errs, "overflowed entries", n_over)
    _x9_rules(errs, "config1")
    assert errs["BF16X3"] > errs["BF16X6"]
    assert errs["BF16X6"] >= 0.99 * errs["BF16X9"]


# ---------------------------------------------------------------- layer stacks

def _stack_case(cfg, gi, modes):
    g = synth.gemms(cfg)[gi]
    a, b = synth.make_a(g), synth.make_b(g)
    a_op, b_op = op(a, g.trans_a), op(b, g.trans_b)
    say(f"config{cfg} {g.name} M={g.M} N={g.N} K={g.K} oracle")
    ref = oracle.gemm_f64(a, b, g.trans_a, g.trans_b)
    errs = {}
    for mode in modes:
        say(f"config{cfg} {g.name} {mode}")
        out = run(a, b, mode, g.trans_a, g.trans_b)
        errs[mode], _ = check_result(out, ref, a_op, b_op, "BF16X9" if mode == "AUTO" else mode,
                                     label=f"config{cfg} {g.name}")
    say(f"config{cfg} {g.name} err_F", errs)
    _x9_rules(errs, f"config{cfg} {g.name}")
    return errs


@pytest.mark.parametrize("gi", range(8))
def test_config2_stack(gi):
    _stack_case(2, gi, ("NATIVE_F32", "BF16X9", "AUTO"))


@pytest.mark.parametrize("gi", range(8))
def test_config4_stack(gi):
    errs = _stack_case(4, gi, ("NATIVE_F32", "BF16X9", "BF16X6", "AUTO"))
    assert errs["BF16X6"] <= 2e-6


@pytest.mark.parametrize("gi", range(8))
def test_config3_full_size_sampled(gi):
    """552,960-row GEMMs at full size, in the launch configuration the
    benchmark times; the oracle checks a fixed 1-in-64 row sample (plus the
    last row), each sampled row element by element."""
    import torch

    import emulated_fp32_matrix_amd as emu

    g = synth.gemms(3)[gi]
    say(f"config3 {g.name} M={g.M} N={g.N} K={g.K}: generating inputs")
    a = synth.make_a(g)
    b = synth.make_b(g)
    rows = synth.sample_rows(g.M, 64, gi)
    dev = torch.device("cuda:0")
    ad = torch.from_numpy(a).to(dev)
    bd = torch.from_numpy(b).to(dev)
    del a
    ref = oracle.gemm_f64(synth.make_a(g, rows=rows), b, g.trans_a, g.trans_b)
    a_rows = synth.make_a(g, rows=rows)
    errs = {}
    for mode in ("NATIVE_F32", "BF16X9"):
        say(f"config3 {g.name} {mode}")
        c = emu.sgemm(ad, bd, mode=mode, trans_a=g.trans_a, trans_b=g.trans_b)
        torch.cuda.synchronize()
        out = c[torch.from_numpy(rows).to(dev)].cpu().numpy()
        del c
        errs[mode], _ = check_result(out, ref, a_rows, op(b, g.trans_b), mode,
                                     label=f"config3 {g.name}")
    say(f"config3 {g.name} sampled err_F", errs)
    _x9_rules(errs, f"config3 {g.name}")


# ---------------------------------------------------------------- shapes, layouts

SHAPES = [(1, 1, 1), (7, 5, 3), (31, 33, 17), (32, 32, 16), (128, 128, 32), (129, 127, 33),
          (200, 300, 100), (257, 130, 260), (64, 512, 40), (300, 64, 700), (1000, 20, 9)]


@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("mode", MODES)
def test_shapes_and_transposes(ta, tb, mode):
    rng = np.random.default_rng(17)
    for M, N, K in SHAPES:
        a_op = rng.standard_normal((M, K)).astype(np.float32)
        b_op = rng.standard_normal((K, N)).astype(np.float32)
        ref = oracle.gemm_f64(a_op, b_op)
        say(f"shape {M}x{N}x{K} ta={ta} tb={tb} {mode}")
        out = run(_store(a_op, ta), _store(b_op, tb), mode, ta, tb)
        check_result(out, ref, a_op, b_op, mode, label=f"{M}x{N}x{K} {ta}{tb}")


@pytest.mark.parametrize("mode", ["NATIVE_F32", "BF16X9", "BF16X3"])
def test_unaligned_and_odd_leading_dims(mode):
    """Pointers off 16-byte alignment and leading dimensions that are not
    multiples of 4 take the scalar load path; results must not change."""
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(3)
    M, N, K = 150, 70, 45
    for ta, tb in TRANS:
        a_op = rng.standard_normal((M, K)).astype(np.float32)
        b_op = rng.standard_normal((K, N)).astype(np.float32)
        A, B = _store(a_op, ta), _store(b_op, tb)
        base = run(A, B, mode, ta, tb)
        # embed in wider buffers with odd leading dimensions, shifted by one float
        lda, ldb, ldc = A.shape[1] + 3, B.shape[1] + 5, N + 1
        Abuf = np.zeros((A.shape[0], lda + 1), np.float32)
        Abuf[:, 1:1 + A.shape[1]] = A
        Bbuf = np.zeros((B.shape[0], ldb + 1), np.float32)
        Bbuf[:, 1:1 + B.shape[1]] = B
        ad = torch.from_numpy(Abuf.ravel()).to(dev)
        bd = torch.from_numpy(Bbuf.ravel()).to(dev)
        cd = torch.full((M * ldc + 1,), 7.0, dtype=torch.float32, device=dev)
        say(f"unaligned ta={ta} tb={tb} {mode}")
        st = emu.emu_sgemm(int(ta), int(tb), M, N, K, 1.0, ad.data_ptr() + 4, lda + 1,
                           bd.data_ptr() + 4, ldb + 1, 0.0, cd.data_ptr() + 4, ldc, mode,
                           torch.cuda.current_stream().cuda_stream)
        assert st == emu.STATUS_SUCCESS
        torch.cuda.synchronize()
        c = cd.cpu().numpy()[1:].reshape(M, ldc)
        assert np.array_equal(c[:, :N], base)
        assert np.all(c[:, N:] == 7.0)  # padding columns untouched


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("ta,tb", TRANS)
def test_identity_returns_a_bitwise(ta, tb):
    rng = np.random.default_rng(5)
    g = synth.gemms(1)[0]
    a = np.concatenate([rng.standard_normal((100, 160)).astype(np.float32),
                        synth.make_a(g)[:100, :160]])
    eye = np.eye(160, dtype=np.float32)
    h, m, _ = oracle.split_bf16x3(a)
    x3 = (oracle.bf16_bits_to_f64(h) + oracle.bf16_bits_to_f64(m) * 2.0**-8).astype(np.float32)
    for mode in MODES:
        say(f"identity ta={ta} tb={tb} {mode}")
        out = run(_store(a, ta), _store(eye, tb), mode, ta, tb)
        want = x3 if mode == "BF16X3" else a
        assert np.array_equal(out, want), f"{mode}: B = I must return {'hi + mid' if mode == 'BF16X3' else 'A'} exactly"


def test_integer_matrices_exact():
    rng = np.random.default_rng(6)
    for K in (1, 33, 256, 1024):
        a = rng.integers(-128, 129, (70, K)).astype(np.float32)
        b = rng.integers(-128, 129, (K, 50)).astype(np.float32)
        exact = (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float64)
        for mode in MODES:
            say(f"integer K={K} {mode}")
            out = run(a, b, mode)
            assert np.array_equal(out.astype(np.float64), exact), f"{mode} K={K}"


def _sym_inputs():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((190, 300)).astype(np.float32)
    b = rng.standard_normal((300, 140)).astype(np.float32)
    return a, b


@pytest.mark.parametrize("mode", MODES)
def test_determinism(mode):
    a, b = _sym_inputs()
    say(f"determinism {mode}")
    base = run(a, b, mode)
    for _ in range(10):
        assert np.array_equal(run(a, b, mode), base), f"{mode}: not deterministic"


@pytest.mark.parametrize("mode", MODES)
def test_power_of_two_scaling(mode):
    """emu(2^s A) == 2^s emu(A) bit for bit (no over- or underflow)."""
    a, b = _sym_inputs()
    base = run(a, b, mode)
    for s in (-24, 7, 40):
        say(f"scaling 2^{s} {mode}")
        out = run((a * np.float32(2.0**s)).astype(np.float32), b, mode)
        assert np.array_equal(out, (base * np.float32(2.0**s)).astype(np.float32)), (mode, s)


@pytest.mark.parametrize("mode", MODES)
def test_sign_symmetry(mode):
    """emu(-A) == -emu(A).  Bit for bit on the FP32 MFMA path; the bf16 MFMA
    accumulation is not sign-symmetric in its last bit, so there both
    results must meet the element-by-element bound and the mismatch count is
    reported."""
    a, b = _sym_inputs()
    say(f"sign symmetry {mode}")
    base = run(a, b, mode)
    neg = run(-a, b, mode)
    if mode == "NATIVE_F32":
        assert np.array_equal(neg, -base)
    else:
        ref = oracle.gemm_f64(a, b)
        check_result(base, ref, a, b, mode, label="+A")
        check_result(-neg, ref, a, b, mode, label="-A")
        n_diff = int((neg != -base).sum())
        say(f"sign symmetry {mode}: {n_diff} of {base.size} entries differ in the last bits")


def test_row_independence():
    """A row's result does not depend on the other rows (lets full-size
    results be checked on a row sample)."""
    rng = np.random.default_rng(9)
    a = rng.standard_normal((1000, 256)).astype(np.float32)
    b = rng.standard_normal((256, 384)).astype(np.float32)
    rows = np.array([0, 5, 127, 128, 129, 500, 999])
    for mode in MODES:
        say(f"row independence {mode}")
        full = run(a, b, mode)
        part = run(a[rows], b, mode)
        assert np.array_equal(full[rows], part), mode


# ---------------------------------------------------------------- alpha, beta, edges

@pytest.mark.parametrize("mode", MODES)
def test_alpha_beta(mode):
    rng = np.random.default_rng(10)
    M, N, K = 140, 90, 70
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((K, N)).astype(np.float32)
    c = rng.standard_normal((M, N)).astype(np.float32)
    for alpha, beta in [(1.0, 1.0), (-0.5, 2.0), (3.0, -1.0)]:
        say(f"alpha={alpha} beta={beta} {mode}")
        out = run(a, b, mode, alpha=alpha, beta=beta, c_np=c)
        ref = oracle.gemm_f64(a, b, alpha=alpha, beta=beta, c=c)
        check_result(out, ref, a, b, mode, alpha, beta, c, label="alpha/beta")
    say(f"beta=0 with NaN C {mode}")
    out = run(a, b, mode, beta=0.0, c_np=np.full((M, N), np.nan, np.float32))
    assert np.isfinite(out).all()


def test_k_zero_and_alpha_zero():
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    M, N = 33, 65
    c0 = np.random.default_rng(1).standard_normal((M, N)).astype(np.float32)
    for beta in (0.0, 2.5):
        say(f"K=0 beta={beta}")
        c = torch.from_numpy(c0).to(dev)
        st = emu.emu_sgemm(0, 0, M, N, 0, 1.0, 0, 1, 0, N, beta, c.data_ptr(), N, "BF16X9",
                           torch.cuda.current_stream().cuda_stream)
        assert st == emu.STATUS_SUCCESS
        torch.cuda.synchronize()
        assert np.array_equal(c.cpu().numpy(), (c0 * np.float32(beta)) if beta else np.zeros_like(c0))
    a = np.ones((M, 8), np.float32)
    b = np.ones((8, N), np.float32)
    say("alpha=0")
    out = run(a, b, "BF16X9", alpha=0.0, beta=0.5, c_np=c0)
    assert np.array_equal(out, c0 * np.float32(0.5))


def test_nonfinite_inputs_propagate():
    a = np.random.default_rng(2).standard_normal((64, 64)).astype(np.float32)
    b = np.random.default_rng(3).standard_normal((64, 64)).astype(np.float32)
    a[3, 5] = np.nan
    a[10, 7] = np.inf
    for mode in MODES + ("BF16X1",):
        say(f"non-finite {mode}")
        out = run(a, b, mode)
        assert not np.isfinite(out[3]).any() and not np.isfinite(out[10]).any(), mode
        others = np.delete(out, [3, 10], axis=0)
        assert np.isfinite(others).all(), mode


def test_auto_matches_selected_mode():
    import emulated_fp32_matrix_amd as emu

    rng = np.random.default_rng(11)
    for M, N, K in [(4096, 256, 256), (64, 64, 8), (2000, 1000, 600)]:
        a = rng.standard_normal((M, K)).astype(np.float32)
        b = rng.standard_normal((K, N)).astype(np.float32)
        chosen = emu.select_mode(M, N, K)
        say(f"AUTO {M}x{N}x{K} -> {chosen}")
        assert np.array_equal(run(a, b, "AUTO"), run(a, b, chosen))


def test_inf_in_first_column_ragged_k():
    """Inf in column 0 of A with K not a multiple of 32: k past K must add
    exact zeros (the direct-load paths fill that part of the last k-step from
    column 0 and then zero it).  NATIVE_F32: the row is exactly the FP64
    result, +-Inf (B[0, j] != 0), not NaN.  The emulated modes' fused split
    gives Inf a finite hi (0x7F7F) and carries the Inf in a lower piece
    (lo' in BF16X9 and X6, mid' in BF16X3; BF16X1 keeps hi = Inf), whose
    products with B's pieces give Inf or NaN: there the row must be
    non-finite and the others finite."""
    rng = np.random.default_rng(12)
    for K in (36, 100, 260):
        a = rng.standard_normal((130, K)).astype(np.float32)
        b = rng.standard_normal((K, 140)).astype(np.float32)
        a[7, 0] = np.inf
        a[128, 0] = -np.inf
        with np.errstate(invalid="ignore", over="ignore"):
            ref = oracle.gemm_f64(a, b)
        for mode in MODES + ("BF16X1",):
            say(f"inf column 0 K={K} {mode}")
            out = run(a, b, mode)
            for r in (7, 128):
                if mode == "NATIVE_F32":
                    assert np.array_equal(out[r], ref[r].astype(np.float32)), (mode, K, r)
                else:
                    assert not np.isfinite(out[r]).any(), (mode, K, r)
            others = np.delete(out, [7, 128], axis=0)
            assert np.isfinite(others).all(), (mode, K)


@pytest.mark.parametrize("tb", [False, True])
def test_native_kernels_agree_bitwise(tb):
    """The native FP32 path has two kernels: the turn-taking one for a
    k-contiguous, 16-byte addressable A and the register-staged one for any
    other A (here: the same A one float off 16-byte alignment).  Both form
    every MFMA from the same k pair in the same order, so they agree bit for
    bit, on full and ragged tiles and with alpha, beta and a bias."""
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(13)
    for M, N, K in [(256, 256, 256), (300, 200, 100), (129, 385, 36), (1000, 128, 768)]:
        a = rng.standard_normal((M, K)).astype(np.float32)
        b_op = rng.standard_normal((K, N)).astype(np.float32)
        B = _store(b_op, tb)
        c0 = rng.standard_normal((M, N)).astype(np.float32)
        bias = rng.standard_normal(N).astype(np.float32)
        bd = torch.from_numpy(np.ascontiguousarray(B)).to(dev)
        biasd = torch.from_numpy(bias).to(dev)
        abuf = torch.zeros(M * K + 4, dtype=torch.float32, device=dev)
        abuf[4:] = torch.from_numpy(a.ravel()).to(dev)   # 16-byte aligned copy
        abuf2 = torch.zeros(M * K + 1, dtype=torch.float32, device=dev)
        abuf2[1:] = torch.from_numpy(a.ravel()).to(dev)  # 4 bytes off alignment
        outs = []
        for ptr in (abuf.data_ptr() + 16, abuf2.data_ptr() + 4):
            for alpha, beta, use_bias in [(1.0, 0.0, False), (-0.75, 1.5, True)]:
                cd = torch.from_numpy(c0).to(dev)
                say(f"native kernels {M}x{N}x{K} tb={tb} alpha={alpha} beta={beta} ptr%16={ptr % 16}")
                st = emu.emu_sgemm_bias(0, int(tb), M, N, K, alpha, ptr, K, bd.data_ptr(), B.shape[1], beta,
                                        cd.data_ptr(), N, biasd.data_ptr() if use_bias else 0, "NATIVE_F32",
                                        torch.cuda.current_stream().cuda_stream)
                assert st == emu.STATUS_SUCCESS
                torch.cuda.synchronize()
                outs.append(cd.cpu().numpy())
        assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3]), (M, N, K, tb)
        check_result(outs[0], oracle.gemm_f64(a, b_op), a, b_op, "NATIVE_F32", label=f"native {M}x{N}x{K}")


# ------------------------------------------------- leading dimensions past 2^31

BIG_LD = (1 << 24) + 64   # a 128-row tile of A (or 32 k-rows of B) spans more than 2^31 elements


@pytest.mark.parametrize("mode", list(MODES) + ["AUTO"])
@pytest.mark.parametrize("which", ["lda", "ldb_t", "ldc"])
def test_leading_dimensions_past_32bit_offsets(which, mode):
    """Huge leading dimensions (a tile of A, or of op(B) stored transposed,
    spanning more than 2^31 elements; or C rows 2^26 bytes apart): tiny
    shapes over 67 MB buffers.  Such A takes the pre-split path of the
    emulated modes and the 64-bit-offset staged kernel of NATIVE_F32, C the
    element-wise stores; the result equals the same product on compact
    operands bit for bit and the FP64 oracle within its bound."""
    import torch

    import emulated_fp32_matrix_amd as emu

    dev = torch.device("cuda:0")
    M, N, K = 3, 40, 72
    rng = np.random.default_rng(11)
    a = rng.standard_normal((M, K)).astype(np.float32)
    bop = rng.standard_normal((K, N)).astype(np.float32)
    tb = which == "ldb_t"
    say(f"leading dimension {which} = {BIG_LD}, {mode}")
    ga = torch.from_numpy(a).to(dev)
    gb = torch.from_numpy(np.ascontiguousarray(bop.T) if tb else bop).to(dev)
    want = emu.sgemm(ga, gb, mode=mode, trans_b=tb)
    if which == "lda":
        buf = torch.zeros((M - 1) * BIG_LD + K, device=dev)
        ga = buf.as_strided((M, K), (BIG_LD, 1))
        ga.copy_(torch.from_numpy(a).to(dev))
    elif which == "ldb_t":
        buf = torch.zeros((N - 1) * BIG_LD + K, device=dev)
        gb = buf.as_strided((N, K), (BIG_LD, 1))
        gb.copy_(torch.from_numpy(np.ascontiguousarray(bop.T)).to(dev))
    c = None
    if which == "ldc":
        cbuf = torch.full(((M - 1) * (BIG_LD + 32) + N,), float("nan"), device=dev)
        c = cbuf.as_strided((M, N), (BIG_LD + 32, 1))
    got = emu.sgemm(ga, gb, mode=mode, trans_b=tb, c=c)
    torch.cuda.synchronize()
    got, want = got.cpu().numpy(), want.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{which} {mode}: differs from compact"
    run_mode = emu.select_mode(M, N, K, False, tb) if mode == "AUTO" else mode
    check_result(got, oracle.gemm_f64(a, bop), a, bop, run_mode, label=f"{which} {mode}")
    if which == "ldc":   # nothing outside C's rows and columns written
        gap = cbuf.as_strided((M - 1, BIG_LD + 32 - N), (BIG_LD + 32, 1), N).cpu().numpy()
        assert np.isnan(gap).all()
