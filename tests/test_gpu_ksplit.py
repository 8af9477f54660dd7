"""GPU parity of the split-K path (emu_sgemm_ex, and the plan the AUTO policy
chooses: a split of every tile or of the last round of tiles only): bit for
bit against the oracle's model of the same evaluation (oracle.emu_gemm_mfma
with ksplit: each K segment's emulated product t_s, summed in segment order
in FP32, then alpha, beta, bias; tiles a plan leaves whole without a split),
within the FP64 oracle's bound, and the error cases.

The split is for small GEMMs like the 192-atom system of "Unlocking Tensor
Core Performance for Machine Learning Interatomic Potentials", section
"BF16x9 on NVIDIA Blackwell GPUs" (Figures 3 and 4).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_result, say

pytestmark = pytest.mark.gpu


def _gpu(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _run(a, b, mode, ksplit, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, c=None, bias=None):
    import torch

    import emulated_fp32_matrix_amd as emu

    out = emu.sgemm(_gpu(a), _gpu(b), mode=mode, trans_a=trans_a, trans_b=trans_b, alpha=alpha,
                    beta=beta, c=None if c is None else _gpu(c),
                    bias=None if bias is None else _gpu(bias), ksplit=ksplit)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _same(out, model, label):
    diff = out.view(np.uint32) != model.view(np.uint32)
    n = int(diff.sum())
    assert n == 0, f"{label}: {n} of {model.size} differ, e.g. gpu {out[diff][:3]} model {model[diff][:3]}"
    say(f"{label}: {model.size} entries bitwise equal")


@pytest.mark.parametrize("M,N,K,S", [(256, 256, 256, 2), (300, 200, 256, 4), (129, 131, 256, 8),
                                     (200, 384, 200, 7), (64, 512, 96, 3), (500, 128, 1024, 32),
                                     (257, 260, 512, 1)])
def test_explicit_split_bitwise(M, N, K, S):
    rng = np.random.default_rng(M + 7 * N + 13 * K + S)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    _same(_run(a, b, "BF16X9", S), oracle.emu_gemm_mfma(a, b, "BF16X9", ksplit=S),
          f"{M}x{N}x{K} ksplit {S}")


@pytest.mark.parametrize("mode", ["BF16X9", "BF16X6", "BF16X3", "BF16X1"])
def test_split_every_mode_with_epilogue(mode):
    """alpha, beta and a bias with a split (the reduction applies them), with
    N a multiple of 4 (vector reduction) and not (element by element), and
    NT (the input-gradient layout)."""
    rng = np.random.default_rng(3)
    for M, N, K, tb in ((260, 384, 512, False), (131, 70, 256, True)):
        a = rng.standard_normal((M, K)).astype(np.float32)
        bop = rng.standard_normal((K, N)).astype(np.float32)
        c = rng.standard_normal((M, N)).astype(np.float32)
        bias = rng.standard_normal(N).astype(np.float32)
        b = np.ascontiguousarray(bop.T) if tb else bop
        out = _run(a, b, mode, 4, trans_b=tb, alpha=0.75, beta=-1.25, c=c, bias=bias)
        model = oracle.emu_gemm_mfma(a, bop, mode, alpha=0.75, beta=-1.25, c=c, bias=bias, ksplit=4)
        _same(out, model, f"{mode} {M}x{N}x{K} t0{int(tb)} ksplit 4 alpha/beta/bias")


def _split_mask(rows, N, plan):
    """Entries (rows x N) of the output tiles the plan splits: tiles of
    tile_rows x 128 numbered row by row, columns fastest, split from
    split_from on."""
    S, th, sf = plan
    tiles_n = -(-N // 128)
    tile = (np.asarray(rows)[:, None] // th) * tiles_n + np.arange(N)[None, :] // 128
    return tile >= sf


def _plan_model(rows, a, b, mode, plan, trans_b=False, c=None, **kw):
    """The oracle's model of rows `rows` of a call that runs `plan`: split
    tiles at ksplit S, the others without a split."""
    cr = None if c is None else c[rows]
    whole = oracle.emu_gemm_mfma(a[rows], b, mode, trans_b=trans_b, c=cr, **kw)
    if plan[0] == 1:
        return whole
    split = oracle.emu_gemm_mfma(a[rows], b, mode, trans_b=trans_b, c=cr, ksplit=plan[0], **kw)
    N = b.shape[0] if trans_b else b.shape[1]
    return np.where(_split_mask(rows, N, plan), split, whole)


@pytest.mark.parametrize("cfg", [2, 4])
def test_auto_policy_on_the_small_stacks(cfg):
    """EMU_MODE_AUTO on the small stacks: where it runs the emulation it runs
    the plan emu_sgemm_plan reports (a K split of every tile, of the last
    round of tiles only, or none) and equals the oracle's model of that plan
    (sampled rows, among them those around the first split tile); every
    GEMM stays within the FP64 oracle's bound.  An explicit BF16X9 call on
    the same shape does not split."""
    import torch

    import emulated_fp32_matrix_amd as emu

    for g in synth.gemms(cfg):
        a, b = synth.make_a(g), synth.make_b(g)
        mode = emu.select_mode(g.M, g.N, g.K)
        plan = emu.select_plan(g.M, g.N, g.K)
        out = emu.sgemm(_gpu(a), _gpu(b), mode="AUTO", trans_b=g.trans_b)
        eager = emu.sgemm(_gpu(a), _gpu(b), mode="BF16X9", trans_b=g.trans_b)
        torch.cuda.synchronize()
        out, eager = out.cpu().numpy(), eager.cpu().numpy()
        first_split_row = plan[2] // -(-g.N // 128) * plan[1]
        rows = np.unique(np.r_[np.arange(0, g.M, 61), g.M - 1,
                               np.clip(first_split_row + np.arange(-2, 3), 0, g.M - 1)])
        bop = np.ascontiguousarray(b.T) if g.trans_b else b
        _same(eager[rows], oracle.emu_gemm_mfma(a[rows], b, "BF16X9", trans_b=g.trans_b),
              f"workload {cfg} {g.name} BF16X9 rows {rows.size}")
        if mode == "BF16X9":
            model = _plan_model(rows, a, b, "BF16X9", plan, trans_b=g.trans_b)
            _same(out[rows], model, f"workload {cfg} {g.name} AUTO plan {plan} rows {rows.size}")
        check_result(out[rows], oracle.gemm_f64(a[rows], bop), a[rows], bop, mode,
                     label=f"workload {cfg} {g.name} AUTO ({mode}, plan {plan})")


@pytest.mark.parametrize("mode", ["BF16X9", "BF16X6", "BF16X3", "BF16X1"])
@pytest.mark.parametrize("M,N,K,tb", [(3300, 1200, 512, False), (3300, 1199, 512, True),
                                      (4489, 1030, 1024, False)])
def test_last_round_split_bitwise(mode, M, N, K, tb):
    """EMU_KSPLIT_AUTO on shapes whose plan splits only the last round of
    tiles (128-row tiles: 256 whole tiles, then 4 split ones; 64-row tiles:
    512 whole, then 127 split; the first split tile inside a row of tiles;
    M and N ragged; N a multiple of 4 or not: vector or element-wise
    reduction; NN and NT): with alpha, beta and a bias, whole tiles equal
    the model without a split, split tiles the model at ksplit S, bit for
    bit."""
    import emulated_fp32_matrix_amd as emu

    plan = emu.select_plan(M, N, K)
    tiles = -(-M // plan[1]) * -(-N // 128)
    assert plan[0] > 1 and 0 < plan[2] < tiles, f"{M}x{N}x{K}: plan {plan} splits no last round"
    rng = np.random.default_rng(M + N + K + int(tb))
    a = rng.standard_normal((M, K)).astype(np.float32)
    bop = rng.standard_normal((K, N)).astype(np.float32)
    b = np.ascontiguousarray(bop.T) if tb else bop
    c = rng.standard_normal((M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    out = _run(a, b, mode, emu.KSPLIT_AUTO, trans_b=tb, alpha=0.75, beta=-1.25, c=c, bias=bias)
    first_split_row = plan[2] // -(-N // 128) * plan[1]
    rows = np.unique(np.clip(np.r_[np.arange(0, M, 97), first_split_row - 1, first_split_row,
                                   first_split_row + 1, first_split_row + plan[1] - 1, M - 1], 0, M - 1))
    model = _plan_model(rows, a, b, mode, plan, trans_b=tb, c=c, alpha=0.75, beta=-1.25, bias=bias)
    mask = _split_mask(rows, N, plan)
    assert mask.any() and not mask.all()
    _same(out[rows], model, f"{mode} {M}x{N}x{K} t0{int(tb)} plan {plan} alpha/beta/bias")


def test_split_is_deterministic():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((640, 768)).astype(np.float32)
    b = rng.standard_normal((768, 256)).astype(np.float32)
    first = _run(a, b, "BF16X9", 3)
    for _ in range(3):
        assert np.array_equal(_run(a, b, "BF16X9", 3).view(np.uint32), first.view(np.uint32))


def test_split_not_supported_on_the_presplit_path():
    import emulated_fp32_matrix_amd as emu

    a = np.ones((64, 128), np.float32)
    b = np.ones((64, 32), np.float32)
    with pytest.raises(emu.EmuError) as e:
        _run(a, b, "BF16X9", 2, trans_a=True)   # op(A) transposed: A is pre-split
    assert e.value.status == emu.STATUS_NOT_SUPPORTED
    # ksplit = 0 and 1 are fine there
    want = oracle.emu_gemm_mfma(np.ascontiguousarray(a.T), b, "BF16X9")
    for S in (0, 1):
        assert np.array_equal(_run(a, b, "BF16X9", S, trans_a=True), want)
