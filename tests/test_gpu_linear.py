"""GPU parity of the bias epilogue (emu_sgemm_bias) and of EmuLinear.

The bias is the linear layer's y = x W^T + b ("Unlocking Tensor Core
Performance for Machine Learning Interatomic Potentials", section "TF32x3 on
Ampere GPUs"), added after alpha and beta in the GEMM epilogue.  References:
the FP64 oracle with its bias (element by element, within the GEMM's
componentwise bound plus one FP32 rounding of the sum), closed forms bit for
bit, and torch float64 on the CPU for the autograd layer.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import MODES, err_f, op, say

pytestmark = pytest.mark.gpu

DELTA = {"NATIVE_F32": 0.0, "BF16X9": 0.0, "BF16X6": 2.0**-22, "BF16X3": 2.0**-14}


def _gpu(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _run_bias(a, b, bias_np, mode, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, c=None,
              bias_offset=0):
    """emu_sgemm_bias with the bias at a float offset into a device buffer
    (offset 1 makes it 4-byte but not 16-byte aligned)."""
    import torch

    import emulated_fp32_matrix_amd as emu

    buf = torch.zeros(bias_np.size + bias_offset, dtype=torch.float32, device="cuda:0")
    buf[bias_offset:] = _gpu(bias_np)
    bias = buf[bias_offset:]
    out = emu.sgemm(_gpu(a), _gpu(b), mode=mode, trans_a=trans_a, trans_b=trans_b, alpha=alpha,
                    beta=beta, c=None if c is None else _gpu(c), bias=bias)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_bias(out, a_op, b_op, bias, mode, alpha=1.0, beta=0.0, c=None, label=""):
    ref = oracle.gemm_f64(np.ascontiguousarray(a_op), np.ascontiguousarray(b_op), alpha=alpha,
                          beta=beta, c=c, bias=bias)
    K = a_op.shape[1]
    scale = abs(alpha) * (np.abs(a_op).astype(np.float64) @ np.abs(b_op).astype(np.float64))
    if beta != 0.0:
        scale += abs(beta) * np.abs(c.astype(np.float64))
    # the GEMM's bound, then one FP32 rounding of the sum with the bias
    bound = ((2 * K + 10) * 2.0**-24 + DELTA[mode]) * scale + 2.0**-24 * (
        np.abs(ref) + scale + np.abs(bias.astype(np.float64))[None, :])
    diff = np.abs(out.astype(np.float64) - ref)
    worst = float(np.max(diff / bound))
    say(f"{label} {mode}: bound ratio {worst:.3f}, err_F {err_f(out, ref):.3e}")
    assert worst <= 1.0, f"{label} {mode}: bound ratio {worst:.3f}"
    return err_f(out, ref)


SHAPES = [(1, 1, 1), (31, 33, 17), (128, 128, 32), (129, 127, 33), (300, 260, 100), (257, 512, 96)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("mode", MODES)
def test_bias_against_oracle(M, N, K, mode):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    bias = rng.uniform(-2, 2, N).astype(np.float32)
    for ta, tb in ((False, False), (False, True), (True, False)):
        out = _run_bias(a.T.copy() if ta else a, b.T.copy() if tb else b, bias, mode,
                        trans_a=ta, trans_b=tb)
        _check_bias(out, a, b, bias, mode, label=f"{M}x{N}x{K} t{int(ta)}{int(tb)}")


@pytest.mark.parametrize("mode", MODES)
def test_bias_with_alpha_beta_and_unaligned_bias(mode):
    rng = np.random.default_rng(5)
    M, N, K = 260, 384, 64
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((K, N)).astype(np.float32)
    c = rng.standard_normal((M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    for off in (0, 1):   # 16-byte aligned (vector epilogue) and not (element by element)
        out = _run_bias(a, b, bias, mode, alpha=0.75, beta=-1.25, c=c, bias_offset=off)
        _check_bias(out, a, b, bias, mode, alpha=0.75, beta=-1.25, c=c, label=f"offset {off}")


@pytest.mark.parametrize("mode", ["NATIVE_F32", "BF16X9", "BF16X6"])
def test_bias_identity_bitwise(mode):
    """B = I: the GEMM part is A exactly (NATIVE_F32, BF16X9, BF16X6), so the
    result is the FP32 sum A + bias, bit for bit, bias along columns."""
    rng = np.random.default_rng(9)
    M, N = 300, 160
    a = rng.standard_normal((M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    want = oracle.emu_gemm(a, np.eye(N, dtype=np.float32), "BF16X9", bias=bias)
    assert np.array_equal(want, (a + bias[None, :]).astype(np.float32))
    for off in (0, 1):
        out = _run_bias(a, np.eye(N, dtype=np.float32), bias, mode, bias_offset=off)
        assert np.array_equal(out, want), f"{mode} offset {off}: {np.sum(out != want)} mismatches"


@pytest.mark.parametrize("mode", MODES)
def test_bias_quick_return_paths(mode):
    """K = 0 and alpha = 0 give C = beta*C + bias, each entry one FP32
    multiply and one FP32 add (beta = 0: C not read, NaN in C ignored)."""
    import torch

    import emulated_fp32_matrix_amd as emu

    rng = np.random.default_rng(3)
    M, N, K = 70, 90, 40
    c = rng.standard_normal((M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((K, N)).astype(np.float32)
    want = (np.float32(0.5) * c + bias[None, :]).astype(np.float32)
    out = _run_bias(a, b, bias, mode, alpha=0.0, beta=0.5, c=c)
    assert np.array_equal(out, want)
    out = _run_bias(np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32), bias, mode,
                    beta=0.5, c=c)
    assert np.array_equal(out, want)
    cn = _gpu(np.full((M, N), np.nan, np.float32))
    emu.sgemm(_gpu(a), _gpu(b), mode=mode, alpha=0.0, beta=0.0, c=cn, bias=_gpu(bias))
    torch.cuda.synchronize()
    assert np.array_equal(cn.cpu().numpy(), np.broadcast_to(bias, (M, N)))


# ---------------------------------------------------------------- EmuLinear

def _reference(x, w, bias, gy):
    """torch float64 on the CPU: y, and the gradients of sum(y * gy)."""
    import torch

    x64 = x.detach().cpu().double().requires_grad_(True)
    w64 = w.detach().cpu().double().requires_grad_(True)
    b64 = None if bias is None else bias.detach().cpu().double().requires_grad_(True)
    y = torch.nn.functional.linear(x64, w64, b64)
    (y * gy.cpu().double()).sum().backward()
    return y.detach(), x64.grad, w64.grad, None if b64 is None else b64.grad


def _rel(a, ref):
    a = a.detach().cpu().double()
    return float((a - ref).norm() / ref.norm())


@pytest.mark.parametrize("mode", ["BF16X9", "AUTO", "NATIVE_F32", "BF16X6"])
@pytest.mark.parametrize("with_bias", [True, False])
def test_emulinear_forward_backward(mode, with_bias):
    import torch

    from emulated_fp32_matrix_amd.linear import EmuLinear

    torch.manual_seed(0)
    layer = EmuLinear(256, 768, bias=with_bias, mode=mode, device="cuda:0")
    x = torch.randn(3, 400, 256, device="cuda:0", requires_grad=True)
    y = layer(x)
    assert y.shape == (3, 400, 768) and y.dtype == torch.float32
    gy = torch.randn_like(y)
    y.backward(gy)
    ry, rgx, rgw, rgb = _reference(x, layer.weight, layer.bias, gy)
    ey, egx, egw = _rel(y, ry), _rel(x.grad, rgx), _rel(layer.weight.grad, rgw)
    say(f"EmuLinear {mode} bias={with_bias}: y {ey:.2e}, dx {egx:.2e}, dW {egw:.2e}")
    tol = {"BF16X9": 2e-6, "AUTO": 2e-6, "NATIVE_F32": 2e-6, "BF16X6": 2e-6}[mode]
    assert ey <= tol and egx <= tol
    assert egw <= 1e-5   # torch FP32 matmul
    if with_bias:
        assert _rel(layer.bias.grad, rgb) <= 1e-5


def test_emulinear_matches_nn_linear_and_state_dict():
    import torch

    from emulated_fp32_matrix_amd.linear import EmuLinear

    torch.manual_seed(1)
    ref = torch.nn.Linear(512, 256).to("cuda:0")
    layer = EmuLinear.from_linear(ref, mode="BF16X9")
    assert set(layer.state_dict()) == set(ref.state_dict())
    x = torch.randn(1000, 512, device="cuda:0")
    torch.backends.cuda.matmul.allow_tf32 = False
    y_ref64 = torch.nn.functional.linear(x.cpu().double(), ref.weight.detach().cpu().double(),
                                         ref.bias.detach().cpu().double())
    assert _rel(layer(x), y_ref64) <= 2e-6
    # no input gradient requested: only the weight and bias gradients are formed
    layer.zero_grad()
    layer(x).sum().backward()
    assert layer.weight.grad is not None and layer.bias.grad is not None


@pytest.mark.parametrize("mode", ["AUTO", "BF16X9", "BF16X3", "NATIVE_F32"])
def test_emulinear_cached_weights_bitwise(mode):
    """cache_weights=True (weights split once, emu_sgemm_presplit) gives the
    uncached layer's forward output and input gradient bit for bit, for row
    counts where AUTO splits K (6,144) and where it does not; an optimizer
    step invalidates the cache; a second forward with unchanged weights
    reuses it."""
    import torch

    from emulated_fp32_matrix_amd.linear import EmuLinear

    torch.manual_seed(5)
    ref = EmuLinear(256, 768, mode=mode).cuda()
    cached = EmuLinear(256, 768, mode=mode, cache_weights=True).cuda()
    cached.load_state_dict(ref.state_dict())
    opt = torch.optim.SGD(cached.parameters(), lr=0.1)
    opt_ref = torch.optim.SGD(ref.parameters(), lr=0.1)
    for step, rows in enumerate((6144, 300, 6144)):
        x = torch.randn(rows, 256, device="cuda", requires_grad=True)
        xr = x.detach().clone().requires_grad_(True)
        y, yr = cached(x), ref(xr)
        g = torch.randn_like(y)
        y.backward(g)
        yr.backward(g)
        torch.cuda.synchronize()
        assert torch.equal(y.detach().view(torch.int32), yr.detach().view(torch.int32)), (mode, step)
        assert torch.equal(x.grad.view(torch.int32), xr.grad.view(torch.int32)), (mode, step)
        say(f"{mode} step {step} ({rows} rows): cached forward and input gradient bitwise equal")
        opt.step()
        opt_ref.step()
        opt.zero_grad()
        opt_ref.zero_grad()
    if mode != "NATIVE_F32":
        with torch.no_grad():
            cached(torch.randn(64, 256, device="cuda"))
            first = cached._caches[0].planes
            cached(torch.randn(128, 256, device="cuda"))
            assert cached._caches[0].planes is first   # unchanged weights: the same planes
            cached.weight.add_(1.0)
            cached(torch.randn(64, 256, device="cuda"))
            assert cached._caches[0].planes is not first   # in-place update: split again


@pytest.mark.parametrize("mode", ["BF16X9", "AUTO", "NATIVE_F32"])
@pytest.mark.parametrize("cache_weights", [False, True])
def test_emulinear_force_loss_double_backward(mode, cache_weights):
    """Training on forces: E = sum(l2(tanh(l1(x)))), F = -dE/dx with
    create_graph=True (the input-gradient GEMM through the library), then
    L = |F|^2 differentiated again.  Every gradient of L (both layers'
    weights, the first bias, x) is compared with torch float64 on the CPU;
    the second-order terms run through the library's emulated products."""
    import torch

    from emulated_fp32_matrix_amd.linear import EmuLinear

    torch.manual_seed(7)
    l1 = EmuLinear(256, 512, mode=mode, device="cuda:0", cache_weights=cache_weights)
    l2 = EmuLinear(512, 64, mode=mode, device="cuda:0", cache_weights=cache_weights)
    x = torch.randn(3000, 256, device="cuda:0", requires_grad=True)

    def loss_of(f1, f2, xx):
        e = f2(torch.tanh(f1(xx))).sum()
        (gx,) = torch.autograd.grad(e, xx, create_graph=True)
        return ((-gx) ** 2).sum()

    params = [l1.weight, l1.bias, l2.weight]
    got = torch.autograd.grad(loss_of(l1, l2, x), params + [x])
    p64 = [p.detach().cpu().double().requires_grad_(True) for p in (l1.weight, l1.bias, l2.weight, l2.bias)]
    x64 = x.detach().cpu().double().requires_grad_(True)
    want = torch.autograd.grad(
        loss_of(lambda t: torch.nn.functional.linear(t, p64[0], p64[1]),
                lambda t: torch.nn.functional.linear(t, p64[2], p64[3]), x64), p64[:3] + [x64])
    for name, g, w in zip(("W1", "b1", "W2", "x"), got, want):
        rel = _rel(g, w)
        say(f"force loss {mode} cache={cache_weights}: dL/d{name} rel err {rel:.2e}")
        assert rel <= 1e-5, (name, rel)
