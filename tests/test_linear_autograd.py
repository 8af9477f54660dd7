"""Host-side checks of EmuLinear's autograd wiring (CPU only).

The library GEMM behind the layer (``linear._gemm``) is replaced by the same
product in torch, so that the functions' derivatives can be checked without
a GPU: the layer must differentiate like torch.nn.functional.linear to
second order, which is what training on forces needs ("Unlocking Tensor
Core Performance for Machine Learning Interatomic Potentials", section
"TF32x3 on Ampere GPUs": forces come from the input gradient).  The GPU
tests run the same layer through the library.
"""
import pytest
import torch

from emulated_fp32_matrix_amd import linear


def _torch_gemm(a, w, trans_b, mode, bias, cache):
    y = a @ (w.t() if trans_b else w)
    return y if bias is None else y + bias


@pytest.fixture
def torch_backed(monkeypatch):
    monkeypatch.setattr(linear, "_gemm", _torch_gemm)


def test_matmul_function_gradgradcheck(torch_backed):
    torch.manual_seed(0)
    for trans_w in (False, True):
        a = torch.randn(7, 5, dtype=torch.float64, requires_grad=True)
        w = torch.randn(*((4, 5) if trans_w else (5, 4)), dtype=torch.float64, requires_grad=True)
        f = lambda a_, w_: linear._EmuMatmulFunction.apply(a_, w_, trans_w, "BF16X9", None)
        assert torch.autograd.gradcheck(f, (a, w))
        assert torch.autograd.gradgradcheck(f, (a, w))


def _energy_force_loss(fwd1, fwd2, x):
    e = fwd2(torch.tanh(fwd1(x))).sum()
    (gx,) = torch.autograd.grad(e, x, create_graph=True)
    return e, ((-gx) ** 2).sum()


def test_force_loss_gradients_match_nn_linear(torch_backed):
    """E = sum(l2(tanh(l1(x)))), F = -dE/dx (create_graph), L = |F|^2: the
    gradients of L with respect to every parameter and to x equal those of
    the same network built from torch.nn.functional.linear."""
    torch.manual_seed(1)
    l1 = linear.EmuLinear(6, 9, mode="BF16X9")
    l2 = linear.EmuLinear(9, 3, mode="BF16X9")
    x = torch.randn(11, 6, requires_grad=True)
    _, loss = _energy_force_loss(l1, l2, x)
    params = [l1.weight, l1.bias, l2.weight, l2.bias]
    # (the last bias does not enter the forces: its gradient is None)
    got = torch.autograd.grad(loss, params + [x], allow_unused=True)

    p64 = [p.detach().double().requires_grad_(True) for p in params]
    x64 = x.detach().double().requires_grad_(True)
    f1 = lambda t: torch.nn.functional.linear(t, p64[0], p64[1])
    f2 = lambda t: torch.nn.functional.linear(t, p64[2], p64[3])
    _, loss64 = _energy_force_loss(f1, f2, x64)
    want = torch.autograd.grad(loss64, p64 + [x64], allow_unused=True)
    assert [g is None for g in got] == [False, False, False, True, False]
    assert [w is None for w in want] == [False, False, False, True, False]
    for g, w in zip(got, want):
        if w is None:
            continue
        rel = float((g.double() - w).norm() / w.norm())
        assert rel < 1e-5, rel


def test_first_order_unchanged_without_create_graph(torch_backed):
    torch.manual_seed(2)
    layer = linear.EmuLinear(8, 5, mode="BF16X9")
    x = torch.randn(3, 4, 8, requires_grad=True)
    y = layer(x)
    gy = torch.randn_like(y)
    y.backward(gy)
    x2 = x.detach().clone().requires_grad_(True)
    w2 = layer.weight.detach().clone().requires_grad_(True)
    b2 = layer.bias.detach().clone().requires_grad_(True)
    torch.nn.functional.linear(x2, w2, b2).backward(gy)
    for g, w in ((x.grad, x2.grad), (layer.weight.grad, w2.grad), (layer.bias.grad, b2.grad)):
        assert torch.allclose(g, w, rtol=1e-5, atol=1e-6)
