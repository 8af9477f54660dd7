"""EmuLinear: a float-in / float-out linear layer whose forward GEMM and
input-gradient GEMM run through the emulated-FP32 library.

"Unlocking Tensor Core Performance for Machine Learning Interatomic
Potentials", section "TF32x3 on Ampere GPUs", describes such a layer: a
drop-in replacement for a standard linear layer, FP32 tensors in and out,
whose forward product and the gradient propagated to its input (from which
an interatomic potential derives forces) both use the emulated arithmetic,
while the weight gradient stays in ordinary precision.

Here, with the weight stored like torch.nn.Linear ([out_features,
in_features]):
  forward   y  = x W^T + b   emu_sgemm_bias, op(B) = W^T (transB = T), bias
                             added in the GEMM epilogue;
  backward  dx = dy W        emu_sgemm (transB = N);
            dW = dy^T x      torch FP32 matmul (TF32 off), db = sum of dy rows.

The backward is itself differentiable (create_graph=True), as training on
forces needs: dx = dy W is an autograd function whose own gradients are
again an emulated product (for dy) and an FP32 weight-gradient product (for
W), and dW, db are torch operations.

The mode ("AUTO" = the performant policy, "BF16X9" = eager, "BF16X6",
"BF16X3", "NATIVE_F32") applies to both library GEMMs.

With cache_weights=True the layer keeps the BF16 planes of W (for the
forward GEMM) and of W^T (for the input gradient), made by emu_presplit_b,
and runs the emulated GEMMs through emu_sgemm_presplit, which then skips
splitting the weights on every call; results are bit-identical.  The cache
is keyed by the weight's storage, shape, version counter and the mode, so an
optimizer step or load_state_dict (in-place updates) invalidates it.
"""
from __future__ import annotations

import math

import torch

from . import KSPLIT_AUTO, presplit_b, select_mode, sgemm, sgemm_presplit

_EMULATED = ("BF16X9", "BF16X6", "BF16X3", "BF16X1")


class _PlanesCache:
    """Planes of one op(B) of a weight, rebuilt when the weight changes."""

    def __init__(self, trans_b):
        self.trans_b = trans_b
        self.key = None
        self.planes = None

    def get(self, w, mode):
        key = (w.data_ptr(), tuple(w.shape), w._version, mode, w.device)
        if key != self.key:
            self.planes = presplit_b(w, mode=mode, trans_b=self.trans_b)
            self.key = key
        return self.planes


def _gemm(a, w, trans_b, mode, bias, cache):
    """a @ op(w) (+ bias) in `mode`; with a cache and an emulated mode (the
    one AUTO would run, when mode is AUTO) through the weight's planes, with
    the K split plan the library would choose itself, so the result is the
    same bit for bit."""
    if cache is None:
        return sgemm(a, w, mode=mode, trans_b=trans_b, bias=bias)
    M, K = a.shape
    N = w.shape[0] if trans_b else w.shape[1]
    run = select_mode(M, N, K) if mode == "AUTO" else mode
    if run not in _EMULATED:
        return sgemm(a, w, mode=run, trans_b=trans_b, bias=bias)
    # the library splits K only under AUTO (KSPLIT_AUTO: its plan in the
    # mode AUTO runs) and only where A is split inside the GEMM
    ksplit = KSPLIT_AUTO if mode == "AUTO" else 1
    return sgemm_presplit(a, cache.get(w, run), bias=bias, ksplit=ksplit)


def _as_rows(t, width):
    t2 = t.reshape(-1, width)
    return t2 if t2.is_contiguous() else t2.contiguous()


def _fp32_matmul(a, b):
    """a @ b in torch FP32 with TF32 off: the weight-gradient products, which
    stay in ordinary precision."""
    prev = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        return a.matmul(b)
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev


def _cache_for(caches, trans_w):
    # caches = (planes of W^T, planes of W)
    return None if not caches else caches[0 if trans_w else 1]


class _EmuMatmulFunction(torch.autograd.Function):
    """y = a @ op(w), op(w) = w^T (trans_w) or w, through the library: the
    layer's input-gradient product dx = dy W, differentiable again, so that
    a loss on forces (a first derivative of the energy) can be
    differentiated once more (create_graph=True).  Its gradients:
    d/da = g @ op(w)^T, again this emulated product; d/dw = g^T a (trans_w)
    or a^T g, a weight-gradient product in torch FP32."""

    @staticmethod
    def forward(ctx, a, w, trans_w, mode, caches):
        a2 = a if a.is_contiguous() else a.contiguous()
        wc = w if w.is_contiguous() else w.contiguous()
        y = _gemm(a2, wc, trans_w, mode, None, _cache_for(caches, trans_w) if wc is w else None)
        ctx.save_for_backward(a, w)
        ctx.trans_w = trans_w
        ctx.mode = mode
        ctx.caches = caches
        return y

    @staticmethod
    def backward(ctx, g):
        a, w = ctx.saved_tensors
        g2 = g if g.is_contiguous() else g.contiguous()
        ga = gw = None
        if ctx.needs_input_grad[0]:
            ga = _EmuMatmulFunction.apply(g2, w, not ctx.trans_w, ctx.mode, ctx.caches)
        if ctx.needs_input_grad[1]:
            gw = _fp32_matmul(g2.t(), a) if ctx.trans_w else _fp32_matmul(a.t(), g2)
        return ga, gw, None, None, None


class _EmuLinearFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, mode, caches):
        if x.dtype != torch.float32 or weight.dtype != torch.float32:
            raise TypeError("EmuLinear computes in float32")
        out_f, in_f = weight.shape
        x2 = _as_rows(x, in_f)
        w = weight if weight.is_contiguous() else weight.contiguous()
        y = _gemm(x2, w, True, mode, bias, caches[0] if caches and w is weight else None)
        # the inputs themselves are saved, so that the products formed from
        # them in backward stay connected to the graph (double backward)
        ctx.save_for_backward(x, weight)
        ctx.has_bias = bias is not None
        ctx.mode = mode
        ctx.caches = caches
        return y.reshape(*x.shape[:-1], out_f)

    @staticmethod
    def backward(ctx, gy):
        x, weight = ctx.saved_tensors
        out_f, in_f = weight.shape
        gy2 = _as_rows(gy, out_f)
        gx = gw = gb = None
        if ctx.needs_input_grad[0]:
            # dx = dy W: emulated, and differentiable (force training)
            gx = _EmuMatmulFunction.apply(gy2, weight, False, ctx.mode, ctx.caches).reshape(x.shape)
        if ctx.needs_input_grad[1]:
            gw = _fp32_matmul(gy2.t(), _as_rows(x, in_f))
        if ctx.has_bias and ctx.needs_input_grad[2]:
            gb = gy2.sum(dim=0)
        return gx, gw, gb, None, None


class EmuLinear(torch.nn.Module):
    """torch.nn.Linear with its forward and input-gradient GEMMs emulated.

    Parameters and initialisation match torch.nn.Linear, so state dicts load
    either way; :meth:`from_linear` wraps an existing layer's parameters.
    """

    def __init__(self, in_features, out_features, bias=True, mode="AUTO", device=None,
                 cache_weights=False):
        super().__init__()
        self.in_features = in_features
        self.out_features = out_features
        self.mode = mode
        # planes of W^T (forward) and W (input gradient), or None
        self._caches = (_PlanesCache(True), _PlanesCache(False)) if cache_weights else None
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features, device=device,
                                                     dtype=torch.float32))
        if bias:
            self.bias = torch.nn.Parameter(torch.empty(out_features, device=device,
                                                       dtype=torch.float32))
        else:
            self.register_parameter("bias", None)
        self.reset_parameters()

    def reset_parameters(self):
        # the same scheme as torch.nn.Linear
        torch.nn.init.kaiming_uniform_(self.weight, a=math.sqrt(5))
        if self.bias is not None:
            bound = 1.0 / math.sqrt(self.in_features) if self.in_features > 0 else 0.0
            torch.nn.init.uniform_(self.bias, -bound, bound)

    @classmethod
    def from_linear(cls, linear, mode="AUTO", cache_weights=False):
        m = cls(linear.in_features, linear.out_features, bias=linear.bias is not None, mode=mode,
                device=linear.weight.device, cache_weights=cache_weights)
        with torch.no_grad():
            m.weight.copy_(linear.weight)
            if linear.bias is not None:
                m.bias.copy_(linear.bias)
        return m

    def forward(self, x):
        return _EmuLinearFunction.apply(x, self.weight, self.bias, self.mode, self._caches)

    def extra_repr(self):
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, mode={self.mode}, "
                f"cache_weights={self._caches is not None}")
