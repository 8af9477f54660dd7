"""CPU oracle for the emulated-FP32 GEMM (ctypes wrapper over ``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg import this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and it never
imports the product path.

Functions (numpy in, numpy out; every array is C-contiguous):

* :func:`bf16_round`  -- FP32 -> BF16 round-to-nearest-even, saturating.
* :func:`split_bf16x3` -- the exact three-piece split (hi, mid', lo') of
  "Unlocking Tensor Core Performance for Machine Learning Interatomic
  Potentials", section "How Tensor Core FP32 bridges the hardware gap",
  Figure 1.
* :func:`gemm_f64` -- FP64-accumulated reference GEMM (the page's FP64
  reference, section "Limitations and decision criteria").
* :func:`emu_gemm` -- scalar model of the band-accumulated emulated GEMM
  (Figure 1; Figure 2's equation for the reduced variants).
* :func:`mfma_bf16_dot16` -- a model of one gfx950 bf16 matrix instruction
  (acc + 16 products in two passes of 8, aligned, truncated, one rounding),
  characterised on the hardware in the manner of "Accurate Models of NVIDIA
  Tensor Cores", section "Results"; rules in ``oracle.c``.
* :func:`emu_gemm_mfma` -- the emulated GEMM evaluated the way the GPU
  kernels evaluate it, every band accumulated through that model, for
  bit-for-bit comparison.
* :func:`native_gemm_mfma` -- the FP32 GEMM evaluated the way the native
  kernels evaluate it: the gfx950 FP32 matrix instruction is two IEEE fused
  multiply-adds, characterised on the hardware the same way; rules in
  ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

NBANDS = {"BF16X9": 5, "BF16X6": 3, "BF16X3": 2, "BF16X1": 1}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.oracle_bf16_round.argtypes = [vp, i64, vp]
    lib.oracle_bf16_round.restype = None
    lib.oracle_split_bf16x3.argtypes = [vp, i64, vp, vp, vp]
    lib.oracle_split_bf16x3.restype = None
    lib.oracle_gemm_f64.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_double,
                                    vp, i64, vp, i64, ctypes.c_double, vp, i64, vp]
    lib.oracle_gemm_f64.restype = None
    lib.oracle_emu_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_float, vp, i64, vp, i64,
                                    ctypes.c_float, vp, i64, vp, vp]
    lib.oracle_emu_gemm.restype = None
    lib.oracle_mfma_bf16_dot16.argtypes = [i64, vp, vp, vp, vp]
    lib.oracle_mfma_bf16_dot16.restype = None
    lib.oracle_emu_gemm_mfma.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_float, vp, i64, vp, i64,
                                         ctypes.c_float, vp, i64, vp, vp]
    lib.oracle_emu_gemm_mfma.restype = None
    lib.oracle_native_gemm_mfma.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_float,
                                            vp, i64, vp, i64, ctypes.c_float, vp, i64, vp, vp]
    lib.oracle_native_gemm_mfma.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def bf16_round(x) -> np.ndarray:
    """BF16 bit patterns (uint16) of R(x): round to nearest even, saturating."""
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_bf16_round(_ptr(x), x.size, _ptr(out))
    return out


def split_bf16x3(x):
    """(hi, mid', lo') BF16 bit patterns (uint16 arrays shaped like ``x``)."""
    x = _f32(x)
    hi = np.empty(x.shape, dtype=np.uint16)
    mid = np.empty(x.shape, dtype=np.uint16)
    lo = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_split_bf16x3(_ptr(x), x.size, _ptr(hi), _ptr(mid), _ptr(lo))
    return hi, mid, lo


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of BF16 bit patterns as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _shapes(a, b, trans_a, trans_b):
    if a.ndim != 2 or b.ndim != 2:
        raise ValueError("A and B must be 2-D")
    M, K = (a.shape[1], a.shape[0]) if trans_a else a.shape
    Kb, N = (b.shape[1], b.shape[0]) if trans_b else b.shape
    if K != Kb:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    return M, N, K


def _bias(bias, N):
    if bias is None:
        return None
    bias = _f32(bias)
    if bias.shape != (N,):
        raise ValueError(f"bias must have shape ({N},)")
    return bias


def gemm_f64(a, b, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, c=None,
             bias=None) -> np.ndarray:
    """FP64-accumulated alpha*op(A)@op(B) + beta*C of FP32 inputs (float64 M x N).

    ``bias`` (length N, FP32) is added to every row last, in FP64: the linear
    layer y = x W^T + b of "Unlocking Tensor Core Performance for Machine
    Learning Interatomic Potentials", section "TF32x3 on Ampere GPUs".
    """
    a = _f32(a)
    b = _f32(b)
    M, N, K = _shapes(a, b, trans_a, trans_b)
    out = np.empty((M, N), dtype=np.float64)
    if beta != 0.0:
        c = _f32(c)
        assert c.shape == (M, N)
        cp, ldc = _ptr(c), N
    else:
        cp, ldc = None, max(N, 1)
    bias = _bias(bias, N)
    _load().oracle_gemm_f64(int(trans_a), int(trans_b), M, N, K, float(alpha), _ptr(a),
                            a.shape[1], _ptr(b), b.shape[1], float(beta), cp, ldc, _ptr(out))
    if bias is not None:
        out += bias.astype(np.float64)[None, :]
    return out


def emu_gemm(a, b, mode="BF16X9", trans_a=False, trans_b=False, alpha=1.0, beta=0.0, c=None,
             acc_f64=False, bias=None) -> np.ndarray:
    """Scalar model of the emulated GEMM.

    ``mode`` is BF16X9, BF16X6 or BF16X3 (or an explicit band count 1..5).
    Returns float32 (FP32 band accumulation) or float64 (``acc_f64``).
    ``bias`` (length N) is added to every row after alpha and beta, with one
    more rounding in the output's precision.
    """
    nb = NBANDS[mode] if isinstance(mode, str) else int(mode)
    a = _f32(a)
    b = _f32(b)
    M, N, K = _shapes(a, b, trans_a, trans_b)
    if acc_f64:
        out64 = np.empty((M, N), dtype=np.float64)
        out32 = None
    else:
        out32 = np.empty((M, N), dtype=np.float32)
        out64 = None
    if beta != 0.0:
        c = _f32(c)
        assert c.shape == (M, N)
        cp, ldc = _ptr(c), N
    else:
        cp, ldc = None, max(N, 1)
    bias = _bias(bias, N)
    _load().oracle_emu_gemm(int(trans_a), int(trans_b), M, N, K, nb, int(acc_f64), float(alpha),
                            _ptr(a), a.shape[1], _ptr(b), b.shape[1], float(beta), cp, ldc,
                            _ptr(out32) if out32 is not None else None,
                            _ptr(out64) if out64 is not None else None)
    if bias is not None:
        if acc_f64:
            out64 += bias.astype(np.float64)[None, :]
        else:
            out32 = (out32 + bias[None, :]).astype(np.float32)   # one float32 rounding per entry
    return out64 if acc_f64 else out32


def mfma_bf16_dot16(acc, a_bits, b_bits) -> np.ndarray:
    """The model of one gfx950 bf16 matrix instruction per row: acc (n,)
    float32, a_bits/b_bits (n, 16) BF16 bit patterns; returns acc + the 16
    products as the matrix unit forms it (two passes of 8; rules in
    oracle.c)."""
    acc = _f32(acc)
    a_bits = np.ascontiguousarray(a_bits, dtype=np.uint16)
    b_bits = np.ascontiguousarray(b_bits, dtype=np.uint16)
    n = acc.shape[0]
    assert a_bits.shape == (n, 16) and b_bits.shape == (n, 16)
    out = np.empty(n, dtype=np.float32)
    _load().oracle_mfma_bf16_dot16(n, _ptr(acc), _ptr(a_bits), _ptr(b_bits), _ptr(out))
    return out


def emu_gemm_mfma(a, b, mode="BF16X9", trans_a=False, trans_b=False, alpha=1.0, beta=0.0,
                  c=None, bias=None, ksplit=1) -> np.ndarray:
    """The emulated GEMM as the GPU kernels evaluate it, bit for bit: the
    band model with every band accumulated by the kernels' sequence of
    matrix instructions under the matrix-unit model (float32 M x N).
    ``ksplit`` = S > 1 (dividing ceil(K/32)): K in S segments, each
    segment's recombined result t_s, summed in segment order."""
    nb = NBANDS[mode] if isinstance(mode, str) else int(mode)
    a = _f32(a)
    b = _f32(b)
    M, N, K = _shapes(a, b, trans_a, trans_b)
    out = np.empty((M, N), dtype=np.float32)
    if beta != 0.0:
        c = _f32(c)
        assert c.shape == (M, N)
        cp, ldc = _ptr(c), N
    else:
        cp, ldc = None, max(N, 1)
    bias = _bias(bias, N)
    _load().oracle_emu_gemm_mfma(int(trans_a), int(trans_b), M, N, K, nb, int(ksplit), float(alpha), _ptr(a),
                                 a.shape[1], _ptr(b), b.shape[1], float(beta), cp, ldc,
                                 _ptr(bias) if bias is not None else None, _ptr(out))
    return out


def native_gemm_mfma(a, b, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, c=None,
                     bias=None) -> np.ndarray:
    """The native FP32 GEMM as the GPU kernels evaluate it, bit for bit: per
    element an FMA chain in the k order 0, 16, 1, 17, ..., 15, 31, 32, 48, ...
    from +0, then alpha, beta and bias (float32 M x N)."""
    a = _f32(a)
    b = _f32(b)
    M, N, K = _shapes(a, b, trans_a, trans_b)
    out = np.empty((M, N), dtype=np.float32)
    if beta != 0.0:
        c = _f32(c)
        assert c.shape == (M, N)
        cp, ldc = _ptr(c), N
    else:
        cp, ldc = None, max(N, 1)
    bias = _bias(bias, N)
    _load().oracle_native_gemm_mfma(int(trans_a), int(trans_b), M, N, K, float(alpha), _ptr(a),
                                    a.shape[1], _ptr(b), b.shape[1], float(beta), cp, ldc,
                                    _ptr(bias) if bias is not None else None, _ptr(out))
    return out
