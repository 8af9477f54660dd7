"""Python binding of ``libemu_sgemm.so``: FP32 GEMM emulated on MI355X bf16 MFMA.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/emu_sgemm.h``.  PyTorch
supplies device memory and the stream.  There is no CPU fallback: importing
this package fails if the library has not been built, and every call raises
:class:`EmuError` on a non-success status.

Low-level entry points mirror the C ABI one to one (pointers are ints):
:func:`emu_sgemm`, :func:`emu_sgemm_bias`, :func:`emu_sgemm_ex`,
:func:`emu_sgemm_noalloc`, :func:`emu_split_bf16x3`, :func:`emu_sgemm_select`, :func:`emu_sgemm_ksplit`,
:func:`emu_sgemm_plan`, :func:`emu_status_string`, :func:`emu_abi_version`.  :func:`sgemm` and
:func:`split_bf16x3` accept torch tensors.

Method: "Unlocking Tensor Core Performance for Machine Learning Interatomic
Potentials", section "How Tensor Core FP32 bridges the hardware gap",
Figures 1 and 2.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libemu_sgemm.so")

OP_N, OP_T = 0, 1
MODES = {"NATIVE_F32": 0, "BF16X9": 1, "BF16X6": 2, "BF16X3": 3, "AUTO": 4, "BF16X1": 5}
MODE_NAMES = {v: k for k, v in MODES.items()}
STATUS_SUCCESS = 0
STATUS_INVALID_VALUE = 1
STATUS_NOT_SUPPORTED = 2
STATUS_LAUNCH_FAILED = 3
STATUS_ALLOC_FAILED = 4
STATUS_INTERNAL = 5
STATUS_SCRATCH_TOO_SMALL = 6
NOALLOC_SCRATCH_BYTES = 64 << 20   # EMU_NOALLOC_SCRATCH_BYTES
KSPLIT_AUTO = -1                   # EMU_KSPLIT_AUTO: the AUTO policy's plan in an explicit mode

# C functions declared in include/emu_sgemm.h
EXPORTS = ("emu_sgemm", "emu_sgemm_bias", "emu_sgemm_ex", "emu_split_bf16x3", "emu_sgemm_select",
           "emu_sgemm_ksplit", "emu_presplit_b_bytes", "emu_presplit_b", "emu_sgemm_presplit",
           "emu_sgemm_noalloc", "emu_sgemm_plan", "emu_status_string", "emu_abi_version")


class EmuError(RuntimeError):
    """A C-ABI call returned a status other than EMU_STATUS_SUCCESS."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {emu_status_string(status)} ({status})")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first "
                      "(python -c 'import __graft_entry__ as g; g.build()')")

# torch ships its own HIP runtime with the same soname (libamdhip64.so.7).
# Loading torch first makes the library bind to that runtime, so the
# process has one HIP runtime and torch's streams and allocations are valid
# handles for the library; loading the library first would bring in a
# second runtime from the ROCm installation.
import torch as _torch_runtime  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_lib.emu_sgemm.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, ctypes.c_float, _vp, _i64,
                           _vp, _i64, ctypes.c_float, _vp, _i64, ctypes.c_int, _vp]
_lib.emu_sgemm.restype = ctypes.c_int
_lib.emu_sgemm_bias.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, ctypes.c_float, _vp,
                                _i64, _vp, _i64, ctypes.c_float, _vp, _i64, _vp, ctypes.c_int, _vp]
_lib.emu_sgemm_bias.restype = ctypes.c_int
_lib.emu_sgemm_ex.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, ctypes.c_float, _vp,
                              _i64, _vp, _i64, ctypes.c_float, _vp, _i64, _vp, ctypes.c_int,
                              ctypes.c_int, _vp]
_lib.emu_sgemm_ex.restype = ctypes.c_int
_lib.emu_sgemm_noalloc.argtypes = _lib.emu_sgemm_ex.argtypes
_lib.emu_sgemm_noalloc.restype = ctypes.c_int
_lib.emu_sgemm_ksplit.argtypes = [_i64, _i64, _i64, ctypes.POINTER(ctypes.c_int)]
_lib.emu_sgemm_ksplit.restype = ctypes.c_int
_lib.emu_sgemm_plan.argtypes = [_i64, _i64, _i64, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                ctypes.POINTER(ctypes.c_int64)]
_lib.emu_sgemm_plan.restype = ctypes.c_int
_lib.emu_presplit_b_bytes.argtypes = [_i64, _i64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
_lib.emu_presplit_b_bytes.restype = ctypes.c_int
_lib.emu_presplit_b.argtypes = [ctypes.c_int, _i64, _i64, _vp, _i64, ctypes.c_int, _vp, _vp]
_lib.emu_presplit_b.restype = ctypes.c_int
_lib.emu_sgemm_presplit.argtypes = [ctypes.c_int, _i64, _i64, _i64, ctypes.c_float, _vp, _i64, _vp,
                                    ctypes.c_float, _vp, _i64, _vp, ctypes.c_int, ctypes.c_int, _vp]
_lib.emu_sgemm_presplit.restype = ctypes.c_int
_lib.emu_split_bf16x3.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp]
_lib.emu_split_bf16x3.restype = ctypes.c_int
_lib.emu_sgemm_select.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64,
                                  ctypes.POINTER(ctypes.c_int)]
_lib.emu_sgemm_select.restype = ctypes.c_int
_lib.emu_status_string.argtypes = [ctypes.c_int]
_lib.emu_status_string.restype = ctypes.c_char_p
_lib.emu_abi_version.argtypes = []
_lib.emu_abi_version.restype = ctypes.c_int


def _mode(mode) -> int:
    if isinstance(mode, str):
        return MODES[mode.upper()]
    return int(mode)


# ---- C ABI, one to one -------------------------------------------------------

def emu_status_string(status: int) -> str:
    return _lib.emu_status_string(int(status)).decode()


def emu_abi_version() -> int:
    return int(_lib.emu_abi_version())


def emu_sgemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, mode, stream) -> int:
    """Raw call; returns the status code (pointers and stream are ints)."""
    return int(_lib.emu_sgemm(int(transA), int(transB), int(M), int(N), int(K), float(alpha),
                              A or None, int(lda), B or None, int(ldb), float(beta), C or None,
                              int(ldc), _mode(mode), stream or None))


def emu_sgemm_bias(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, mode,
                   stream) -> int:
    """Raw call; returns the status code (pointers and stream are ints)."""
    return int(_lib.emu_sgemm_bias(int(transA), int(transB), int(M), int(N), int(K), float(alpha),
                                   A or None, int(lda), B or None, int(ldb), float(beta), C or None,
                                   int(ldc), bias or None, _mode(mode), stream or None))


def emu_sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, mode,
                 ksplit, stream) -> int:
    """Raw call; returns the status code (pointers and stream are ints)."""
    return int(_lib.emu_sgemm_ex(int(transA), int(transB), int(M), int(N), int(K), float(alpha),
                                 A or None, int(lda), B or None, int(ldb), float(beta), C or None,
                                 int(ldc), bias or None, _mode(mode), int(ksplit), stream or None))


def emu_sgemm_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, mode,
                      ksplit, stream) -> int:
    """Raw call of the allocation-free variant of emu_sgemm_ex; returns the
    status code (pointers and stream are ints)."""
    return int(_lib.emu_sgemm_noalloc(int(transA), int(transB), int(M), int(N), int(K), float(alpha),
                                      A or None, int(lda), B or None, int(ldb), float(beta), C or None,
                                      int(ldc), bias or None, _mode(mode), int(ksplit), stream or None))


def emu_sgemm_ksplit(M, N, K):
    """(status, K split the library chooses for this shape or None)."""
    out = ctypes.c_int(-1)
    st = int(_lib.emu_sgemm_ksplit(int(M), int(N), int(K), ctypes.byref(out)))
    return st, (out.value if st == STATUS_SUCCESS else None)


def emu_sgemm_plan(M, N, K):
    """(status, (ksplit, tile_rows, split_from) of the AUTO plan, or None)."""
    sp, th, sf = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_int64(-1)
    st = int(_lib.emu_sgemm_plan(int(M), int(N), int(K), ctypes.byref(sp), ctypes.byref(th),
                                 ctypes.byref(sf)))
    return st, ((sp.value, th.value, sf.value) if st == STATUS_SUCCESS else None)


def emu_presplit_b_bytes(N, K, mode):
    """(status, bytes) of emu_presplit_b_bytes."""
    out = ctypes.c_size_t(0)
    st = int(_lib.emu_presplit_b_bytes(int(N), int(K), _mode(mode), ctypes.byref(out)))
    return st, int(out.value)


def emu_presplit_b(transB, N, K, B, ldb, mode, planes, stream) -> int:
    return int(_lib.emu_presplit_b(int(transB), int(N), int(K), B or None, int(ldb), _mode(mode),
                                   planes or None, stream or None))


def emu_sgemm_presplit(transA, M, N, K, alpha, A, lda, planes, beta, C, ldc, bias, mode, ksplit,
                       stream) -> int:
    return int(_lib.emu_sgemm_presplit(int(transA), int(M), int(N), int(K), float(alpha), A or None,
                                       int(lda), planes or None, float(beta), C or None, int(ldc),
                                       bias or None, _mode(mode), int(ksplit), stream or None))


def emu_split_bf16x3(x, n, hi, mid, lo, stream) -> int:
    return int(_lib.emu_split_bf16x3(x or None, int(n), hi or None, mid or None, lo or None,
                                     stream or None))


def emu_sgemm_select(transA, transB, M, N, K):
    """(status, chosen mode name or None)."""
    out = ctypes.c_int(-1)
    st = int(_lib.emu_sgemm_select(int(transA), int(transB), int(M), int(N), int(K),
                                   ctypes.byref(out)))
    return st, (MODE_NAMES.get(out.value) if st == STATUS_SUCCESS else None)


# ---- torch-tensor convenience (marshalling only) -----------------------------

def _torch():
    import torch

    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check_matrix(x, name):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_cuda:
        raise TypeError(f"{name} must be a float32 CUDA tensor")
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if x.stride(1) != 1 and x.numel() > 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")


def _ld(x):
    return max(int(x.stride(0)), int(x.shape[1]), 1)


def sgemm(a, b, mode="BF16X9", trans_a=False, trans_b=False, alpha=1.0, beta=0.0, c=None,
          stream=None, bias=None, ksplit=None):
    """C = alpha * op(a) @ op(b) + beta * c (+ bias[j] on every row) through
    ``emu_sgemm`` (``emu_sgemm_bias`` when ``bias`` is given, ``emu_sgemm_ex``
    when ``ksplit`` is given: 0 = the library's choice, S >= 1 = exactly S
    K segments on every output tile, ``KSPLIT_AUTO`` = the AUTO policy's plan
    in the mode given).

    ``a``/``b`` are the stored (row-major) matrices; ``trans_*`` select op().
    Returns ``c`` (allocated when None).  Asynchronous on ``stream``
    (default: torch's current stream).
    """
    torch = _torch()
    _check_matrix(a, "a")
    _check_matrix(b, "b")
    M, K = (a.shape[1], a.shape[0]) if trans_a else (a.shape[0], a.shape[1])
    Kb, N = (b.shape[1], b.shape[0]) if trans_b else (b.shape[0], b.shape[1])
    if K != Kb:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    if c is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs c")
        c = torch.empty((M, N), dtype=torch.float32, device=a.device)
    else:
        _check_matrix(c, "c")
        if tuple(c.shape) != (M, N):
            raise ValueError(f"c must be {M}x{N}")
    if bias is not None and (not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32
                             or not bias.is_cuda or bias.dim() != 1 or bias.shape[0] != N
                             or (N > 1 and bias.stride(0) != 1)):
        raise TypeError(f"bias must be a contiguous float32 CUDA vector of length {N}")
    if ksplit is not None:
        st = emu_sgemm_ex(OP_T if trans_a else OP_N, OP_T if trans_b else OP_N, M, N, K, alpha,
                          a.data_ptr(), _ld(a), b.data_ptr(), _ld(b), beta, c.data_ptr(), _ld(c),
                          bias.data_ptr() if bias is not None else 0, mode, ksplit,
                          _stream_handle(stream))
        if st != STATUS_SUCCESS:
            raise EmuError(st, "emu_sgemm_ex")
        return c
    if bias is None:
        st = emu_sgemm(OP_T if trans_a else OP_N, OP_T if trans_b else OP_N, M, N, K, alpha,
                       a.data_ptr(), _ld(a), b.data_ptr(), _ld(b), beta, c.data_ptr(), _ld(c),
                       mode, _stream_handle(stream))
        if st != STATUS_SUCCESS:
            raise EmuError(st, "emu_sgemm")
        return c
    st = emu_sgemm_bias(OP_T if trans_a else OP_N, OP_T if trans_b else OP_N, M, N, K, alpha,
                        a.data_ptr(), _ld(a), b.data_ptr(), _ld(b), beta, c.data_ptr(), _ld(c),
                        bias.data_ptr(), mode, _stream_handle(stream))
    if st != STATUS_SUCCESS:
        raise EmuError(st, "emu_sgemm_bias")
    return c


class PresplitB:
    """op(B) split once into the BF16 planes of ``mode`` (``presplit_b``):
    ``planes`` is a uint8 CUDA tensor in the library's own layout, valid for
    GEMMs with this N, K and mode (``sgemm_presplit``)."""

    def __init__(self, planes, N, K, mode):
        self.planes, self.N, self.K, self.mode = planes, int(N), int(K), mode


def presplit_b(b, mode="BF16X9", trans_b=False, stream=None):
    """Split op(b) (K x N; ``b`` stored as for ``sgemm``) once, for use by
    ``sgemm_presplit`` in ``mode`` (BF16X9, BF16X6, BF16X3 or BF16X1)."""
    torch = _torch()
    _check_matrix(b, "b")
    K, N = (b.shape[1], b.shape[0]) if trans_b else (b.shape[0], b.shape[1])
    st, nbytes = emu_presplit_b_bytes(N, K, mode)
    if st != STATUS_SUCCESS:
        raise EmuError(st, "emu_presplit_b_bytes")
    planes = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=b.device)
    st = emu_presplit_b(OP_T if trans_b else OP_N, N, K, b.data_ptr(), _ld(b), mode,
                        planes.data_ptr(), _stream_handle(stream))
    if st != STATUS_SUCCESS:
        raise EmuError(st, "emu_presplit_b")
    return PresplitB(planes, N, K, mode)


def sgemm_presplit(a, pb, trans_a=False, alpha=1.0, beta=0.0, c=None, bias=None, ksplit=0,
                   stream=None):
    """C = alpha * op(a) @ op(B) + beta * c (+ bias) through
    ``emu_sgemm_presplit``, op(B) given by ``pb = presplit_b(...)``; equal
    bit for bit to ``sgemm(a, b, pb.mode, ..., ksplit=ksplit)``."""
    torch = _torch()
    _check_matrix(a, "a")
    if not isinstance(pb, PresplitB):
        raise TypeError("pb must come from presplit_b")
    M, K = (a.shape[1], a.shape[0]) if trans_a else (a.shape[0], a.shape[1])
    N = pb.N
    if K != pb.K:
        raise ValueError(f"inner dimensions differ: {K} vs {pb.K}")
    if pb.planes.device != a.device:
        raise ValueError("a and the planes must be on one device")
    if c is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs c")
        c = torch.empty((M, N), dtype=torch.float32, device=a.device)
    else:
        _check_matrix(c, "c")
        if tuple(c.shape) != (M, N):
            raise ValueError(f"c must be {M}x{N}")
    if bias is not None and (not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32
                             or not bias.is_cuda or bias.dim() != 1 or bias.shape[0] != N
                             or (N > 1 and bias.stride(0) != 1)):
        raise TypeError(f"bias must be a contiguous float32 CUDA vector of length {N}")
    st = emu_sgemm_presplit(OP_T if trans_a else OP_N, M, N, K, alpha, a.data_ptr(), _ld(a),
                            pb.planes.data_ptr(), beta, c.data_ptr(), _ld(c),
                            bias.data_ptr() if bias is not None else 0, pb.mode, ksplit,
                            _stream_handle(stream))
    if st != STATUS_SUCCESS:
        raise EmuError(st, "emu_sgemm_presplit")
    return c


def split_bf16x3(x, stream=None):
    """(hi, mid', lo') int16 tensors holding the BF16 bit patterns of the
    exact three-piece split of the float32 CUDA tensor ``x`` (any shape,
    contiguous)."""
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 CUDA tensor")
    hi = torch.empty(x.shape, dtype=torch.int16, device=x.device)
    mid = torch.empty_like(hi)
    lo = torch.empty_like(hi)
    st = emu_split_bf16x3(x.data_ptr(), x.numel(), hi.data_ptr(), mid.data_ptr(), lo.data_ptr(),
                          _stream_handle(stream))
    if st != STATUS_SUCCESS:
        raise EmuError(st, "emu_split_bf16x3")
    return hi, mid, lo


def select_mode(M, N, K, trans_a=False, trans_b=False) -> str:
    """Mode the AUTO ("performant") policy runs for this shape."""
    st, name = emu_sgemm_select(OP_T if trans_a else OP_N, OP_T if trans_b else OP_N, M, N, K)
    if st != STATUS_SUCCESS:
        raise EmuError(st, "emu_sgemm_select")
    return name


def select_ksplit(M, N, K) -> int:
    """K split the emulated modes use for this shape when A allows one."""
    st, sp = emu_sgemm_ksplit(M, N, K)
    if st != STATUS_SUCCESS:
        raise EmuError(st, "emu_sgemm_ksplit")
    return sp


def select_plan(M, N, K):
    """(ksplit, tile_rows, split_from) of the AUTO policy's emulated plan:
    tiles of tile_rows x 128, numbered row by row, those from split_from on
    split into ksplit K segments."""
    st, plan = emu_sgemm_plan(M, N, K)
    if st != STATUS_SUCCESS:
        raise EmuError(st, "emu_sgemm_plan")
    return plan
