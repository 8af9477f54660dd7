"""Seeded synthetic inputs for the emulated-FP32 GEMM workloads.

Shared by the tests, the benchmark and the smoke check, for both the HIP path
and the CPU oracle.  This module holds none of the method's arithmetic: only
random draws, their distributions and the shapes of the workloads.

The workloads stand in for the systems measured on "Unlocking Tensor Core
Performance for Machine Learning Interatomic Potentials" (section
"Benchmarking Tensor Core FP32 matrix math on PET": a 192-atom water box, its
17,280-atom supercell and a larger checkpoint), whose model weights and
structures are not available here.  Each atom contributes 32 neighbour
tokens; the linear layers of one transformer block are run as the forward GEMM
Y = X.W (NN) and the input-gradient GEMM dX = dY.W^T (NT) that forces need
(section "TF32x3 on Ampere GPUs": gradients are propagated to layer inputs
through the same emulated arithmetic).

Workloads (index: description)
  0  one GEMM 256^3, A, B ~ U(-1, 1), seed 0
  1  one GEMM 2048^3, stress values s*U(1,2)*2^U(-30,30), 1% zeros,
     0.1% values s*U(0.5,1)*FLT_MAX/2^40, seed 1
  2  192 atoms x 32 = 6,144 rows, d = 256 stack (8 GEMMs), seed 2
  3  17,280 atoms x 32 = 552,960 rows, d = 256 stack (8 GEMMs), seed 3
  4  6,144 rows, d = 1024 stack (8 GEMMs), seed 4
Stack tensors: X ~ N(0,1) (rows x in), W ~ N(0, 1/in) (in x out, row-major),
dY ~ N(0,1) (rows x out); independent per linear layer.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

ROW_BLOCK = 4096  # rows drawn from one generator; lets any row range be made alone
FLT_MAX = float(np.finfo(np.float32).max)

_D256 = (("qkv", 256, 768), ("out", 256, 256), ("ffn1", 256, 512), ("ffn2", 512, 256))
_D1024 = (("qkv", 1024, 3072), ("out", 1024, 1024), ("ffn1", 1024, 4096), ("ffn2", 4096, 1024))

CONFIG_NAMES = {
    0: "gemm-256^3 uniform(-1,1)",
    1: "gemm-2048^3 stress",
    2: "mlip-stack 192 atoms x 32 nbrs (6,144 rows), d=256",
    3: "mlip-stack 17,280 atoms x 32 nbrs (552,960 rows), d=256",
    4: "mlip-stack 6,144 rows, d=1024",
}
STACK_ROWS = {2: 192 * 32, 3: 17280 * 32, 4: 192 * 32}
STACK_LAYERS = {2: _D256, 3: _D256, 4: _D1024}


@dataclass(frozen=True)
class Gemm:
    """One GEMM of a workload: C (M x N) = op(A) . op(B), row-major."""

    config: int
    name: str
    trans_a: bool
    trans_b: bool
    M: int
    N: int
    K: int
    layer: int  # linear-layer index inside a stack, -1 otherwise
    a_tensor: str  # "X" / "dY" for stacks, "A" otherwise
    a_cols: int  # columns of the stored A array
    b_shape: tuple  # shape of the stored B array

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def lda(self) -> int:
        return self.a_cols

    @property
    def ldb(self) -> int:
        return self.b_shape[1]


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def gemms(config: int) -> list:
    """The GEMMs of workload ``config``, in run order."""
    if config == 0:
        return [Gemm(0, "gemm", False, False, 256, 256, 256, -1, "A", 256, (256, 256))]
    if config == 1:
        return [Gemm(1, "gemm", False, False, 2048, 2048, 2048, -1, "A", 2048, (2048, 2048))]
    T = STACK_ROWS[config]
    out = []
    for li, (lname, din, dout) in enumerate(STACK_LAYERS[config]):
        # forward Y = X.W: NN with A = X (T x in), B = W (in x out)
        out.append(Gemm(config, f"{lname}.fwd", False, False, T, dout, din, li, "X", din, (din, dout)))
        # input gradient dX = dY.W^T: NT with A = dY (T x out), B = W stored in x out
        out.append(Gemm(config, f"{lname}.dX", False, True, T, din, dout, li, "dY", dout, (din, dout)))
    return out


def _uniform_pair(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.uniform(-1.0, 1.0, size=(256, 256)).astype(np.float32)
    b = rng.uniform(-1.0, 1.0, size=(256, 256)).astype(np.float32)
    return a, b


def stress_values(rng: np.random.Generator, shape) -> np.ndarray:
    """s*U(1,2)*2^U(-30,30) (continuous exponent, drawn in float64, rounded once
    to float32), then 1% exact +0.0 and 0.1% values s*U(0.5,1)*FLT_MAX/2^40."""
    n = int(np.prod(shape))
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.uniform(-30.0, 30.0, n)
    v = sign * mant * np.exp2(expo)
    zero = rng.random(n) < 0.01
    big = (rng.random(n) < 0.001) & ~zero
    bsign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    bmag = rng.uniform(0.5, 1.0, n) * (FLT_MAX / 2.0**40)
    v = np.where(big, bsign * bmag, v)
    v = np.where(zero, 0.0, v)
    return v.astype(np.float32).reshape(shape)


def _stress_pair(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    a = stress_values(rng, (2048, 2048))
    b = stress_values(rng, (2048, 2048))
    return a, b


_pair_cache: dict = {}


def _pair(config):
    if config not in _pair_cache:
        _pair_cache[config] = _uniform_pair(0) if config == 0 else _stress_pair(1)
    return _pair_cache[config]


def _normal_block(config, layer, tensor_id, block, rows, cols):
    return _rng(config, layer, tensor_id, block).standard_normal((rows, cols), dtype=np.float32)


def normal_rows(config: int, layer: int, tensor_id: int, total_rows: int, cols: int,
                rows=None, threads: int | None = None) -> np.ndarray:
    """Rows of a (total_rows x cols) N(0,1) float32 matrix.

    ``rows`` is None (all rows), a (start, stop) pair, or an index array.  Row
    block b (ROW_BLOCK rows) always comes from generator key
    (config, layer, tensor_id, b), so any subset equals the same rows of the
    full matrix.
    """
    if rows is None:
        rows = (0, total_rows)
    if isinstance(rows, tuple):
        start, stop = rows
        idx = None
    else:
        idx = np.asarray(rows, dtype=np.int64)
        start, stop = (int(idx.min()), int(idx.max()) + 1) if idx.size else (0, 0)
    b0, b1 = start // ROW_BLOCK, (stop + ROW_BLOCK - 1) // ROW_BLOCK
    blocks = list(range(b0, b1))

    def make(b):
        r0 = b * ROW_BLOCK
        nrows = min(ROW_BLOCK, total_rows - r0)
        return _normal_block(config, layer, tensor_id, b, nrows, cols)

    if idx is None:
        out = np.empty((stop - start, cols), dtype=np.float32)

        def fill(b):
            blk = make(b)
            r0 = b * ROW_BLOCK
            lo, hi = max(start, r0), min(stop, r0 + blk.shape[0])
            out[lo - start:hi - start] = blk[lo - r0:hi - r0]

        nthreads = threads or min(16, os.cpu_count() or 1)
        if len(blocks) > 1 and nthreads > 1:
            with _cf.ThreadPoolExecutor(nthreads) as ex:
                list(ex.map(fill, blocks))
        else:
            for b in blocks:
                fill(b)
        return out
    out = np.empty((idx.size, cols), dtype=np.float32)
    for b in blocks:
        sel = np.nonzero((idx >= b * ROW_BLOCK) & (idx < (b + 1) * ROW_BLOCK))[0]
        if sel.size == 0:
            continue
        blk = make(b)
        out[sel] = blk[idx[sel] - b * ROW_BLOCK]
    return out


def weight(config: int, layer: int) -> np.ndarray:
    """W (in x out, row-major) ~ N(0, 1/in) of linear ``layer`` of a stack."""
    _, din, dout = STACK_LAYERS[config][layer]
    w = _rng(config, layer, 1).standard_normal((din, dout)) / np.sqrt(din)
    return w.astype(np.float32)


_TENSOR_ID = {"X": 0, "dY": 2}


def make_a(g: Gemm, rows=None, threads=None) -> np.ndarray:
    """The stored A array of GEMM ``g`` (or the given rows of it)."""
    if g.config in (0, 1):
        a = _pair(g.config)[0]
        if rows is None:
            return a
        if isinstance(rows, tuple):
            return a[rows[0]:rows[1]]
        return a[np.asarray(rows)]
    return normal_rows(g.config, g.layer, _TENSOR_ID[g.a_tensor], g.M, g.a_cols, rows, threads)


def make_b(g: Gemm) -> np.ndarray:
    """The stored B array of GEMM ``g``."""
    if g.config in (0, 1):
        return _pair(g.config)[1]
    return weight(g.config, g.layer)


def sample_rows(M: int, stride: int = 64, offset: int = 0) -> np.ndarray:
    """Fixed row sample 1-in-``stride`` (plus the last row) used to check
    full-size GEMMs row by row."""
    idx = np.arange(offset % stride, M, stride, dtype=np.int64)
    if idx.size == 0 or idx[-1] != M - 1:
        idx = np.append(idx, M - 1)
    return idx
