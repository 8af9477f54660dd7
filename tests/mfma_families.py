"""Random families of matrix-instruction inputs (exact BF16 operands) for
the tests of the matrix-unit model: operands A (M x 32) and B (32 x N) whose
entry (i, j) is one K = 32 dot product, i.e. two instructions of 16
products.  Inputs only: no arithmetic of the method or of the model.

* wide exponents: random signs and significands over 2^-30..2^30, 15 %
  zeros;
* cancellation: the second instruction's products nearly cancel the
  first's sum;
* binade edges: accumulators at and just below powers of two, small second
  products;
* ties: products that land on half-units of the grid;
* round bits: an accumulator +-(1.5 + 0 or 1 ulp) 2^x built exactly by the
  first instruction, then a half-ulp term and a power-of-two term 2^(x-t),
  t = 25..41, of either sign: the sum's bits past the 24th decide the FP32
  rounding, so the number of bits kept before it and their rounding show.
"""
import numpy as np

FAMILIES = ["wide exponents", "cancellation", "binade edges", "ties", "round bits"]


def _bf16(rng, shape, lo, hi):
    m = rng.integers(128, 256, shape) * rng.choice([-1, 1], shape)
    return (m * 2.0 ** (rng.integers(lo, hi, shape) - 7)).astype(np.float32)


def family(name, rng, M, N):
    """Operands A (M x 32), B (32 x N), all exact BF16 numbers."""
    if name == "wide exponents":
        a, b = _bf16(rng, (M, 32), -30, 30), _bf16(rng, (32, N), -30, 30)
        a[rng.random((M, 32)) < 0.15] = 0.0
    elif name == "cancellation":
        # the second instruction's products nearly cancel the first's sum:
        # a_k negated, b_k one BF16 unit (of 2^-7 relative) off or equal
        a, b = _bf16(rng, (M, 32), -4, 4), _bf16(rng, (32, N), -4, 4)
        a[:, 16:24] = -a[:, 0:8]
        m = rng.integers(129, 255, (8, N)) * rng.choice([-1, 1], (8, N))
        e = rng.integers(-4, 4, (8, N)) - 7
        b[0:8, :] = (m * 2.0**e).astype(np.float32)
        b[16:24, :] = ((m + rng.integers(-1, 2, (8, N))) * 2.0**e).astype(np.float32)
    elif name == "binade edges":
        # accumulators just below and at powers of two, small second products
        a = np.zeros((M, 32), np.float32)
        b = np.zeros((32, N), np.float32)
        a[:, 0] = 2.0 ** rng.integers(-3, 4, M)
        b[0, :] = 1.0
        a[:, 1] = -(2.0 ** rng.integers(-30, -20, M))
        b[1, :] = rng.choice([0.0, 1.0, 2.0, 4.0], N)
        a[:, 16:] = _bf16(rng, (M, 16), -26, -10)
        b[16:, :] = _bf16(rng, (16, N), -6, 6)
    elif name == "ties":
        # products of 1.5 x 2^-12 style operands land on half-units of the grid
        a = (1.5 * 2.0 ** rng.integers(-14, -9, (M, 32)) * rng.choice([-1, 1], (M, 32))).astype(np.float32)
        b = (2.0 ** rng.integers(-14, -9, (32, N)) * rng.choice([-1, 1], (32, N))).astype(np.float32)
        a[:, 0] = 1.0
        b[0, :] = rng.choice([1.0, -1.0, 2.0], N)
        a[:, 16] = 1.0
        b[16, :] = rng.choice([0.0, 1.0], N)
    elif name == "round bits":
        a = np.zeros((M, 32), np.float32)
        b = np.zeros((32, N), np.float32)
        x = rng.integers(-10, 10, M)
        sgn = rng.choice([-1.0, 1.0], M)
        t = rng.integers(25, 42, M)
        a[:, 0] = sgn * 1.5 * 2.0**x
        a[:, 1] = sgn * 2.0 ** (x - 23) * rng.integers(0, 2, M)
        b[0, :] = 1.0
        b[1, :] = 1.0
        a[:, 16] = sgn * 2.0 ** (x - 24)
        a[:, 17] = sgn * 2.0 ** (x - t)
        b[16, :] = rng.choice([0.0, 1.0], N)
        b[17, :] = rng.choice([-1.0, 0.0, 1.0], N)
    else:
        raise ValueError(name)
    return a, b
