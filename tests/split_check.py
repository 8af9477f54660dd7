"""ctypes binding of ``split_check.c``: the property check of a three-piece
split over a range of FP32 bit patterns (exact reconstruction, finite
pieces, the nearest-piece bounds, the non-finite conventions).

Test code only.  ``build()`` compiles the checker with gcc next to this
file; ``__graft_entry__.build()`` calls it with the other builds, and
:func:`check_range` builds it on first use when it is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "split_check.c")
_LIB = os.path.join(_HERE, "libsplit_check.so")
_lib = None


def build(verbose: bool = False) -> str:
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.split_check_range.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_int64)]
        lib.split_check_range.restype = ctypes.c_int64
        _lib = lib
    return _lib


def check_range(first: int, hi, mid, lo):
    """(failures, first failing index or -1) for the pieces of the bit
    patterns first, first + 1, ... (mod 2^32), one per element of the uint16
    arrays hi, mid, lo."""
    arrs = [np.ascontiguousarray(x, dtype=np.uint16).ravel() for x in (hi, mid, lo)]
    n = arrs[0].size
    assert all(a.size == n for a in arrs)
    fb = ctypes.c_int64(-1)
    bad = _load().split_check_range(int(first), n, *(a.ctypes.data_as(ctypes.c_void_p) for a in arrs),
                                    ctypes.byref(fb))
    return int(bad), int(fb.value)


if __name__ == "__main__":
    print(build(verbose=True))
