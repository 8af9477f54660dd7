"""Compile the CPU oracle (``oracle.c`` -> ``liboracle.so``) with gcc.

Test infrastructure: building the checker is not using it on the product path.
``-ffp-contract=off`` keeps every binary32 operation in the source a single
IEEE operation (no fused multiply-add contraction).
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
