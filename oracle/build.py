"""Build the CPU oracle shared library (``oracle/libspecoracle.so``) with gcc.

Test infrastructure: the oracle is the checker, never the product.  Strict IEEE
double arithmetic (no fast-math, no FMA contraction) so the oracle's results
follow the definitions literally.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["philox.c", "verify.c", "expand.c", "draft.c"]
LIB = os.path.join(HERE, "libspecoracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", LIB + ".tmp",
    ] + [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
