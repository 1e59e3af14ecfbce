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


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, sanitize: bool = False, out: str = None) -> str:
    """Build the oracle library (at ``out``, default oracle/libspecoracle.so).
    sanitize: with AddressSanitizer and UndefinedBehaviorSanitizer (a process
    that loads it must preload gcc's libasan and libubsan)."""
    lib = out or LIB
    cmd = [
        "gcc", "-O1" if sanitize else "-O2", "-g" if sanitize else "-g0", "-std=c11", "-fPIC", "-shared",
        "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
    ] + (SANITIZE_FLAGS if sanitize else []) + [
        "-o", lib + ".tmp",
    ] + [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv,
                out=sys.argv[sys.argv.index("-o") + 1] if "-o" in sys.argv else None))
