"""Build ``libspecverify.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

Flags: no packed-fp32 instructions, no floating-point contraction beyond the
explicit fma calls in the sources (the sampling pass recomputes weights and
must reproduce them bit for bit), -O3.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["verify.hip", "expand.hip", "draft.hip", "shard.hip", "api.hip"]
LIB = os.path.join(HERE, "libspecverify.so")
ARCH = os.environ.get("SPEC_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def compile_flags():
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    cmd = [hipcc()] + compile_flags() + ["-shared", "-o", LIB + ".tmp"] + \
        [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
