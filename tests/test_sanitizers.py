"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The oracle, built by gcc with -fsanitize=address,undefined (oracle/build.py
  --sanitize): its pins -- Philox known answers, closed forms, exhaustive
  enumeration, chi-square with planted mistakes, special cases, expansion
  fixtures, draft sampling, ragged counts -- run in a child Python process
  that preloads gcc's sanitizer runtimes and loads that build.
* The library's host code (argument checks, workspace sizing, the boundary
  price and the phase planner), built by hipcc with the sanitizers on the
  host side only, called from two C programs compiled with clang's
  sanitizers: the header's C99 caller and a driver of the same calls over
  many inputs (tests/c/host_fuzz.c).

Any sanitizer report makes the child fail (UBSan does not recover).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rejection_sampling_verify_03_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from oracle import build as oracle_build
    lib = oracle_build.build(sanitize=True, out=str(tmp_path / "libspecoracle_san.so"))
    tests = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py"))
    env = dict(os.environ, SPEC_ORACLE_LIB=lib, LD_PRELOAD=asan + ":" + ubsan, OMP_NUM_THREADS="4", **SAN_ENV)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + tests, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail


def _hipcc():
    p = os.path.join(ROCM, "bin", "hipcc")
    return p if os.path.exists(p) else shutil.which("hipcc")


def test_host_code_under_sanitizers(tmp_path):
    hipcc, clang = _hipcc(), os.path.join(ROCM, "llvm", "bin", "clang")
    if hipcc is None or not os.path.exists(clang):
        pytest.skip("no hipcc / clang")
    lib = tmp_path / "libspecverify_san.so"
    sources = [os.path.join(CSRC, s) for s in ("api.hip", "verify.hip", "expand.hip", "draft.hip", "shard.hip")]
    # the device code as in the product build; the sanitizers on the host side only
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=undefined",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", str(lib)] + sources,
                   check=True, capture_output=True, timeout=600)
    for prog in ("abi_host_calls.c", "host_fuzz.c"):
        exe = tmp_path / prog[:-2]
        subprocess.run([clang, "-std=c99", "-g", "-Wall", "-Wextra", "-Werror",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", prog),
                        "-o", str(exe), str(lib), "-lm", "-Wl,-rpath," + str(tmp_path),
                        "-Wl,-rpath," + os.path.join(ROCM, "lib")], check=True, timeout=300)
        r = subprocess.run([str(exe)], capture_output=True, text=True, env=dict(os.environ, **SAN_ENV),
                           timeout=300)
        assert r.returncode == 0, (prog, r.stdout[-2000:], r.stderr[-3000:])
        assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, (prog, r.stderr[-3000:])
    assert r.stdout.startswith("ok "), r.stdout
