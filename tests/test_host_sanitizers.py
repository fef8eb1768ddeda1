"""The host side of libpdq under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The C entry points' argument checks, size arithmetic and status strings run
on the host.  This test compiles pdq_api.hip (the host code of every entry
point) with both sanitizers on the host pass only (device code unchanged and
never run here), links it with the library's other objects into a temporary
library, and runs the ABI validation tests (tests/test_abi.py) against it in
a child process with the sanitizer runtime preloaded.  Any report stops that
process, so the child's exit status is the outcome.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "w8a8_int8_quantized_absmax_amd")
OBJ = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _runtime():
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if out.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_validation_under_host_sanitizers(tmp_path):
    others = [o for o in sorted(glob.glob(os.path.join(OBJ, "*.o"))) if not o.endswith("pdq_api.o")]
    if not os.path.exists(HIPCC) or len(others) < 5:
        pytest.skip("hipcc or the library's objects are missing (run __graft_entry__.build() first)")
    rt = _runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    obj = str(tmp_path / "pdq_api_san.o")
    lib = str(tmp_path / "libpdq_san.so")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN,
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    res = subprocess.run([HIPCC, *flags, "-c", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                          os.path.join(PKG, "csrc", "pdq_api.hip"), "-o", obj], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-shared-libasan", obj, *others,
                          "-o", lib], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, PDQ_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (run.stdout + run.stderr)[-4000:]
    assert run.returncode == 0, tail
    assert "passed" in run.stdout and "Sanitizer" not in run.stdout + run.stderr, tail
