"""Compile libpdq.so (HIP, gfx950) in-tree: `python -m w8a8_int8_quantized_absmax_amd.build_lib`."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpdq.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE binary32: correctly rounded division, no contraction into FMA,
    # denormals kept; the quantization codes depend on it.
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-FP32 instructions in the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _quiet(text: str) -> str:
    return "\n".join(line for line in text.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in line)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpdq)")


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip to an object (in parallel), then link libpdq.so."""
    from concurrent.futures import ThreadPoolExecutor

    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *HIPCC_FLAGS, "-c", "-I", INCLUDE, "-I", CSRC, src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        return obj, res.returncode, _quiet(res.stdout + res.stderr)

    with ThreadPoolExecutor(max_workers=min(len(sources), os.cpu_count() or 1, 8)) as ex:
        results = list(ex.map(compile_one, sources))
    for obj, rc, out in results:
        if rc != 0:
            raise RuntimeError(f"libpdq build failed ({obj}):\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _, _ in results], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"libpdq link failed:\n{_quiet(res.stdout + res.stderr)}")
    # the library must load (every symbol resolved) before it replaces the
    # previous one: a kernel whose host stub the compiler did not emit only
    # shows up here (loaded in a child process, which makes no HIP call)
    chk = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({tmp!r})"], capture_output=True,
                         text=True)
    if chk.returncode != 0:
        raise RuntimeError(f"libpdq does not load:\n{chk.stderr.strip()[-2000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
