"""Compile the plain C client of libpdq (host code only, gcc): `python tests/c_client/build.py`.

The client links libpdq.so (built first) and the HIP runtime; its run path
finds the library relative to the binary, so the tree can move.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "pdq_c_client")


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or "cc"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           os.path.join(HERE, "pdq_c_client.c"), "-o", BIN + ".tmp",
           "-L", os.path.join(ROOT, "w8a8_int8_quantized_absmax_amd"), "-lpdq",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../w8a8_int8_quantized_absmax_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C client build failed:\n{res.stdout}{res.stderr}")
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
