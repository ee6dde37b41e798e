"""Builds libgemm_relu.so (gfx950 only) in-tree with hipcc.

Usage: ``python -m tiled_dense_gemm_f16_amd.build`` or ``build()`` from Python.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "gemm_relu.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgemm_relu.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile the HIP library. Always compiles (no staleness shortcut)."""
    out = out or LIB
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {out}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
