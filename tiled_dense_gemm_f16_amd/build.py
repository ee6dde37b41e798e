"""Builds libgemm_relu.so (gfx950 only) in-tree with hipcc: the GEMM
(csrc/gemm_relu.hip) and the softmax / attention kernels (csrc/attention.hip)
compiled in parallel and linked into one shared library.

Usage: ``python -m tiled_dense_gemm_f16_amd.build`` or ``build()`` from Python.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "gemm_relu.hip")
SRCS = [SRC, os.path.join(PKG, "csrc", "attention.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgemm_relu.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile the HIP library. Always compiles (no staleness shortcut)."""
    import concurrent.futures

    out = out or LIB
    tag = f".tmp{os.getpid()}"
    objs = [out + f".{os.path.splitext(os.path.basename(src))[0]}{tag}.o" for src in SRCS]

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        return subprocess.run(cmd, capture_output=True, text=True)

    cmds = [[hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", "-c", src, "-o", obj]
            for src, obj in zip(SRCS, objs)]
    try:
        with concurrent.futures.ThreadPoolExecutor(len(cmds)) as ex:
            results = list(ex.map(run, cmds))
        for res, src in zip(results, SRCS):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed ({res.returncode}) compiling {src}")
        tmp = out + tag
        res = run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed ({res.returncode}) linking {out}")
        os.replace(tmp, out)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
