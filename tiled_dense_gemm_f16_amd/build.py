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


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the library's
# argument checking, tile choice and workspace code (each -fsanitize= applies
# to the host pass only; GPU code is built as usual). The result needs the
# compiler's ASan runtime preloaded into the process (asan_runtime()).
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
SANITIZED_LIB = os.path.join(PKG, "libgemm_relu_asan.so")
# The timestamp build (GR_STAMPS): the same kernels with per-workgroup
# timestamps at a few points (see common.hpp), for stamps.py.
STAMPS_LIB = os.path.join(PKG, "libgemm_relu_stamps.so")
# The matrix-core ceiling probe: a stand-alone program (no library, no
# Python) that times back-to-back matrix ops with the shader clock and board
# power it reads from sysfs.
CEILING_SRC = os.path.join(PKG, "csrc", "mfma_ceiling.hip")
CEILING_BIN = os.path.join(PKG, "mfma_ceiling")


def asan_runtime() -> str:
    """The shared ASan runtime of the compiler that builds the library."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    out = subprocess.run([os.path.join(rocm, "llvm", "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError("the compiler's ASan runtime was not found")
    return out


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None,
          sanitize: bool = False, stamps: bool = False) -> str:
    """Compile the HIP library. Always compiles (no staleness shortcut).
    sanitize=True builds SANITIZED_LIB with SANITIZE_FLAGS instead;
    stamps=True builds STAMPS_LIB with per-workgroup timestamps."""
    import concurrent.futures

    if sanitize:
        extra_flags = [*(extra_flags or []), *SANITIZE_FLAGS]
        out = out or SANITIZED_LIB
    if stamps:
        extra_flags = [*(extra_flags or []), "-DGR_STAMPS"]
        out = out or STAMPS_LIB
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
        link_flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] if sanitize else []
        res = run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_flags, *objs, "-o", tmp])
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed ({res.returncode}) linking {out}")
        os.replace(tmp, out)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return out


def build_ceiling(verbose: bool = False) -> str:
    """Compile the matrix-core ceiling probe (CEILING_BIN)."""
    tmp = CEILING_BIN + f".tmp{os.getpid()}"
    cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f != "-fPIC"], CEILING_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}) compiling {CEILING_SRC}")
    os.replace(tmp, CEILING_BIN)
    return CEILING_BIN


if __name__ == "__main__":
    if "--ceiling" in sys.argv[1:]:
        print(build_ceiling(verbose=True))
    else:
        print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:], stamps="--stamps" in sys.argv[1:]))
