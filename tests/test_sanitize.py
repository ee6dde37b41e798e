"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

The oracle is rebuilt with gcc's -fsanitize=address,undefined and its pins
run against it; the HIP library is rebuilt with the same sanitizers on its
host code (argument checks, tile choice, workspace bookkeeping; the GPU code
is unchanged) and the host-only ABI tests run against it. Each run is a
subprocess with the matching sanitizer runtime preloaded; any report aborts
it (UBSan does not recover), so a clean exit means no report.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _run(env_extra: dict, args: list[str]) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *args],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_asan_and_ubsan():
    env = {"ORACLE_SANITIZE": "1"}
    subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"], cwd=ROOT,
                   env={**os.environ, **env}, check=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    assert os.path.isabs(libasan), "gcc's libasan not found"
    r = _run({**env, "LD_PRELOAD": libasan},
             ["tests/test_oracle.py", "tests/test_attention_oracle.py", "-k", "not planted"])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_abi_checks_under_asan_and_ubsan():
    from tiled_dense_gemm_f16_amd import build as hip_build
    lib = hip_build.build(sanitize=True)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "the host code is not instrumented"
    r = _run({"GEMM_RELU_LIB": lib, "LD_PRELOAD": hip_build.asan_runtime()}, ["tests/test_abi.py", "-m", "not gpu"])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
