"""The matrix-core ceiling probe (csrc/mfma_ceiling.hip) is a stand-alone
gfx950 program; on the CPU it must compile, and it must refuse a bad
argument before touching a GPU."""
import os
import subprocess

import pytest

from tiled_dense_gemm_f16_amd import build as build_mod


@pytest.mark.skipif(not os.path.exists(build_mod.hipcc()), reason="hipcc not installed")
def test_ceiling_probe_compiles(tmp_path, monkeypatch):
    out = tmp_path / "mfma_ceiling"
    monkeypatch.setattr(build_mod, "CEILING_BIN", str(out))
    assert build_mod.build_ceiling() == str(out)
    assert out.exists() and os.access(out, os.X_OK)
    # usage errors are caught before any HIP call
    res = subprocess.run([str(out), "0"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2 and "usage" in res.stderr
    res = subprocess.run([str(out), "31"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2


def test_ceiling_probe_source_names_the_gemm_instruction():
    src = open(build_mod.CEILING_SRC).read()
    assert "__builtin_amdgcn_mfma_f32_32x32x16_f16" in src
