"""The offline tile sweep on the GPU: every candidate is launched, validated
and timed, the winner is stored and read back, and the stored launch gives the
oracle's result."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import tiled_dense_gemm_f16_amd as gr  # noqa: E402
from tiled_dense_gemm_f16_amd import tune  # noqa: E402


def say(*msg):
    print(*msg, file=sys.stderr, flush=True)


def oracle_check(c_bits, a_bits, b_bits, bias_bits):
    """The tuner's checker in the tests: the CPU oracle, within the contract's
    tolerance (plus the fp32 bound of the GELU epilogue)."""
    if bias_bits is None:
        want = oracle.gemm_relu_f16(a_bits, b_bits)
    else:
        want = oracle.gemm_bias_gelu_f16(a_bits, b_bits, bias_bits)
    g = c_bits.view(np.float16).astype(np.float64)
    o = want.view(np.float16).astype(np.float64)
    return int((~(np.abs(g - o) <= 1e-2 + 1e-2 * np.abs(o))).sum())


@pytest.mark.parametrize("epilogue", ["relu", "bias_gelu"])
def test_sweep_validates_every_candidate(epilogue, tmp_path):
    M, N, K = 320, 512, 264
    say(f"[tune] {epilogue} {M}x{N}x{K}")
    r = tune.tune(M, N, K, epilogue=epilogue, graph=4, replays=3, check=oracle_check)
    failed = [x for x in r["results"] if not x["ok"]]
    assert not failed, failed
    assert len(r["results"]) == len(tune.candidates(M, N, K))
    times = [x["us"] for x in r["results"]]
    assert times == sorted(times) and all(t > 0 for t in times)
    assert r["best"] is r["results"][0] and r["arch"].startswith("gfx950")
    assert r["default"] is not None and r["default"]["tile"] == gr.select_tile(M, N, K)
    path = str(tmp_path / "tuned.json")
    tune.save(r, path)
    kw = tune.lookup(path, r["arch"], epilogue, M, N, K)
    assert kw == {k: r["best"][k] for k in ("tile", "block_order", "group_m")}


def test_failed_candidate_is_never_chosen():
    bad = {"tile": gr.tile_count(), "tile_name": "none", "block_order": 0, "group_m": 0}
    r = tune.tune(64, 64, 64, graph=2, replays=1, only=[bad])
    assert r["best"] is None and not r["results"][0]["ok"]
    good = {"tile": 2, "tile_name": gr.tile_name(2), "block_order": 0, "group_m": 0}
    r = tune.tune(64, 64, 64, graph=2, replays=1, only=[bad, good])
    assert r["best"]["tile"] == 2 and [x["ok"] for x in r["results"]] == [True, False]


def test_checker_rejects_wrong_outputs():
    # a checker that rejects everything: no candidate may be chosen
    r = tune.tune(64, 128, 64, graph=2, replays=1, check=lambda c, *_: c.size)
    assert r["best"] is None and all(not x["ok"] for x in r["results"])
    # the default (agreement with the library's default launch) accepts the
    # candidates that compute the product
    r = tune.tune(64, 128, 64, graph=2, replays=1)
    assert r["best"] is not None and all(x["ok"] for x in r["results"])


def test_stored_winner_matches_the_oracle(tmp_path):
    w = workloads.Workload("tune_1000x1016x1000", 1000, 1016, 1000, "uniform", 1.0, 0)
    r = tune.tune(w.M, w.N, w.K, graph=4, replays=3, check=oracle_check)
    path = str(tmp_path / "tuned.json")
    tune.save(r, path)
    kw = tune.lookup(path, r["arch"], "relu", w.M, w.N, w.K)
    say(f"[tune] winner {kw} {r['best']['tile_name']}")
    a, b = workloads.workload_inputs(w)
    c = gr.gemm_relu(a.cuda(), b.cuda(), **kw)
    torch.cuda.synchronize()
    got = workloads.as_u16(c.cpu())
    ref = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    parity.check(got, ref, label=f"tuned {kw}")
    assert np.array_equal(got.shape, ref.shape)
