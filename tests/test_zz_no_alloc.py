"""The allocation-free entry point, gemm_relu_f16_noalloc, on the GPU.

Its split-K scratch is the library's fixed per-GPU array instead of a
per-stream workspace; its results must be those of gemm_relu_f16 (the same
kernels and split counts, so the same bits) and within the oracle's
tolerance, on calls in a row that reuse the array, under graph capture, and
with the size limit enforced.
"""
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


def say(*msg):
    print(*msg, file=sys.stderr, flush=True)


def call_both(a, b, stream=None):
    """C from gemm_relu_f16_noalloc and from gemm_relu_f16, both through the C ABI."""
    M, K = a.shape
    N = b.shape[1]
    s = stream or torch.cuda.current_stream()
    c0 = torch.full((M, N), 5.0, dtype=torch.float16, device="cuda")
    c1 = torch.full((M, N), 6.0, dtype=torch.float16, device="cuda")
    with torch.cuda.stream(s):
        st0 = gr.gemm_relu_f16_noalloc(M, N, K, a.data_ptr(), b.data_ptr(), c0.data_ptr(), s.cuda_stream)
        st1 = gr.gemm_relu_f16(M, N, K, a.data_ptr(), b.data_ptr(), c1.data_ptr(), s.cuda_stream)
    torch.cuda.synchronize()
    assert st0 == gr.OK, gr.strerror(st0)
    assert st1 == gr.OK, gr.strerror(st1)
    return workloads.as_u16(c0.cpu()), workloads.as_u16(c1.cpu())


@pytest.mark.parametrize("first,second", [
    ((16, 8192, 8192), (16, 2048, 4096)),     # split-K with 4, then 8 splits
    ((24, 4096, 4096), (32, 1024, 2048)),     # 64 tiles, 4 splits; then 32 tiles, 4 splits
    ((1000, 1016, 1000), (16, 8192, 1024)),   # no scratch, then split-K
])
def test_two_calls_in_a_row_match_gemm_relu_f16(first, second):
    for i, (M, N, K) in enumerate((first, second)):
        w = workloads.Workload(f"noalloc_{M}x{N}x{K}", M, N, K, "normal", 1.0, 90 + i)
        say(f"[noalloc] call {i}: {M}x{N}x{K} tile {gr.tile_name(gr.select_tile(M, N, K))}")
        a, b = workloads.workload_inputs(w)
        got, ref = call_both(a.cuda(), b.cuda())
        assert np.array_equal(got, ref), f"call {i}: differs from gemm_relu_f16"
        want, absdot = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b), want_absdot=True)
        parity.check(got, want, absdot=absdot, K=K, label=f"noalloc call {i} {M}x{N}x{K}")


def test_integer_sums_bit_exact_and_repeatable():
    M, N, K = 16, 4096, 8192
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=93)
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    ad, bd = a.cuda(), b.cuda()
    for rep in range(5):
        got, ref = call_both(ad, bd)
        assert np.array_equal(got, want), f"repeat {rep}"
        assert np.array_equal(ref, want)


def test_captured_calls_replay_correctly():
    M, N, K = 32, 2048, 8192
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=94)
    a2, b2 = workloads.make_inputs(16, 1024, 2048, dist="intsmall", seed=95)
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    want2 = oracle.gemm_relu_f16(workloads.as_u16(a2), workloads.as_u16(b2))
    ad, bd, a2d, b2d = a.cuda(), b.cuda(), a2.cuda(), b2.cuda()
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    out2 = torch.empty((16, 1024), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = gr.gemm_relu_f16_noalloc(M, N, K, ad.data_ptr(), bd.data_ptr(), out.data_ptr(), s.cuda_stream)
    assert st == gr.OK, gr.strerror(st)
    for rep in range(3):
        out.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(workloads.as_u16(out.cpu()), want), f"replay {rep}"
        # eager use of the same array between replays
        st = gr.gemm_relu_f16_noalloc(16, 1024, 2048, a2d.data_ptr(), b2d.data_ptr(), out2.data_ptr(), 0)
        assert st == gr.OK
        torch.cuda.synchronize()
        assert np.array_equal(workloads.as_u16(out2.cpu()), want2), f"eager {rep}"


def test_too_large_for_the_scratch_is_refused():
    # 32 rows, 33 tiles of 32 x 128: 4 splits, 2.03 MiB of partial sums
    M, N, K = 32, 4160, 8192
    assert gr.tile_name(gr.select_tile(M, N, K)).startswith("splitk_32x128")
    assert 4 * M * N * 4 > gr.NOALLOC_MAX_PARTIAL_BYTES
    a = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    b = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    c = torch.full((M, N), 9.0, dtype=torch.float16, device="cuda")
    st = gr.gemm_relu_f16_noalloc(M, N, K, a.data_ptr(), b.data_ptr(), c.data_ptr(), 0)
    torch.cuda.synchronize()
    assert st == gr.ETOOBIG
    assert bool((c == 9.0).all())   # nothing was launched
    # the array is still usable after a refusal (32 x 8192 x 8192: 128 tiles
    # of 16 x 128, 2 splits, 2 MiB of partial sums)
    M, N, K = 32, 8192, 8192
    assert "splitk" in gr.tile_name(gr.select_tile(M, N, K))
    w = workloads.Workload("noalloc_after_refusal", M, N, K, "normal", 0.02, 96)
    a, b = workloads.workload_inputs(w)
    got, ref = call_both(a.cuda(), b.cuda())
    assert np.array_equal(got, ref)
