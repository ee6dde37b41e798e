"""Transposed operands on the GPU: C = epilogue(op(A) @ op(B)) with A stored
K x M and/or B stored N x K, through gemm_relu_f16_op / gemm_bias_gelu_f16_op,
compared with the oracle reading the same stored bytes."""
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

LAYOUTS = [(False, True), (True, False), (True, True)]
LAYOUT_IDS = ["NT", "TN", "TT"]


def say(*msg):
    print(*msg, file=sys.stderr, flush=True)


def stored(t, trans):
    """How a logical CPU operand is laid out in memory under a transpose flag."""
    return t.t().contiguous() if trans else t.contiguous()


def run_op(a_st, b_st, ta, tb, bias=None, **kw):
    a, b = a_st.cuda(), b_st.cuda()
    if bias is None:
        c = gr.gemm_relu(a, b, trans_a=ta, trans_b=tb, **kw)
    else:
        c = gr.gemm_bias_gelu(a, b, bias.cuda(), trans_a=ta, trans_b=tb, **kw)
    torch.cuda.synchronize()
    return workloads.as_u16(c.cpu())


# integer-valued inputs: every fp32 sum is exact, so any tile in any layout
# must match the oracle bit for bit -- a wrong index or a dropped tile shows
SHAPES = [(200, 136, 264), (64, 256, 96), (17, 24, 40), (256, 512, 1000), (37, 21, 45), (9, 8, 8), (1, 520, 64)]


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_integer_every_tile(ta, tb, M, N, K):
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=M + 3 * N + 7 * K + ta + 2 * tb)
    A, B = stored(a, ta), stored(b, tb)
    want = oracle.gemm_relu_f16(workloads.as_u16(A), workloads.as_u16(B), trans_a=ta, trans_b=tb)
    for tile in [None] + list(range(gr.tile_count())):
        say(f"[trans int] {'T' if ta else 'N'}{'T' if tb else 'N'} M={M} N={N} K={K} tile={tile}")
        got = run_op(A, B, ta, tb, tile=tile)
        assert np.array_equal(got, want), f"tile {tile}: {int(np.sum(got != want))} mismatches"


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("w", [workloads.SQUARE_256, workloads.SQUARE_1024, workloads.RAGGED, workloads.SKINNY],
                         ids=lambda w: w.name)
def test_workloads_transposed(ta, tb, w):
    a, b = workloads.workload_inputs(w)
    A, B = stored(a, ta), stored(b, tb)
    say(f"[trans] {w.name} {'T' if ta else 'N'}{'T' if tb else 'N'} tile="
        f"{gr.select_tile(w.M, w.N, w.K, trans_a=ta, trans_b=tb)}")
    want, absdot = oracle.gemm_relu_f16(workloads.as_u16(A), workloads.as_u16(B), want_absdot=True,
                                        trans_a=ta, trans_b=tb)
    parity.check(run_op(A, B, ta, tb), want, absdot=absdot, K=w.K, label=f"{w.name} {ta}{tb}")
    # both signs of A, so errors on negative sums are not hidden by the ReLU
    A2 = stored((-a).contiguous(), ta)
    want2 = oracle.gemm_relu_f16(workloads.as_u16(A2), workloads.as_u16(B), trans_a=ta, trans_b=tb)
    parity.check(run_op(A2, B, ta, tb), want2, label=f"{w.name} {ta}{tb} -A")


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
def test_4096_sampled_transposed(ta, tb):
    w = workloads.SQUARE_4096
    a, b = workloads.workload_inputs(w)
    A, B = stored(a, ta), stored(b, tb)
    say(f"[trans] 4096 sampled {'T' if ta else 'N'}{'T' if tb else 'N'}")
    got = run_op(A, B, ta, tb)
    rng = np.random.default_rng(1)
    ii = rng.integers(0, w.M, 4096)
    jj = rng.integers(0, w.N, 4096)
    want, absdot = oracle.gemm_relu_f16_points(workloads.as_u16(A), workloads.as_u16(B), ii, jj,
                                               want_absdot=True, trans_a=ta, trans_b=tb)
    parity.check(got[ii, jj], want, absdot=absdot, K=w.K, label="4096 sampled")


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
def test_bias_gelu_transposed(ta, tb):
    M, N, K = 200, 264, 520
    a, b = workloads.make_inputs(M, N, K, dist="normal", seed=21)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(22)
    bias = (torch.randn(N, generator=gen) * K ** 0.5).half()
    bias_abs = np.abs(oracle.f16_to_f64(workloads.as_u16(bias)))
    A, B = stored(a, ta), stored(b, tb)
    want, absdot = oracle.gemm_bias_gelu_f16(workloads.as_u16(A), workloads.as_u16(B), workloads.as_u16(bias),
                                             want_absdot=True, trans_a=ta, trans_b=tb)
    for tile in (None, 0, 3, 4, 9, 10):
        say(f"[trans gelu] {'T' if ta else 'N'}{'T' if tb else 'N'} tile={tile}")
        parity.check_gelu(run_op(A, B, ta, tb, bias=bias, tile=tile), want, absdot=absdot, K=K,
                          bias_abs=bias_abs[None, :], label=f"gelu tile {tile}")


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("tile", [4, 5, 6])
def test_splitk_transposed(ta, tb, tile):
    # several K splits (the workspace combine) with transposed operands
    M, N, K = 40, 1032, 3072
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=9)
    A, B = stored(a, ta), stored(b, tb)
    want = oracle.gemm_relu_f16(workloads.as_u16(A), workloads.as_u16(B), trans_a=ta, trans_b=tb)
    say(f"[trans splitk] {'T' if ta else 'N'}{'T' if tb else 'N'} tile={gr.tile_name(tile)}")
    for rep in range(2):
        got = run_op(A, B, ta, tb, tile=tile)
        assert np.array_equal(got, want), f"launch {rep}: {int(np.sum(got != want))} mismatches"


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("M,N,K", [(200, 136, 264), (64, 256, 512), (37, 21, 45), (16, 1024, 2048)])
def test_guard_bands_transposed(ta, tb, M, N, K):
    # NaN after each stored operand (an out-of-range read poisons C) and a
    # sentinel around C (an out-of-range write shows)
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=5)
    A, B = stored(a, ta), stored(b, tb)
    want = oracle.gemm_relu_f16(workloads.as_u16(A), workloads.as_u16(B), trans_a=ta, trans_b=tb)
    G = 4096
    nan = float("nan")
    abuf = torch.full((M * K + G,), nan, dtype=torch.float16, device="cuda")
    bbuf = torch.full((K * N + G,), nan, dtype=torch.float16, device="cuda")
    abuf[:M * K] = A.reshape(-1).cuda()
    bbuf[:K * N] = B.reshape(-1).cuda()
    sentinel = torch.tensor([0x7777], dtype=torch.int16).view(torch.float16).item()
    cbuf = torch.full((G + M * N + G,), sentinel, dtype=torch.float16, device="cuda")
    av = abuf[:M * K].view(*A.shape)
    bv = bbuf[:K * N].view(*B.shape)
    cv = cbuf[G:G + M * N].view(M, N)
    for tile in (None, 0, 2, 4, 10):
        say(f"[trans guard] {'T' if ta else 'N'}{'T' if tb else 'N'} M={M} N={N} K={K} tile={tile}")
        cbuf[G:G + M * N] = sentinel
        gr.gemm_relu(av, bv, out=cv, trans_a=ta, trans_b=tb, tile=tile)
        torch.cuda.synchronize()
        cb = workloads.as_u16(cbuf.cpu())
        assert (cb[:G] == 0x7777).all() and (cb[G + M * N:] == 0x7777).all(), "write outside C"
        assert np.array_equal(cb[G:G + M * N].reshape(M, N), want), f"tile {tile}"


def test_nn_through_op_entry_point_matches_plain_call():
    w = workloads.RAGGED
    a, b = workloads.workload_inputs(w)
    ad, bd = a.cuda(), b.cuda()
    c1 = gr.gemm_relu(ad, bd)
    c2 = torch.empty_like(c1)
    st = gr.gemm_relu_f16_op(w.M, w.N, w.K, ad.data_ptr(), gr.OP_N, bd.data_ptr(), gr.OP_N, c2.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert st == gr.OK
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
