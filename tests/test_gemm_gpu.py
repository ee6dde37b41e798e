"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Every case draws seeded inputs on the CPU, runs gemm_relu_f16 on cuda:0 and
compares with the oracle element by element: within rtol = atol = 1e-2 for
floating-point inputs (plus the tighter fp32-accumulation bound), bit for bit
for integer-valued inputs, whose fp32 sums are exact in any order.
"""
from __future__ import annotations

import itertools
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


def run(a_cpu, b_cpu, **kw) -> np.ndarray:
    a = a_cpu.cuda()
    b = b_cpu.cuda()
    c = gr.gemm_relu(a, b, **kw)
    torch.cuda.synchronize()
    return workloads.as_u16(c.cpu())


def neg(t):
    return (-t).contiguous()


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("w", [workloads.SQUARE_256, workloads.SQUARE_1024, workloads.RAGGED, workloads.SKINNY,
                               *[s for s in workloads.SHARDS if s.M == workloads.SKINNY.M]],
                         ids=lambda w: w.name)
def test_workload_full_parity(w):
    say(f"[parity] {w.name} M={w.M} N={w.N} K={w.K} seed={w.seed} tile={gr.select_tile(w.M, w.N, w.K)}")
    a, b = workloads.workload_inputs(w)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    for sign, aa, AA in ((+1, a, A), (-1, neg(a), workloads.as_u16(neg(a)))):
        got = run(aa, b)
        want, absdot = oracle.gemm_relu_f16(AA, B, want_absdot=True)
        st = parity.check(got, want, absdot=absdot, K=w.K, label=f"{w.name} sign={sign}")
        say(f"  sign={sign:+d} {st}")


@pytest.mark.parametrize("w", [workloads.SQUARE_4096, *[s for s in workloads.SHARDS if s.M == 4096]],
                         ids=lambda w: w.name)
def test_workload_4096_sampled(w):
    say(f"[parity] {w.name} sampled, tile={gr.select_tile(w.M, w.N, w.K)}")
    a, b = workloads.workload_inputs(w)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    got = run(a, b)
    got_neg = run(neg(a), b)
    # properties at full size: finite, non-negative, never both signs positive
    g = parity.f16_values(got)
    gn = parity.f16_values(got_neg)
    assert np.isfinite(g).all() and (g >= 0).all()
    assert not ((g > 0) & (gn > 0)).any()
    # whole rows at the start, middle and end (every column tile, every lane)
    for r0, r1 in ((0, 8), (2044, 2052), (4088, 4096)):
        want, absdot = oracle.gemm_relu_f16(A, B, rows=(r0, r1), want_absdot=True)
        parity.check(got[r0:r1], want, absdot=absdot, K=w.K, label=f"rows {r0}:{r1}")
    # random elements, both signs
    rng = np.random.default_rng(4096)
    ii = rng.integers(0, w.M, 4096)
    jj = rng.integers(0, w.N, 4096)
    want, absdot = oracle.gemm_relu_f16_points(A, B, ii, jj, want_absdot=True)
    parity.check(got[ii, jj], want, absdot=absdot, K=w.K, label="points")
    AN = workloads.as_u16(neg(a))
    want_n, absdot_n = oracle.gemm_relu_f16_points(AN, B, ii, jj, want_absdot=True)
    parity.check(got_neg[ii, jj], want_n, absdot=absdot_n, K=w.K, label="points, -A")


# ---------------------------------------------------------------------------
# bit-exact cases: integer-valued inputs make every fp32 partial sum exact
# ---------------------------------------------------------------------------

INT_SHAPES = [(256, 256, 256), (1000, 1016, 1000), (16, 8192, 8192), (512, 512, 4096),
              (33, 47, 129), (100, 77, 333), (1, 1, 1), (300, 260, 64)]


@pytest.mark.parametrize("M,N,K", INT_SHAPES)
def test_integer_inputs_bit_exact(M, N, K):
    say(f"[exact] M={M} N={N} K={K} tile={gr.select_tile(M, N, K)}")
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=M + N + K)
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    got = run(a, b)
    assert np.array_equal(got, want), f"{np.sum(got != want)} mismatches"


# Each tile walks K from a step set by its position; with a K tail (K not a
# multiple of the step) the partial step lands anywhere in the walk. Integer
# inputs keep every fp32 sum exact, so any walk order must give the oracle's
# bits: the 256 x 256 tile past one round (where it skews), the 64 x 256
# tiles with four and five slots and the 64 x 64 tile, operands as stored and
# transposed; and the tiles that load A two steps at a time, whose walk starts
# on an even step (the K tail inside the last pair) and does not skew when the
# step count is odd (K = 984: 31 steps).
SKEW_CASES = [(0, 4160, 4160, 1000, False, False), (0, 4160, 4160, 1000, True, True), (0, 4160, 4160, 1000, False, True),
              (10, 1088, 1024, 1000, False, False), (10, 1088, 1024, 1000, True, False),
              (13, 1088, 1024, 1000, False, False), (13, 1088, 1024, 1000, False, True),
              (11, 1088, 1088, 1000, False, False), (9, 2112, 2048, 1000, False, False),
              (14, 4160, 4160, 1000, False, False), (14, 4160, 4160, 1000, False, True),
              (14, 4160, 4160, 984, False, False), (15, 2112, 2048, 1000, False, False),
              (15, 2112, 2048, 984, False, True), (16, 1088, 1024, 1000, False, False),
              (16, 1088, 1024, 1000, False, True)]


@pytest.mark.parametrize("tile,M,N,K,ta,tb", SKEW_CASES)
def test_skewed_k_walk_with_k_tail_bit_exact(tile, M, N, K, ta, tb):
    say(f"[skew] tile={tile} {gr.tile_name(tile)} M={M} N={N} K={K} ta={ta} tb={tb}")
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=M + 3 * N + 7 * K + tile)
    a_st = a.t().contiguous() if ta else a
    b_st = b.t().contiguous() if tb else b
    c = gr.gemm_relu(a_st.cuda(), b_st.cuda(), trans_a=ta, trans_b=tb, tile=tile)
    torch.cuda.synchronize()
    got = workloads.as_u16(c.cpu())
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    if M * N * K <= 2 ** 31:
        want = oracle.gemm_relu_f16(A, B)
        assert np.array_equal(got, want), f"{np.sum(got != want)} mismatches"
    else:
        # whole rows at the start, middle and end: every column tile, every
        # row tile's position in its group
        for r0 in (0, M // 2 - 4, M - 8):
            want = oracle.gemm_relu_f16(A, B, rows=(r0, r0 + 8))
            assert np.array_equal(got[r0:r0 + 8], want), f"rows {r0}: {np.sum(got[r0:r0 + 8] != want)} mismatches"
        rng = np.random.default_rng(M + K)
        ii, jj = rng.integers(0, M, 4096), rng.integers(0, N, 4096)
        want = oracle.gemm_relu_f16_points(A, B, ii, jj)
        assert np.array_equal(got[ii, jj], want), f"{np.sum(got[ii, jj] != want)} point mismatches"


def _tile_named(name):
    return next(t for t in range(gr.tile_count()) if gr.tile_name(t) == name)


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 1024), (1280, 2304, 1000), (4096, 4096, 4096)])
def test_paired_a_tile_same_bits_as_plain_on_one_round(M, N, K):
    # Loading A two steps at a time changes where the operands wait in LDS,
    # not the order of the sums: on a grid of one round (where the 256 x 256
    # K walk does not skew) both tiles give the same bits on N(0,1) inputs
    plain = _tile_named("256x256x32s4_w2x2_mfma32x32x16_lds-dma")
    paired = _tile_named("256x256x32s4_w2x2_mfma32x32x16_lds-dma-a2")
    say(f"[paired] M={M} N={N} K={K} tiles {plain} {paired}")
    a, b = workloads.make_inputs(M, N, K, dist="normal", seed=M + N + K)
    a, b = a.cuda(), b.cuda()
    c0 = gr.gemm_relu(a, b, tile=plain)
    c1 = gr.gemm_relu(a, b, tile=paired)
    torch.cuda.synchronize()
    assert torch.equal(c0.view(torch.int16), c1.view(torch.int16))


EDGE = [1, 7, 8, 9, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 257]


def edge_triples():
    # every value in every position, paired with a spread of partners
    out = set()
    for i, v in enumerate(EDGE):
        p = EDGE[(i * 5 + 3) % len(EDGE)]
        q = EDGE[(i * 7 + 11) % len(EDGE)]
        out.update({(v, p, q), (p, v, q), (q, p, v)})
    return sorted(out)


@pytest.mark.parametrize("M,N,K", edge_triples())
def test_edge_shapes_every_tile(M, N, K):
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=M * 7 + N * 3 + K)
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    for tile in [None] + list(range(gr.tile_count())):
        say(f"[edge] M={M} N={N} K={K} tile={tile}")
        got = run(a, b, tile=tile)
        assert np.array_equal(got, want), f"tile {tile}: {np.sum(got != want)} mismatches"


@pytest.mark.parametrize("tile", range(gr.tile_count()))
@pytest.mark.parametrize("w", [workloads.SQUARE_1024, workloads.RAGGED], ids=lambda w: w.name)
def test_each_tile_on_workloads(w, tile):
    say(f"[tile] {w.name} tile={tile} {gr.tile_name(tile)}")
    a, b = workloads.workload_inputs(w)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    want, absdot = oracle.gemm_relu_f16(A, B, want_absdot=True)
    parity.check(run(a, b, tile=tile), want, absdot=absdot, K=w.K, label=f"tile {tile}")


@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (100, 72, 40), (16, 512, 256)])
def test_tiny_negative_sums_give_plus_zero(M, N, K):
    """Sums that round to zero in fp16 leave the epilogue as +0 (0x0000),
    whatever their sign: products of +-2^-14 and +-2^-14 are +-2^-28, below
    half the smallest fp16 subnormal, so the ReLU of the rounded value must
    be +0, as in the oracle (ReLU first, then the rounding). Half of the rows
    also get a term of ordinary size, so not every output is zero."""
    rng = np.random.default_rng(M + N + K)
    a = np.zeros((M, K), dtype=np.float16)
    b = np.zeros((K, N), dtype=np.float16)
    tiny = np.float16(2.0 ** -14)
    a[:, 0] = tiny * rng.choice([-1, 1], M).astype(np.float16)
    b[0, :] = tiny * rng.choice([-1, 1], N).astype(np.float16)
    a[: M // 2, 1] = rng.choice([-1, 1], M // 2).astype(np.float16)
    b[1, :] = rng.integers(-2, 3, N).astype(np.float16)
    at = torch.from_numpy(a.view(np.int16)).view(torch.float16)
    bt = torch.from_numpy(b.view(np.int16)).view(torch.float16)
    want = oracle.gemm_relu_f16(workloads.as_u16(at), workloads.as_u16(bt))
    assert (want[M // 2:] == 0).all() and (want[: M // 2] != 0).any()
    for tile in [None] + list(range(gr.tile_count())):
        say(f"[tiny] M={M} N={N} K={K} tile={tile}")
        got = run(at, bt, tile=tile)
        assert not (got == 0x8000).any(), f"tile {tile}: -0 in the output"
        assert np.array_equal(got, want), f"tile {tile}: {np.sum(got != want)} mismatches"


# ---------------------------------------------------------------------------
# split-K: partial sums across workgroups, combined by the last one
# ---------------------------------------------------------------------------

SPLITK_SHAPES = [(16, 8192, 8192), (1, 4096, 8192), (5, 1032, 1000), (16, 136, 129 * 8),
                 (17, 520, 4096), (32, 128, 64), (40, 2056, 3000), (64, 4096, 4096), (9, 8, 8)]


@pytest.mark.parametrize("tile", [4, 5, 6])
@pytest.mark.parametrize("M,N,K", SPLITK_SHAPES)
def test_splitk_bit_exact_and_repeatable(M, N, K, tile):
    say(f"[splitk] M={M} N={N} K={K} tile={gr.tile_name(tile)}")
    assert "splitk" in gr.tile_name(tile)
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=3 * M + N + K)
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    ad, bd = a.cuda(), b.cuda()
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    # several launches in a row on one workspace: the tile counters reset themselves
    for rep in range(3):
        out.fill_(7.0)
        gr.gemm_relu(ad, bd, out=out, tile=tile)
        torch.cuda.synchronize()
        got = workloads.as_u16(out.cpu())
        assert np.array_equal(got, want), f"launch {rep}: {np.sum(got != want)} mismatches"


@pytest.mark.parametrize("tile", [4, 5, 6])
def test_splitk_tiles_on_larger_m(tile):
    # a pinned split-K tile on more rows than it holds: several row tiles
    M, N, K = 100, 264, 1032
    say(f"[splitk rows] tile={gr.tile_name(tile)} M={M} N={N} K={K}")
    a, b = workloads.make_inputs(M, N, K, dist="normal", seed=11)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    want, absdot = oracle.gemm_relu_f16(A, B, want_absdot=True)
    parity.check(run(a, b, tile=tile), want, absdot=absdot, K=K, label=f"tile {tile}")


def test_splitk_two_streams_and_shapes_interleaved():
    # different streams own different workspaces; shapes that need more
    # counters or partials than an earlier call grow the workspace
    shapes = [(16, 1024, 2048), (16, 8192, 8192), (3, 256, 512)]
    inputs = []
    for i, (M, N, K) in enumerate(shapes):
        a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=100 + i)
        inputs.append((a.cuda(), b.cuda(), oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(2):
        for i, (ad, bd, want) in enumerate(inputs):
            s = streams[(i + rep) % 2]
            with torch.cuda.stream(s):
                outs.append((gr.gemm_relu(ad, bd), want))
    torch.cuda.synchronize()
    for c, want in outs:
        assert np.array_equal(workloads.as_u16(c.cpu()), want)


# ---------------------------------------------------------------------------
# the fused bias + GELU epilogue: C = GELU(A @ B + bias)
# ---------------------------------------------------------------------------

def make_bias(N, seed, scale=1.0):
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return (torch.randn(N, generator=gen) * scale).to(torch.float16)


def run_gelu(a_cpu, b_cpu, bias_cpu, **kw) -> np.ndarray:
    c = gr.gemm_bias_gelu(a_cpu.cuda(), b_cpu.cuda(), bias_cpu.cuda(), **kw)
    torch.cuda.synchronize()
    return workloads.as_u16(c.cpu())


@pytest.mark.parametrize("w", [workloads.SQUARE_256, workloads.SQUARE_1024, workloads.RAGGED,
                               workloads.SKINNY], ids=lambda w: w.name)
def test_bias_gelu_workload_parity(w):
    say(f"[gelu] {w.name} tile={gr.select_tile(w.M, w.N, w.K)}")
    a, b = workloads.workload_inputs(w)
    # bias on the scale of the sums, so both terms matter
    scale = float(np.sqrt(w.K)) * w.scale * w.scale
    bias = make_bias(w.N, seed=w.N, scale=scale)
    A, B, BI = workloads.as_u16(a), workloads.as_u16(b), workloads.as_u16(bias)
    want, absdot = oracle.gemm_bias_gelu_f16(A, B, BI, want_absdot=True)
    st = parity.check_gelu(run_gelu(a, b, bias), want, absdot=absdot, K=w.K,
                           bias_abs=np.abs(parity.f16_values(BI))[None, :], label=w.name)
    say(f"  {st}")


def test_bias_gelu_4096_sampled():
    w = workloads.SQUARE_4096
    say(f"[gelu] {w.name} sampled, tile={gr.select_tile(w.M, w.N, w.K)}")
    a, b = workloads.workload_inputs(w)
    bias = make_bias(w.N, seed=7, scale=64.0)
    A, B, BI = workloads.as_u16(a), workloads.as_u16(b), workloads.as_u16(bias)
    got = run_gelu(a, b, bias)
    bias_abs = np.abs(parity.f16_values(BI))
    for r0, r1 in ((0, 4), (2046, 2050), (4092, 4096)):
        want, absdot = oracle.gemm_bias_gelu_f16(A, B, BI, rows=(r0, r1), want_absdot=True)
        parity.check_gelu(got[r0:r1], want, absdot=absdot, K=w.K, bias_abs=bias_abs[None, :], label=f"rows {r0}:{r1}")
    rng = np.random.default_rng(77)
    ii = rng.integers(0, w.M, 2048)
    jj = rng.integers(0, w.N, 2048)
    want, absdot = oracle.gemm_bias_gelu_f16_points(A, B, BI, ii, jj, want_absdot=True)
    parity.check_gelu(got[ii, jj], want, absdot=absdot, K=w.K, bias_abs=bias_abs[jj], label="points")


@pytest.mark.parametrize("tile", range(gr.tile_count()))
def test_bias_gelu_every_tile_ragged(tile):
    M, N, K = 200, 264, 136
    say(f"[gelu tile] {gr.tile_name(tile)} M={M} N={N} K={K}")
    a, b = workloads.make_inputs(M, N, K, dist="uniform", scale=1.0, seed=31)
    bias = make_bias(N, seed=32, scale=3.0)
    A, B, BI = workloads.as_u16(a), workloads.as_u16(b), workloads.as_u16(bias)
    want, absdot = oracle.gemm_bias_gelu_f16(A, B, BI, want_absdot=True)
    parity.check_gelu(run_gelu(a, b, bias, tile=tile), want, absdot=absdot, K=K,
                      bias_abs=np.abs(parity.f16_values(BI))[None, :], label=f"tile {tile}")


@pytest.mark.parametrize("M,N,K", [(33, 47, 129), (16, 8192, 1024), (300, 264, 64), (1, 8, 8), (77, 40, 24)])
def test_bias_gelu_integer_sums(M, N, K):
    # integer inputs make the fp32 sum exact; only GELU's fp32 evaluation can
    # move a result, by at most one fp16 unit at a rounding boundary
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=M + 3 * N + K)
    bias = make_bias(N, seed=N, scale=2.0)
    A, B, BI = workloads.as_u16(a), workloads.as_u16(b), workloads.as_u16(bias)
    want = oracle.gemm_bias_gelu_f16(A, B, BI)
    got = run_gelu(a, b, bias)
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    sign_zero = ((got | want) & 0x7FFF) == 0  # +0 and -0
    diff[sign_zero] = 0
    assert diff.max() <= 1, f"max difference {diff.max()} fp16 units"
    assert (diff != 0).mean() < 0.01, f"{(diff != 0).sum()} of {diff.size} differ by one unit"


# ---------------------------------------------------------------------------
# memory safety: NaN guard bands after the inputs, sentinels around C
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,off", [(1000, 1016, 1000, 0), (129, 65, 257, 0), (16, 8192, 1000, 0),
                                       (100, 96, 200, 1), (77, 40, 24, 3)])
def test_guard_bands(M, N, K, off):
    say(f"[guard] M={M} N={N} K={K} elem offset={off}")
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=5)
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    G = 4096  # guard elements
    nan = float("nan")
    abuf = torch.full((off + M * K + G,), nan, dtype=torch.float16, device="cuda")
    bbuf = torch.full((off + K * N + G,), nan, dtype=torch.float16, device="cuda")
    abuf[off:off + M * K] = a.reshape(-1).cuda()
    bbuf[off:off + K * N] = b.reshape(-1).cuda()
    sentinel = torch.tensor([0x7777], dtype=torch.int16).view(torch.float16).item()
    cbuf = torch.full((G + off + M * N + G,), sentinel, dtype=torch.float16, device="cuda")
    av = abuf[off:off + M * K].view(M, K)
    bv = bbuf[off:off + K * N].view(K, N)
    cv = cbuf[G + off:G + off + M * N].view(M, N)
    gr.gemm_relu(av, bv, out=cv)
    torch.cuda.synchronize()
    cb = workloads.as_u16(cbuf.cpu())
    assert (cb[:G + off] == 0x7777).all(), "write before C"
    assert (cb[G + off + M * N:] == 0x7777).all(), "write after C"
    assert np.array_equal(cb[G + off:G + off + M * N].reshape(M, N), want)


# ---------------------------------------------------------------------------
# invariance and hygiene
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("w", [workloads.RAGGED, workloads.SKINNY,
                               workloads.Workload("gemm_relu_f16_32x8192x2048_normal0.02", 32, 8192, 2048, "normal", 0.02)],
                         ids=lambda w: w.name)
def test_block_order_does_not_change_results(w):
    # (the split-K tiles accept either order and keep one mapping of
    # workgroups to tiles and splits)
    a, b = workloads.workload_inputs(w)
    ref = run(a, b)
    for order, gm in ((gr.ORDER_ROW_MAJOR, 0), (gr.ORDER_DEFAULT, 1), (gr.ORDER_DEFAULT, 2),
                      (gr.ORDER_DEFAULT, 8), (gr.ORDER_DEFAULT, 64)):
        say(f"[order] {w.name} order={order} group_m={gm}")
        assert np.array_equal(run(a, b, block_order=order, group_m=gm), ref)


@pytest.mark.parametrize("w", [workloads.SQUARE_1024, workloads.RAGGED, workloads.SKINNY], ids=lambda w: w.name)
def test_deterministic_over_repeats(w):
    say(f"[determinism] {w.name}")
    a, b = workloads.workload_inputs(w)
    a, b = a.cuda(), b.cuda()
    ref = gr.gemm_relu(a, b).clone()
    out = torch.empty_like(ref)
    for _ in range(50):
        out.fill_(1.0)
        gr.gemm_relu(a, b, out=out)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    torch.cuda.synchronize()


def test_nondefault_stream():
    w = workloads.SQUARE_1024
    a, b = workloads.workload_inputs(w)
    ref = run(a, b)
    s = torch.cuda.Stream()
    ad, bd = a.cuda(), b.cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c = gr.gemm_relu(ad, bd)
    s.synchronize()
    assert np.array_equal(workloads.as_u16(c.cpu()), ref)


def test_k_zero_gives_zero():
    a = torch.empty((33, 0), dtype=torch.float16, device="cuda")
    b = torch.empty((0, 40), dtype=torch.float16, device="cuda")
    c = torch.full((33, 40), 3.0, dtype=torch.float16, device="cuda")
    gr.gemm_relu(a, b, out=c)
    torch.cuda.synchronize()
    assert not c.float().abs().sum().item()


def test_raw_abi_call_and_empty_shapes():
    a, b = workloads.make_inputs(64, 64, 64, seed=1)
    ad, bd = a.cuda(), b.cuda()
    c = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    st = gr.gemm_relu_f16(64, 64, 64, ad.data_ptr(), bd.data_ptr(), c.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    assert st == gr.OK
    torch.cuda.synchronize()
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    parity.check(workloads.as_u16(c.cpu()), want, label="raw call")
    assert gr.gemm_relu_f16(0, 64, 64, ad.data_ptr(), bd.data_ptr(), c.data_ptr(), 0) == gr.OK


def test_splitk_workspace_under_graph_capture():
    # a stream being captured cannot get a new workspace (allocation and a
    # memset would land in the graph): the call is refused, nothing is
    # recorded; after one call outside capture, capture and replays work
    M, N, K = 16, 1024, 4096
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=77)
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    ad, bd = a.cuda(), b.cuda()
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    assert "splitk" in gr.tile_name(gr.select_tile(M, N, K))
    g = torch.cuda.CUDAGraph()
    st = None
    with torch.cuda.graph(g, stream=s):
        st = gr.gemm_relu_f16(M, N, K, ad.data_ptr(), bd.data_ptr(), out.data_ptr(), s.cuda_stream)
    assert st == gr.EUNSUPPORTED
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        gr.gemm_relu(ad, bd, out=out)   # creates the workspace on s
    torch.cuda.synchronize()
    assert np.array_equal(workloads.as_u16(out.cpu()), want)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s):
        st = gr.gemm_relu_f16(M, N, K, ad.data_ptr(), bd.data_ptr(), out.data_ptr(), s.cuda_stream)
    assert st == gr.OK
    for rep in range(3):
        out.fill_(3.0)
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert np.array_equal(workloads.as_u16(out.cpu()), want), f"replay {rep}"



def test_workspace_growth_keeps_captured_graphs_valid():
    # a graph captured while the stream's workspace was small keeps that
    # workspace's address; a later, larger call grows the workspace, and the
    # graph's replays must still find their partial sums and counters where
    # they were (the replaced workspace is kept, not freed)
    Ms, Ns, Ks = 16, 512, 4096      # 4 tiles of 16 x 128 -> 32 splits, 1 MiB of partials
    Ml, Nl, Kl = 32, 4096, 4096     # larger: 64 tiles of 16 x 128 -> 4 splits, 2 MiB of partials
    a, b = workloads.make_inputs(Ms, Ns, Ks, dist="intsmall", seed=81)
    al, bl = workloads.make_inputs(Ml, Nl, Kl, dist="intsmall", seed=82)
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    want_l = oracle.gemm_relu_f16(workloads.as_u16(al), workloads.as_u16(bl))
    assert "splitk" in gr.tile_name(gr.select_tile(Ms, Ns, Ks))
    assert "splitk" in gr.tile_name(gr.select_tile(Ml, Nl, Kl))
    ad, bd, ald, bld = a.cuda(), b.cuda(), al.cuda(), bl.cuda()
    out = torch.empty((Ms, Ns), dtype=torch.float16, device="cuda")
    out_l = torch.empty((Ml, Nl), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    say(f"[workspace] capture {Ms}x{Ns}x{Ks}, then grow with {Ml}x{Nl}x{Kl}")
    with torch.cuda.stream(s):
        gr.gemm_relu(ad, bd, out=out)   # creates the small workspace on s
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = gr.gemm_relu_f16(Ms, Ns, Ks, ad.data_ptr(), bd.data_ptr(), out.data_ptr(), s.cuda_stream)
    assert st == gr.OK
    with torch.cuda.stream(s):
        gr.gemm_relu(ald, bld, out=out_l)   # grows the workspace of s
    torch.cuda.synchronize()
    assert np.array_equal(workloads.as_u16(out_l.cpu()), want_l)
    # fresh device memory that could reuse freed addresses
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
    for rep in range(3):
        out.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(workloads.as_u16(out.cpu()), want), f"replay {rep}"
        with torch.cuda.stream(s):
            gr.gemm_relu(ald, bld, out=out_l)   # eager work on the grown workspace between replays
        torch.cuda.synchronize()
        assert np.array_equal(workloads.as_u16(out_l.cpu()), want_l), f"eager {rep}"
    assert all(bool((j == 7.0).all()) for j in junk)


@pytest.mark.parametrize("group_m", [2 ** 31 - 1, 2 ** 28 + 1, 5])
@pytest.mark.parametrize("tile", [0, 9, 2])
def test_huge_group_m_is_the_whole_grid(group_m, tile):
    # a group of more tile-rows than the grid has is one group of all of them:
    # every tile is still written exactly once
    M, N, K = 1024, 1024, 96
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=83)
    want = oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b))
    say(f"[group_m] tile {tile} group_m {group_m}")
    got = run(a, b, tile=tile, group_m=group_m)
    assert np.array_equal(got, want)
