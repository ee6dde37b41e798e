"""Row softmax and the attention forward pass on the GPU, through the C ABI,
against the oracle (float64 from the same fp16 bytes).

Bars:
 * softmax: within one fp16 unit in the last place of the oracle's value (the
   kernel's fp32 exp / sum / divide is far inside half an fp16 ulp, so only the
   final rounding may differ, and only by one step);
 * attention: rtol = atol = 1e-2 on every element, and the bound the fp32 /
   fp16 arithmetic implies: half an fp16 ulp of each side plus 1.5 * 2^-10 *
   sum_j p_j |V[j][d]| (p is rounded to fp16 before the product with V, a
   relative 2^-11 per term, and the row sum uses the unrounded p), plus the
   score error of the fp32 dot products; and the log-sum-exp within 1e-4.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import tiled_dense_gemm_f16_amd as gr  # noqa: E402


def say(*msg):
    print(*msg, file=sys.stderr, flush=True)


def f16_vals(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def ulp16(x):
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def randn_f16(shape, seed, scale=1.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).half()


# ---------------------------------------------------------------------------
# row softmax
# ---------------------------------------------------------------------------

SOFTMAX_SHAPES = [(1, 1), (7, 13), (64, 512), (33, 1000), (17, 1001), (256, 4096), (8, 8192), (4, 10000),
                  (3, 8200), (1000, 64)]


@pytest.mark.parametrize("scale", [1.0, 8.0])
@pytest.mark.parametrize("rows,cols", SOFTMAX_SHAPES)
def test_softmax_rows(rows, cols, scale):
    say(f"[softmax] rows={rows} cols={cols} scale={scale}")
    x = randn_f16((rows, cols), seed=rows * 7 + cols, scale=scale)
    want = f16_vals(oracle.softmax_rows_f16(workloads.as_u16(x)))
    got = f16_vals(workloads.as_u16(gr.softmax_rows(x.cuda()).cpu()))
    err = np.abs(got - want)
    bound = ulp16(want) + 2.0 ** -24
    assert (err <= bound).all(), f"max err {err.max()} at {np.unravel_index(err.argmax(), err.shape)}"


def test_softmax_in_place_and_large_values():
    x = randn_f16((32, 2048), seed=3, scale=1.0)
    x[:, 0] = 60000.0   # far above the rest: the row's maximum must come out first
    x[:, 1] = 59990.0
    want = f16_vals(oracle.softmax_rows_f16(workloads.as_u16(x)))
    xd = x.cuda()
    gr.softmax_rows(xd, out=xd)
    torch.cuda.synchronize()
    got = f16_vals(workloads.as_u16(xd.cpu()))
    assert np.isfinite(got).all()
    assert (np.abs(got - want) <= ulp16(want) + 2.0 ** -24).all()


# ---------------------------------------------------------------------------
# attention forward
# ---------------------------------------------------------------------------

def run_attn(q, k, v, causal, scale):
    o, lse = gr.flash_attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    return workloads.as_u16(o.cpu()), lse.cpu().numpy().astype(np.float64)


def check_attn(got_bits, want_bits, pv, lse_got, lse_want, K_abs_dot, label):
    g, o = f16_vals(got_bits), f16_vals(want_bits)
    err = np.abs(g - o)
    bad = ~(err <= 1e-2 + 1e-2 * np.abs(o))
    assert not bad.any(), f"{label}: {int(bad.sum())} outside rtol/atol 1e-2, max err {err.max()}"
    bound = 0.5 * ulp16(o) + 0.5 * ulp16(g) + 1.5 * 2.0 ** -10 * pv + K_abs_dot + 1e-7
    ratio = float((err / bound).max(initial=0.0))
    assert ratio <= 1.0, f"{label}: beyond the fp32/fp16 bound (ratio {ratio:.3f})"
    lerr = np.abs(lse_got - lse_want)
    assert (lerr <= 1e-4 * (1 + np.abs(lse_want))).all(), f"{label}: lse err {lerr.max()}"
    return ratio


def score_bound(q, k, scale):
    """Scale of the fp32 score error, carried into O: D * 2^-24 * max_j sum_d |q||k| * scale
    per row, times max |V| -- small next to the p rounding but stated."""
    qa = np.abs(f16_vals(workloads.as_u16(q)))
    ka = np.abs(f16_vals(workloads.as_u16(k)))
    D = q.shape[-1]
    s = np.einsum("bhid,bhjd->bhij", qa, ka).max(axis=-1) * abs(scale)
    return (D * 2.0 ** -24 * s)[..., None] * 4.0


ATTN_SHAPES = [(1, 1, 1, 1), (1, 2, 64, 64), (2, 3, 300, 300), (1, 2, 256, 512), (1, 1, 513, 100),
               (1, 2, 1024, 1024), (1, 1, 70, 1500)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Sq,Skv", ATTN_SHAPES)
def test_attention_full(B, H, Sq, Skv, causal, D):
    say(f"[attn] B={B} H={H} Sq={Sq} Skv={Skv} D={D} causal={causal}")
    seed = B * 1000 + H * 100 + Sq + 3 * Skv + D + causal
    q = randn_f16((B, H, Sq, D), seed)
    k = randn_f16((B, H, Skv, D), seed + 1)
    v = randn_f16((B, H, Skv, D), seed + 2)
    scale = 1.0 / math.sqrt(D)
    got, lse = run_attn(q, k, v, causal, scale)
    want, lse_o, pv = oracle.attention_f16(workloads.as_u16(q), workloads.as_u16(k), workloads.as_u16(v), scale,
                                           causal, want_lse=True, want_pv=True)
    r = check_attn(got, want, pv, lse, lse_o, score_bound(q, k, scale), f"B{B} H{H} Sq{Sq} Skv{Skv} D{D} c{causal}")
    say(f"[attn]   max ratio to bound {r:.3f}")


@pytest.mark.parametrize("causal", [False, True])
def test_attention_sampled_large(causal):
    # the bench shape: B = 4, H = 32, S = 4096, D = 128; sampled rows
    B, H, S, D = 4, 32, 4096, 128
    say(f"[attn] sampled B={B} H={H} S={S} D={D} causal={causal}")
    q = randn_f16((B, H, S, D), 41)
    k = randn_f16((B, H, S, D), 42)
    v = randn_f16((B, H, S, D), 43)
    scale = 1.0 / math.sqrt(D)
    got, lse = run_attn(q, k, v, causal, scale)
    rng = np.random.default_rng(5)
    bh = rng.integers(0, B * H, 256)
    qi = np.concatenate([rng.integers(0, S, 252), [0, 1, S - 1, 2047]])
    want, lse_o, pv = oracle.attention_rows_f16(workloads.as_u16(q), workloads.as_u16(k), workloads.as_u16(v), scale,
                                                causal, bh, qi, want_lse=True, want_pv=True)
    g = got.reshape(B * H, S, D)[bh, qi]
    lg = lse.reshape(B * H, S)[bh, qi]
    check_attn(g, want, pv, lg, lse_o, 1e-4, "sampled")


def test_attention_one_visible_key_and_empty():
    # causal row 0 sees only key 0: O[0] = V[0] exactly; Skv = 0 gives zeros
    q = randn_f16((1, 2, 40, 64), 7)
    k = randn_f16((1, 2, 40, 64), 8)
    v = randn_f16((1, 2, 40, 64), 9)
    got, _ = run_attn(q, k, v, True, 0.125)
    assert np.array_equal(got[:, :, 0], workloads.as_u16(v)[:, :, 0])
    q0 = q.cuda()
    e = torch.empty((1, 2, 0, 64), dtype=torch.float16, device="cuda")
    o, lse = gr.flash_attn_fwd(q0, e, e, return_lse=True)
    torch.cuda.synchronize()
    assert (o == 0).all() and torch.isinf(lse).all() and (lse < 0).all()


def test_attention_deterministic():
    q = randn_f16((2, 4, 700, 128), 21).cuda()
    k = randn_f16((2, 4, 900, 128), 22).cuda()
    v = randn_f16((2, 4, 900, 128), 23).cuda()
    ref = gr.flash_attn_fwd(q, k, v, causal=True)
    for _ in range(20):
        assert torch.equal(gr.flash_attn_fwd(q, k, v, causal=True).view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
def test_attention_scale_sign_and_zero(scale):
    # the kernels take row maxima through the sign of the scale; zero gives
    # uniform weights over the visible keys
    q = randn_f16((1, 2, 150, 64), 31)
    k = randn_f16((1, 2, 170, 64), 32)
    v = randn_f16((1, 2, 170, 64), 33)
    for causal in (False, True):
        got, lse = run_attn(q, k, v, causal, scale)
        want, lse_o, pv = oracle.attention_f16(workloads.as_u16(q), workloads.as_u16(k), workloads.as_u16(v),
                                               scale, causal, want_lse=True, want_pv=True)
        check_attn(got, want, pv, lse, lse_o, score_bound(q, k, scale), f"scale {scale} causal {causal}")


@pytest.mark.parametrize("D", [64, 128])
def test_attention_wide_score_range(D):
    # scores with a standard deviation near 9 (natural units): row maxima jump
    # by more than the lazy-rescaling threshold many times along a row, and
    # most rows are nearly one-hot
    B, H, S = 1, 4, 777
    q = randn_f16((B, H, S, D), 61, scale=3.0)
    k = randn_f16((B, H, S, D), 62, scale=3.0)
    v = randn_f16((B, H, S, D), 63)
    scale = 1.0 / math.sqrt(D)
    for causal in (False, True):
        say(f"[attn] wide range D={D} causal={causal}")
        got, lse = run_attn(q, k, v, causal, scale)
        want, lse_o, pv = oracle.attention_f16(workloads.as_u16(q), workloads.as_u16(k), workloads.as_u16(v),
                                               scale, causal, want_lse=True, want_pv=True)
        check_attn(got, want, pv, lse, lse_o, score_bound(q, k, scale), f"wide D{D} c{causal}")

