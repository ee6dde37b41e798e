"""Pins of the row-softmax and attention oracle (CPU only).

The oracle is checked against things fixed independently of its code:
scipy's softmax / logsumexp and numpy products in float64 (library routines
for the textbook definitions), closed forms (a constant row, one visible key,
all-equal scores), invariances (a shift of a softmax row, a joint permutation
of keys and values), and planted mistakes in a copy of its source that these
pins must catch.
"""
from __future__ import annotations

import importlib.util
import math
import os
import shutil

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def f16(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def vals(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def near_tie(y: np.ndarray) -> np.ndarray:
    """True where float64 y lies within 1e-12 (relative) of a midpoint between
    two fp16 values: there either rounding is acceptable."""
    h = y.astype(np.float16).astype(np.float64)
    up = np.nextafter(y.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(y.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    mids = np.stack([(h + up) / 2, (h + dn) / 2])
    return (np.abs(mids - y) <= 1e-12 * np.maximum(np.abs(y), 1e-30)).any(axis=0)


# ---------------------------------------------------------------------------
# row softmax
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,scale", [(1, 1, 1.0), (7, 13, 1.0), (16, 1000, 3.0), (5, 4096, 0.2)])
def test_softmax_matches_scipy(rows, cols, scale):
    rng = np.random.default_rng(rows * 31 + cols)
    X = f16(rng.standard_normal((rows, cols)) * scale)
    Y, yd = oracle.softmax_rows_f16(X, want_double=True)
    ref = softmax(vals(X), axis=1)
    assert np.allclose(yd, ref, rtol=1e-13, atol=1e-300)
    want = ref.astype(np.float16).view(np.uint16)
    ok = (Y == want) | near_tie(ref)
    assert ok.all()
    assert np.allclose(yd.sum(axis=1), 1.0, rtol=1e-13)


def test_softmax_closed_forms():
    # a constant row: every value 1/n; a dominant value: one-hot after rounding
    Y, yd = oracle.softmax_rows_f16(f16(np.full((2, 8), 3.5)), want_double=True)
    assert np.all(yd == 1.0 / 8) and np.all(vals(Y) == 0.125)
    Y = oracle.softmax_rows_f16(f16([[0.0, -60.0, -61.0, -100.0]]))
    assert list(vals(Y)[0]) == [1.0, 0.0, 0.0, 0.0]
    # large values: the maximum must be taken out before the exponentials
    Y, yd = oracle.softmax_rows_f16(f16([[1000.0, 999.0]]), want_double=True)
    e = math.exp(-1.0)
    assert np.allclose(yd[0], [1 / (1 + e), e / (1 + e)], rtol=1e-14)


def test_softmax_shift_invariance():
    rng = np.random.default_rng(3)
    # integer-valued fp16 inputs stay exact after adding an integer
    x = rng.integers(-20, 20, size=(9, 33)).astype(np.float64)
    Y1 = oracle.softmax_rows_f16(f16(x))
    Y2 = oracle.softmax_rows_f16(f16(x + 17.0))
    assert np.array_equal(Y1, Y2)


# ---------------------------------------------------------------------------
# attention forward
# ---------------------------------------------------------------------------

def ref_attention(Q, K, V, scale, causal):
    """float64 reference from scipy's softmax and numpy products."""
    q, k, v = vals(Q), vals(K), vals(V)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        Sq, Skv = s.shape[-2:]
        mask = np.arange(Skv)[None, :] > np.arange(Sq)[:, None]
        s = np.where(mask, -np.inf, s)
    p = softmax(s, axis=-1)
    return np.einsum("bhij,bhjd->bhid", p, v), logsumexp(s, axis=-1)


def ref_pv(Q, K, V, scale, causal):
    """sum_j p_ij |V[j][d]| from scipy's softmax and a numpy product: the
    error scale of a blocked P V product."""
    q, k, v = vals(Q), vals(K), vals(V)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        Sq, Skv = s.shape[-2:]
        s = np.where(np.arange(Skv)[None, :] > np.arange(Sq)[:, None], -np.inf, s)
    return np.einsum("bhij,bhjd->bhid", softmax(s, axis=-1), np.abs(v))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Sq,Skv,D", [(1, 1, 1, 1, 8), (1, 2, 9, 9, 16), (2, 3, 17, 17, 64),
                                          (1, 2, 5, 23, 32), (1, 1, 40, 12, 128)])
def test_attention_matches_numpy(B, H, Sq, Skv, D, causal):
    rng = np.random.default_rng(B * 1000 + H * 100 + Sq + Skv + D + causal)
    Q = f16(rng.standard_normal((B, H, Sq, D)))
    K = f16(rng.standard_normal((B, H, Skv, D)))
    V = f16(rng.standard_normal((B, H, Skv, D)))
    scale = 1.0 / math.sqrt(D)
    O, od, lse, pv = oracle.attention_f16(Q, K, V, scale, causal, want_double=True, want_lse=True, want_pv=True)
    ref, ref_lse = ref_attention(Q, K, V, scale, causal)
    assert np.allclose(od, ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)
    assert np.allclose(pv, ref_pv(Q, K, V, scale, causal), rtol=1e-12, atol=1e-14)
    want = ref.astype(np.float16).view(np.uint16)
    assert ((O == want) | near_tie(ref)).all()


def test_attention_closed_forms():
    rng = np.random.default_rng(7)
    D, S = 16, 11
    V = f16(rng.standard_normal((1, 1, S, D)))
    K = f16(rng.standard_normal((1, 1, S, D)))
    # all-zero queries: equal scores, so O is the mean of the visible values
    Z = f16(np.zeros((1, 1, S, D)))
    _, od = oracle.attention_f16(Z, K, V, 0.25, False, want_double=True)
    assert np.allclose(od[0, 0], np.broadcast_to(vals(V)[0, 0].mean(axis=0), (S, D)), rtol=1e-13, atol=1e-14)
    _, od = oracle.attention_f16(Z, K, V, 0.25, True, want_double=True)
    for i in range(S):
        assert np.allclose(od[0, 0, i], vals(V)[0, 0, :i + 1].mean(axis=0), rtol=1e-13, atol=1e-14)
    # causal, first query: a single visible key, whose value row is returned exactly
    Q = f16(rng.standard_normal((1, 1, S, D)))
    O = oracle.attention_f16(Q, K, V, 0.25, True)
    assert np.array_equal(O[0, 0, 0], V[0, 0, 0])
    # one key far ahead of the rest: O is its value row
    Kd = np.zeros((1, 1, S, D))
    Kd[0, 0, 4, 0] = 100.0
    Qd = np.zeros((1, 1, S, D))
    Qd[..., 0] = 1.0
    O = oracle.attention_f16(f16(Qd), f16(Kd), V, 1.0, False)
    assert np.array_equal(O[0, 0], np.broadcast_to(V[0, 0, 4], (S, D)))


def test_attention_pv_closed_forms():
    # pv = sum_j p_j |V[j]|: with non-negative values it is the output itself,
    # it ignores the signs of V, and for equal scores it is the mean of |V|
    rng = np.random.default_rng(13)
    S, D = 9, 16
    Q = f16(rng.standard_normal((1, 1, S, D)))
    K = f16(rng.standard_normal((1, 1, S, D)))
    V = f16(rng.standard_normal((1, 1, S, D)))
    Vabs = V & np.uint16(0x7FFF)
    for causal in (False, True):
        _, od_abs = oracle.attention_f16(Q, K, Vabs, 0.3, causal, want_double=True)
        _, pv = oracle.attention_f16(Q, K, V, 0.3, causal, want_pv=True)
        _, pv_neg = oracle.attention_f16(Q, K, V ^ np.uint16(0x8000), 0.3, causal, want_pv=True)
        assert np.allclose(pv, od_abs, rtol=1e-14, atol=0)
        assert np.array_equal(pv, pv_neg)
    Z = f16(np.zeros((1, 1, S, D)))
    _, pv = oracle.attention_f16(Z, K, V, 1.0, True, want_pv=True)
    for i in range(S):
        assert np.allclose(pv[0, 0, i], np.abs(vals(V)[0, 0, :i + 1]).mean(axis=0), rtol=1e-13, atol=1e-15)
    # causal row 0 sees one key: pv is |V[0]| exactly
    assert np.array_equal(pv[0, 0, 0], np.abs(vals(V)[0, 0, 0]))


def test_attention_key_permutation_invariance():
    rng = np.random.default_rng(11)
    Q = f16(rng.standard_normal((1, 2, 6, 32)))
    K = f16(rng.standard_normal((1, 2, 19, 32)))
    V = f16(rng.standard_normal((1, 2, 19, 32)))
    perm = rng.permutation(19)
    _, o1 = oracle.attention_f16(Q, K, V, 0.2, False, want_double=True)
    _, o2 = oracle.attention_f16(Q, K[:, :, perm], V[:, :, perm], 0.2, False, want_double=True)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14)


def test_attention_rows_match_full():
    rng = np.random.default_rng(12)
    Q = f16(rng.standard_normal((2, 2, 10, 16)))
    K = f16(rng.standard_normal((2, 2, 10, 16)))
    V = f16(rng.standard_normal((2, 2, 10, 16)))
    full = oracle.attention_f16(Q, K, V, 0.3, True)
    bh = np.array([0, 3, 2, 1, 3])
    qi = np.array([9, 0, 4, 7, 5])
    rows = oracle.attention_rows_f16(Q, K, V, 0.3, True, bh, qi)
    assert np.array_equal(rows, full.reshape(4, 10, 16)[bh, qi])


# ---------------------------------------------------------------------------
# planted mistakes in a copy of the source must be caught by the pins above
# ---------------------------------------------------------------------------

MUTANTS = {
    "softmax_no_max": ("e[j] = exp(oracle_f16_to_f64(x[j]) - m);", "e[j] = exp(oracle_f16_to_f64(x[j]));"),
    "softmax_short_sum": ("        l += e[j];\n                }", "        if (j + 1 < cols) l += e[j];\n                }"),
    "causal_off_by_one": ("const int64_t nkeys = causal ? (i + 1 < Skv ? i + 1 : Skv) : Skv;",
                          "const int64_t nkeys = causal ? (i < Skv ? (i > 0 ? i : 1) : Skv) : Skv;"),
    "no_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "v_transposed": ("const double v = oracle_f16_to_f64(V[j * D + d]);",
                     "const double v = oracle_f16_to_f64(V[(d * nkeys + j) % (nkeys * D)]);"),
    "no_normalisation": ("const double p = s[j] / l;", "const double p = s[j];"),
    "lse_without_log": ("*lse = nkeys > 0 ? m + log(l) : -INFINITY;", "*lse = nkeys > 0 ? m + l : -INFINITY;"),
    "pv_unnormalised": ("a[d] += p * fabs(v);", "a[d] += s[j] * fabs(v);"),
    "pv_no_abs": ("a[d] += p * fabs(v);", "a[d] += p * v;"),
    "pv_short_sum": ("a[d] += p * fabs(v);", "if (j + 1 < nkeys) a[d] += p * fabs(v);"),
    "k_index_of_q": ("oracle_f16_to_f64(K[j * D + d]);", "oracle_f16_to_f64(K[(j * D + d + 1) % (nkeys * D)]);"),
}


def _pin_suite(mod) -> list[str]:
    fails = []
    checks = [
        ("scipy", lambda: test_softmax_matches_scipy(7, 13, 1.0)),
        ("softmax_closed", test_softmax_closed_forms),
        ("attn_numpy", lambda: test_attention_matches_numpy(1, 2, 9, 9, 16, False)),
        ("attn_numpy_causal", lambda: test_attention_matches_numpy(2, 3, 17, 17, 64, True)),
        ("attn_closed", test_attention_closed_forms),
        ("pv_closed", test_attention_pv_closed_forms),
    ]
    global oracle
    saved = oracle
    oracle = mod
    try:
        for name, fn in checks:
            try:
                fn()
            except Exception:  # an assertion or a crash counts as caught
                fails.append(name)
    finally:
        oracle = saved
    return fails


def test_pins_pass_on_real_oracle():
    assert _pin_suite(oracle) == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, tmp_path):
    src_dir = os.path.join(os.path.dirname(HERE), "oracle")
    old, new = MUTANTS[mutant]
    text = open(os.path.join(src_dir, "attention_oracle.c")).read()
    assert text.count(old) == 1, f"mutation anchor for {mutant} not found"
    dst = tmp_path / "oracle_mut"
    dst.mkdir()
    (dst / "attention_oracle.c").write_text(text.replace(old, new, 1))
    shutil.copy(os.path.join(src_dir, "gemm_relu_oracle.c"), dst / "gemm_relu_oracle.c")
    shutil.copy(os.path.join(src_dir, "__init__.py"), dst / "__init__.py")
    spec = importlib.util.spec_from_file_location(f"oracle_amut_{mutant}", dst / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _pin_suite(mod) != [], f"planted mistake {mutant} went unnoticed"
