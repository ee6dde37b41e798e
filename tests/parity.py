"""Comparison helpers for the GPU parity tests (test code, not product code)."""
from __future__ import annotations

import numpy as np

RTOL = 1e-2
ATOL = 1e-2


def f16_values(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def ulp16(x: np.ndarray) -> np.ndarray:
    """Spacing of fp16 values at |x| (2^-24 in the subnormal range)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -14)))
    return np.exp2(e - 10)


def check(gpu_bits: np.ndarray, ora_bits: np.ndarray, *, absdot: np.ndarray | None = None,
          K: int | None = None, label: str = "") -> dict:
    """Assert |g - o| <= ATOL + RTOL*|o| on every element; return error stats.

    With ``absdot`` (sum_k |a||b| from the oracle) also assert the bound that
    fp32 accumulation implies: |g - o| <= ulp(g)/2 + ulp(o)/2 + 2*K*2^-24*absdot.
    It is much tighter than the contract tolerance on small-valued outputs.
    """
    g = f16_values(gpu_bits)
    o = f16_values(ora_bits)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.isfinite(g).all() or not np.isfinite(o).all(), f"{label}: non-finite GPU output"
    assert (g >= 0).all(), f"{label}: negative output after ReLU"
    err = np.abs(g - o)
    tol = ATOL + RTOL * np.abs(o)
    bad = ~(err <= tol)
    stats = {"n": int(g.size), "max_abs": float(err.max(initial=0.0)),
             "max_rel": float((err / np.maximum(np.abs(o), 1e-30)).max(initial=0.0)),
             "violations": int(bad.sum())}
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(int(v) for v in i)}: gpu {g[tuple(i)]!r} oracle {o[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{label}: {stats['violations']} of {g.size} outside rtol/atol 1e-2; {detail}")
    if absdot is not None:
        bound = 0.5 * ulp16(g) + 0.5 * ulp16(o) + 2.0 * K * 2.0 ** -24 * absdot
        tight_bad = err > bound
        stats["max_ratio_to_fp32_bound"] = float((err / np.maximum(bound, 1e-30)).max(initial=0.0))
        if tight_bad.any():
            i = tuple(np.argwhere(tight_bad)[0])
            raise AssertionError(f"{label}: beyond the fp32-accumulation bound at {i}: gpu {g[i]} "
                                 f"oracle {o[i]} bound {bound[i]}")
    return stats


def check_gelu(gpu_bits: np.ndarray, ora_bits: np.ndarray, *, absdot: np.ndarray, K: int,
               bias_abs: np.ndarray, label: str = "") -> dict:
    """Parity for C = GELU(A @ B + bias): |g - o| <= ATOL + RTOL*|o| on every
    element, and the bound fp32 arithmetic implies -- the accumulation error
    (as for the ReLU path) and the bias addition, scaled by GELU's slope
    (below 1.13 everywhere), plus 64 fp32 ulps for the kernels' GELU (an erfc
    approximation with fractional error below 1.2e-7, evaluated in fp32)."""
    g = f16_values(gpu_bits)
    o = f16_values(ora_bits)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.isfinite(g).all() or not np.isfinite(o).all(), f"{label}: non-finite GPU output"
    assert (g >= -0.1700).all(), f"{label}: value below GELU's minimum"
    err = np.abs(g - o)
    bad = ~(err <= ATOL + RTOL * np.abs(o))
    stats = {"n": int(g.size), "max_abs": float(err.max(initial=0.0)), "violations": int(bad.sum())}
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(int(v) for v in i)}: gpu {g[tuple(i)]!r} oracle {o[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{label}: {stats['violations']} of {g.size} outside rtol/atol 1e-2; {detail}")
    sum_err = 2.0 * K * 2.0 ** -24 * absdot + 2.0 ** -24 * bias_abs
    bound = 0.5 * ulp16(g) + 0.5 * ulp16(o) + 1.13 * sum_err + 64 * 2.0 ** -24 * np.abs(o) + 2.0 ** -30
    tight_bad = err > bound
    stats["max_ratio_to_fp32_bound"] = float((err / bound).max(initial=0.0))
    if tight_bad.any():
        i = tuple(np.argwhere(tight_bad)[0])
        raise AssertionError(f"{label}: beyond the fp32 bound at {i}: gpu {g[i]} oracle {o[i]} bound {bound[i]}")
    return stats
