"""Pins for the CPU oracle (C = ReLU(A @ B), fp16 in/out), all on the CPU.

The oracle is only trusted because these checks tie it to things other than
itself: numpy's independent fp16 conversions, exact rational arithmetic,
closed forms (identity, zero, K = 1), integer sums that are exact in any order,
hand-worked cases under tests/golden/ and invariants of the ReLU. A mutation
test at the end plants plausible mistakes in a copy of the oracle's C source
and checks that every one of them is caught by these pins.
"""
from __future__ import annotations

import math
import os
import re
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# exact helpers (rational arithmetic; independent of the oracle's C code)
# ---------------------------------------------------------------------------

def exact_f16_value(bits: int) -> Fraction:
    """fp16 bit pattern -> exact rational (finite patterns only), via numpy."""
    v = np.array([bits], dtype=np.uint16).view(np.float16)[0]
    assert np.isfinite(v)
    return Fraction(float(v))  # float16 -> float64 is exact


def exact_rne_f16(y: Fraction) -> int:
    """Round a non-negative rational to fp16 bits, nearest, ties to even."""
    assert y >= 0
    if y == 0:
        return 0
    if y >= 65520:
        return 0x7C00
    if y < Fraction(1, 2 ** 14):
        q = Fraction(1, 2 ** 24)
        e = None
    else:
        e = math.floor(math.log2(y))
        # correct floor(log2) exactly for rationals near powers of two
        while Fraction(2) ** e > y:
            e -= 1
        while Fraction(2) ** (e + 1) <= y:
            e += 1
        q = Fraction(2) ** (e - 10)
    n = y / q
    fl = n.numerator // n.denominator
    r = n - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if e is None:
        return int(fl)  # subnormal pattern (1024 is the smallest normal's pattern)
    if fl == 2048:
        fl, e = 1024, e + 1
    if e + 15 >= 31:
        return 0x7C00
    return ((e + 15) << 10) | (fl - 1024)


def exact_gemm_relu(A_bits: np.ndarray, B_bits: np.ndarray) -> tuple[np.ndarray, list]:
    """Exact rational ReLU(A @ B), then exact RNE to fp16."""
    M, K = A_bits.shape
    _, N = B_bits.shape
    Af = [[exact_f16_value(int(A_bits[i, k])) for k in range(K)] for i in range(M)]
    Bf = [[exact_f16_value(int(B_bits[k, j])) for j in range(N)] for k in range(K)]
    out = np.zeros((M, N), dtype=np.uint16)
    sums = []
    for i in range(M):
        row = []
        for j in range(N):
            s = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
            row.append(s)
            out[i, j] = exact_rne_f16(max(s, Fraction(0)))
        sums.append(row)
    return out, sums


def rand_f16_bits(rng: np.random.Generator, shape, scale=1.0) -> np.ndarray:
    x = (rng.standard_normal(shape) * scale).astype(np.float16)
    return x.view(np.uint16)


def f16_bits(values) -> np.ndarray:
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# 1. fp16 decode, exhaustive against numpy
# ---------------------------------------------------------------------------

def test_decode_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # sign of zero is kept
    assert math.copysign(1.0, ours[0x8000]) == -1.0


# ---------------------------------------------------------------------------
# 2. fp16 encode (round to nearest, ties to even)
# ---------------------------------------------------------------------------

def test_encode_round_trips_every_finite_value():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    finite = np.isfinite(vals)
    back = oracle.f64_to_f16(vals[finite].astype(np.float64))
    assert np.array_equal(back, bits[finite])


def test_encode_midpoints_go_to_even_neighbour():
    # all adjacent pairs of finite non-negative fp16 values, 0x0000 .. 0x7bff
    lo = np.arange(0, 0x7BFF, dtype=np.uint16)
    hi = lo + 1
    lo_v = lo.view(np.float16).astype(np.float64)
    hi_v = hi.view(np.float16).astype(np.float64)
    mid = (lo_v + hi_v) / 2  # exact in double
    got = oracle.f64_to_f16(mid)
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, even)
    # a hair either side goes to the nearer neighbour
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    assert np.array_equal(oracle.f64_to_f16(below), lo)
    assert np.array_equal(oracle.f64_to_f16(above), hi)
    # negative side mirrors
    assert np.array_equal(oracle.f64_to_f16(-mid), even | 0x8000)


def test_encode_thresholds():
    enc = lambda x: int(oracle.f64_to_f16(np.array([x]))[0])
    assert enc(65519.99) == 0x7BFF
    assert enc(65520.0) == 0x7C00
    assert enc(-65520.0) == 0xFC00
    assert enc(1e300) == 0x7C00
    assert enc(2.0 ** -25) == 0x0000
    assert enc(2.0 ** -25 * (1 + 2.0 ** -40)) == 0x0001
    assert enc(1 + 2.0 ** -11) == 0x3C00
    assert enc(1 + 3 * 2.0 ** -11) == 0x3C02
    assert enc(float("inf")) == 0x7C00
    assert enc(float("nan")) & 0x7C00 == 0x7C00 and enc(float("nan")) & 0x3FF


def test_encode_random_doubles_match_numpy():
    rng = np.random.default_rng(1234)
    exps = rng.integers(-30, 18, size=1_000_000)
    x = rng.uniform(1.0, 2.0, size=exps.size) * np.exp2(exps.astype(np.float64))
    x *= np.where(rng.random(x.size) < 0.5, -1.0, 1.0)
    ours = oracle.f64_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_exact_rne_helper_matches_numpy():
    # the rational rounding used by the brute-force pins agrees with numpy
    rng = np.random.default_rng(7)
    exps = rng.integers(-28, 17, size=3000)
    x = rng.uniform(1.0, 2.0, size=exps.size) * np.exp2(exps.astype(np.float64))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([exact_rne_f16(Fraction(float(v))) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# 3. hand-worked fixtures (tests/golden/hand_cases.txt)
# ---------------------------------------------------------------------------

def _parse_value(tok: str) -> float:
    m = re.fullmatch(r"(?:(\-?\d+)\*)?2\^(-?\d+)", tok)
    if m:
        mult = int(m.group(1)) if m.group(1) else 1
        return mult * 2.0 ** int(m.group(2))
    return float(tok)


def load_hand_cases():
    cases = []
    with open(os.path.join(HERE, "golden", "hand_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, dims, a, b, c = [p.strip() for p in line.split("|")]
            M, N, K = (int(t) for t in dims.split())
            A = f16_bits([_parse_value(t) for t in a.split()]).reshape(M, K)
            B = f16_bits([_parse_value(t) for t in b.split()]).reshape(K, N)
            # the fixture inputs must be exact fp16 values
            assert np.array_equal(A.view(np.float16).astype(np.float64).ravel(),
                                  np.array([_parse_value(t) for t in a.split()]))
            assert np.array_equal(B.view(np.float16).astype(np.float64).ravel(),
                                  np.array([_parse_value(t) for t in b.split()]))
            C = np.array([int(t, 16) for t in c.split()], dtype=np.uint16).reshape(M, N)
            cases.append((name, A, B, C))
    return cases


HAND = load_hand_cases()


@pytest.mark.parametrize("name,A,B,C", HAND, ids=[c[0] for c in HAND])
def test_hand_worked_cases(name, A, B, C):
    assert np.array_equal(oracle.gemm_relu_f16(A, B), C)
    ii, jj = np.nonzero(np.ones_like(C))
    assert np.array_equal(oracle.gemm_relu_f16_points(A, B, ii, jj), C.ravel())


# ---------------------------------------------------------------------------
# 4. exact brute force on tiny shapes
# ---------------------------------------------------------------------------

SIZES = [1, 2, 3, 5, 7, 16, 17]  # shapes for the exact rational brute force


@pytest.mark.parametrize("M,N,K", [(m, n, k) for m in SIZES for n in (1, 3, 17) for k in (1, 2, 5, 16, 17)][::2])
def test_brute_force_exact(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 100 + K)
    A = rand_f16_bits(rng, (M, K))
    B = rand_f16_bits(rng, (K, N))
    want, sums = exact_gemm_relu(A, B)
    got, pre, absdot = oracle.gemm_relu_f16(A, B, want_pre=True, want_absdot=True)
    for i in range(M):
        for j in range(N):
            exact = sums[i][j]
            # the double sum is within K * 2^-53 * sum|a||b| of the exact sum
            assert abs(Fraction(pre[i, j]) - exact) <= Fraction(K) * Fraction(1, 2 ** 53) * Fraction(absdot[i, j])
            if got[i, j] != want[i, j]:
                # allowed only if a rounding boundary lies within that bound
                bound = Fraction(K) * Fraction(1, 2 ** 53) * Fraction(absdot[i, j])
                lo = exact_rne_f16(max(exact - bound, Fraction(0)))
                hi = exact_rne_f16(max(exact + bound, Fraction(0)))
                if lo == hi:
                    pytest.fail(f"({i},{j}): oracle {got[i, j]:#06x} exact {want[i, j]:#06x}")
    # the points routine gives the same bits
    ii, jj = np.divmod(np.arange(M * N), N)
    assert np.array_equal(oracle.gemm_relu_f16_points(A, B, ii, jj), want.ravel())


def test_brute_force_with_subnormal_inputs():
    rng = np.random.default_rng(99)
    A = rand_f16_bits(rng, (5, 9), scale=2.0 ** -13)   # many fp16 subnormals
    B = rand_f16_bits(rng, (9, 4), scale=64.0)
    assert np.mean((A & 0x7C00) == 0) > 0.2
    want, _ = exact_gemm_relu(A, B)
    assert np.array_equal(oracle.gemm_relu_f16(A, B), want)


# ---------------------------------------------------------------------------
# 5. closed forms
# ---------------------------------------------------------------------------

def relu_bits(X: np.ndarray) -> np.ndarray:
    """ReLU of fp16 values given as bits: negatives and -0 become +0."""
    v = X.view(np.float16)
    return np.where(v > 0, X, np.uint16(0)).astype(np.uint16)


@pytest.mark.parametrize("K,N", [(1, 1), (8, 5), (33, 70)])
def test_identity_left(K, N):
    rng = np.random.default_rng(K + N)
    B = rand_f16_bits(rng, (K, N), scale=3.0)
    I = f16_bits(np.eye(K))
    assert np.array_equal(oracle.gemm_relu_f16(I, B), relu_bits(B))


@pytest.mark.parametrize("M,K", [(1, 1), (6, 8), (45, 31)])
def test_identity_right(M, K):
    rng = np.random.default_rng(M * K)
    A = rand_f16_bits(rng, (M, K), scale=3.0)
    I = f16_bits(np.eye(K))
    assert np.array_equal(oracle.gemm_relu_f16(A, I), relu_bits(A))


def test_zero_operands_and_empty_k():
    rng = np.random.default_rng(3)
    A = rand_f16_bits(rng, (9, 13))
    B = rand_f16_bits(rng, (13, 6))
    assert not oracle.gemm_relu_f16(np.zeros_like(A), B).any()
    assert not oracle.gemm_relu_f16(A, np.zeros_like(B)).any()
    # K = 0: the empty sum is 0
    out = oracle.gemm_relu_f16(np.zeros((4, 0), np.uint16), np.zeros((0, 5), np.uint16))
    assert out.shape == (4, 5) and not out.any()
    # M = 0 or N = 0: nothing to compute
    assert oracle.gemm_relu_f16(np.zeros((0, 3), np.uint16), B[:3]).shape == (0, 6)
    assert oracle.gemm_relu_f16(A[:, :2], np.zeros((2, 0), np.uint16)).shape == (9, 0)


def test_k1_outer_product():
    rng = np.random.default_rng(5)
    a = rand_f16_bits(rng, (40, 1), scale=8.0)
    b = rand_f16_bits(rng, (1, 50), scale=8.0)
    av = a.view(np.float16).astype(np.float64)
    bv = b.view(np.float16).astype(np.float64)
    prod = av @ bv  # each entry is one exact product
    want = np.maximum(prod, 0).astype(np.float16).view(np.uint16)
    want = np.where(prod > 0, want, np.uint16(0))
    assert np.array_equal(oracle.gemm_relu_f16(a, b), want)


# ---------------------------------------------------------------------------
# 6. integer-exact sums (order independent), against integer matmul
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(33, 47, 129), (64, 64, 4096), (5, 130, 1000)])
def test_integer_inputs_exact(M, N, K):
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=11)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    ai = a.numpy().astype(np.int64)
    bi = b.numpy().astype(np.int64)
    s = ai @ bi
    want = np.maximum(s, 0).astype(np.float64).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.gemm_relu_f16(A, B), want)


# ---------------------------------------------------------------------------
# 7. invariants
# ---------------------------------------------------------------------------

def test_nonnegative_and_sign_pairing():
    rng = np.random.default_rng(21)
    A = rand_f16_bits(rng, (37, 53))
    B = rand_f16_bits(rng, (53, 29))
    C = oracle.gemm_relu_f16(A, B).view(np.float16)
    Cn = oracle.gemm_relu_f16(A ^ np.uint16(0x8000), B).view(np.float16)
    assert not np.isnan(C).any() and (C >= 0).all()
    assert not ((C > 0) & (Cn > 0)).any()
    # exactly one of the pair is positive wherever the pre-activation is nonzero
    _, pre = oracle.gemm_relu_f16(A, B, want_pre=True)
    nz = pre != 0
    assert ((C > 0) | (Cn > 0))[nz].all()


def test_power_of_two_scaling():
    rng = np.random.default_rng(22)
    A = rand_f16_bits(rng, (20, 40))
    B = rand_f16_bits(rng, (40, 30))
    A2 = (A.view(np.float16).astype(np.float64) * 2).astype(np.float16).view(np.uint16)
    C = oracle.gemm_relu_f16(A, B).view(np.float16).astype(np.float64)
    C2 = oracle.gemm_relu_f16(A2, B).view(np.float16).astype(np.float64)
    normal = C >= 2.0 ** -14  # away from subnormal rounding; overflow unreachable here
    assert np.array_equal(C2[normal], 2 * C[normal])


def test_rows_and_points_agree_with_full():
    w = workloads.RAGGED
    a, b = workloads.make_inputs(96, 72, 200, w.dist, w.scale, seed=3)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    full = oracle.gemm_relu_f16(A, B)
    assert np.array_equal(oracle.gemm_relu_f16(A, B, rows=(17, 60)), full[17:60])
    rng = np.random.default_rng(0)
    ii = rng.integers(0, 96, 500)
    jj = rng.integers(0, 72, 500)
    assert np.array_equal(oracle.gemm_relu_f16_points(A, B, ii, jj), full[ii, jj])


def test_cross_check_numpy_float64_matmul():
    a, b = workloads.make_inputs(64, 64, 64, "normal", 1.0, seed=0)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    av = a.numpy().astype(np.float64)
    bv = b.numpy().astype(np.float64)
    ref = np.maximum(av @ bv, 0).astype(np.float16).view(np.uint16)
    got = oracle.gemm_relu_f16(A, B)
    diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    # a different fp64 summation order may only flip a near-tie by one ulp
    assert diff.max() <= 1
    assert (diff != 0).sum() <= 2


def test_thread_count_independence():
    a, b = workloads.make_inputs(48, 40, 300, "normal", 1.0, seed=8)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    ref = oracle.gemm_relu_f16(A, B)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    code = ("import sys, numpy as np; sys.path.insert(0, %r); import oracle, workloads;"
            "a,b=workloads.make_inputs(48,40,300,'normal',1.0,seed=8);"
            "np.save(sys.argv[1], oracle.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b)))"
            % os.path.dirname(HERE))
    out = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"oracle1t_{os.getpid()}.npy")
    subprocess.run(["python", "-c", code, out], check=True, env=env)
    try:
        assert np.array_equal(np.load(out), ref)
    finally:
        os.remove(out)


# ---------------------------------------------------------------------------
# 8. mutation check: planted mistakes in a copy of the oracle are caught
# ---------------------------------------------------------------------------

MUTANTS = {
    "drop_last_k_term": ("acc[j] += a * brow[j];", "if (k + 1 < K) acc[j] += a * brow[j];"),
    "transposed_b": ("const double* brow = bd + k * N;", "const double* brow = bd + (k % (N > 0 ? N : 1)) * N;"),
    "wrong_a_index": ("return op_a ? A[k * M + i] : A[i * K + k];",
                      "return op_a ? A[k * M + i] : A[(k * M + i) % (M * K)];"),
    "no_relu": ("return oracle_f64_to_f16_rne(pre > 0.0 ? pre : 0.0);", "return oracle_f64_to_f16_rne(pre);"),
    "relu_as_abs": ("return oracle_f64_to_f16_rne(pre > 0.0 ? pre : 0.0);", "return oracle_f64_to_f16_rne(fabs(pre));"),
    "ties_away": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "truncate": ("if (r > 0.5) return fl + 1.0;", "if (r > 2.0) return fl + 1.0;"),
    "subnormal_scale": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "exponent_bias": ("v = ldexp((double)(1024 + m), e - 25);", "v = ldexp((double)(1024 + m), e - 24);"),
    "overflow_threshold": ("if (a >= 65520.0) return sign | 0x7c00;", "if (a > 65504.0) return sign | 0x7c00;"),
    "sign_flip_b": ("acc[j] += a * brow[j];", "acc[j] += a * (j == 0 ? -brow[j] : brow[j]);"),
}


def _pin_suite(lib_mod) -> list[str]:
    """Run a compact set of the pins above against an oracle module; return failures."""
    fails = []
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    ref = vals.astype(np.float64)
    fin = np.isfinite(vals)
    if not np.array_equal(lib_mod.f16_to_f64(bits)[fin], ref[fin]):
        fails.append("decode")
    if not np.array_equal(lib_mod.f64_to_f16(ref[fin]), bits[fin]):
        fails.append("roundtrip")
    lo = np.arange(0, 0x7BFF, dtype=np.uint16)
    mid = (lo.view(np.float16).astype(np.float64) + (lo + 1).view(np.float16).astype(np.float64)) / 2
    if not np.array_equal(lib_mod.f64_to_f16(mid), np.where(lo % 2 == 0, lo, lo + 1)):
        fails.append("midpoints")
    if int(lib_mod.f64_to_f16(np.array([65519.99]))[0]) != 0x7BFF:
        fails.append("threshold")
    for name, A, B, C in HAND:
        if not np.array_equal(lib_mod.gemm_relu_f16(A, B), C):
            fails.append("hand:" + name)
    rng = np.random.default_rng(0)
    A = rand_f16_bits(rng, (7, 5))
    B = rand_f16_bits(rng, (5, 6))
    if not np.array_equal(lib_mod.gemm_relu_f16(A, B), exact_gemm_relu(A, B)[0]):
        fails.append("brute")
    a, b = workloads.make_inputs(9, 11, 13, dist="intsmall", seed=4)
    s = a.numpy().astype(np.int64) @ b.numpy().astype(np.int64)
    want = np.maximum(s, 0).astype(np.float16).view(np.uint16)
    if not np.array_equal(lib_mod.gemm_relu_f16(workloads.as_u16(a), workloads.as_u16(b)), want):
        fails.append("integer")
    return fails


def test_pins_pass_on_real_oracle():
    assert _pin_suite(oracle) == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, tmp_path):
    import importlib.util
    src_dir = os.path.join(os.path.dirname(HERE), "oracle")
    old, new = MUTANTS[mutant]
    text = open(os.path.join(src_dir, "gemm_relu_oracle.c")).read()
    assert text.count(old) >= 1, f"mutation anchor for {mutant} not found"
    dst = tmp_path / "oracle_mut"
    dst.mkdir()
    (dst / "gemm_relu_oracle.c").write_text(text.replace(old, new, 1))
    shutil.copy(os.path.join(src_dir, "__init__.py"), dst / "__init__.py")
    shutil.copy(os.path.join(src_dir, "attention_oracle.c"), dst / "attention_oracle.c")
    spec = importlib.util.spec_from_file_location(f"oracle_mut_{mutant}", dst / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _pin_suite(mod) != [], f"planted mistake {mutant} went unnoticed"


# ---------------------------------------------------------------------------
# 9. the fused bias + GELU epilogue (C = GELU(A @ B + bias))
# ---------------------------------------------------------------------------

def exact_rne_f16_signed(y: Fraction) -> int:
    return (0x8000 | exact_rne_f16(-y)) if y < 0 else exact_rne_f16(y)


def mp_gelu(x: Fraction) -> Fraction:
    """GELU of an exact rational, evaluated with 80-digit arithmetic and
    returned as the exact binary value of that result."""
    import mpmath
    with mpmath.workdps(80):
        xm = mpmath.mpf(x.numerator) / x.denominator
        g = xm * mpmath.ncdf(xm)
        man, exp = int(g.man), int(g.exp)
        sign = -1 if g < 0 else 1
        v = Fraction(abs(man)) * (Fraction(2) ** exp)
        return sign * v if g != 0 else Fraction(0)


def test_gelu_textbook_values():
    # standard normal distribution function at 1, 2, 3, -1 (normal tables, 15 digits)
    for x, phi in ((1.0, 0.841344746068543), (2.0, 0.977249868051821), (3.0, 0.998650101968370),
                   (-1.0, 0.158655253931457), (0.5, 0.691462461274013)):
        assert abs(float(oracle.gelu(x)) - x * phi) <= 2e-15 * abs(x)
    assert float(oracle.gelu(0.0)) == 0.0
    assert float(oracle.gelu(12.0)) == 12.0          # Phi(12) rounds to 1 in double
    assert float(oracle.gelu(-40.0)) == 0.0          # Phi(-40) underflows


def test_gelu_against_library_normal_cdf():
    from scipy.special import ndtr
    x = np.linspace(-9.0, 9.0, 3601)
    g = oracle.gelu(x)
    ref = x * ndtr(x)
    nz = np.abs(ref) > 1e-300
    assert np.max(np.abs(g[nz] - ref[nz]) / np.abs(ref[nz])) < 1e-13


def test_gelu_odd_part_is_identity():
    # x * Phi(x) - (-x) * Phi(-x) = x * (Phi(x) + Phi(-x)) = x
    x = np.random.default_rng(3).uniform(-8.0, 8.0, 5000)
    d = oracle.gelu(x) - oracle.gelu(-x)
    assert np.max(np.abs(d - x) / np.maximum(np.abs(x), 1e-300)) < 4e-16 * 8


def _bias_gelu_exact(A, B, bias):
    M, K = A.shape
    _, N = B.shape
    Af = [[exact_f16_value(int(A[i, k])) for k in range(K)] for i in range(M)]
    Bf = [[exact_f16_value(int(B[k, j])) for j in range(N)] for k in range(K)]
    bf = [exact_f16_value(int(bias[j])) for j in range(N)]
    out = np.zeros((M, N), dtype=np.uint16)
    pres = []
    for i in range(M):
        row = []
        for j in range(N):
            s = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) + bf[j]
            row.append(s)
            out[i, j] = exact_rne_f16_signed(mp_gelu(s))
        pres.append(row)
    return out, pres


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 2), (7, 3, 5), (5, 17, 16), (16, 4, 17), (2, 9, 0)])
def test_bias_gelu_brute_force_exact(M, N, K):
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    A = rand_f16_bits(rng, (M, K))
    B = rand_f16_bits(rng, (K, N))
    bias = rand_f16_bits(rng, (N,))
    want, pres = _bias_gelu_exact(A, B, bias)
    got, pre, absdot = oracle.gemm_bias_gelu_f16(A, B, bias, want_pre=True, want_absdot=True)
    for i in range(M):
        for j in range(N):
            if got[i, j] == want[i, j]:
                continue
            # a flip is allowed only if an fp16 rounding boundary lies within the
            # oracle's double-precision error: the sum's bound, scaled by
            # GELU's slope (< 1.13), plus a few ulps of the double GELU
            exact = pres[i][j]
            bound = (Fraction(K + 1) * Fraction(1, 2 ** 53) * (Fraction(absdot[i, j]) + abs(exact)) * Fraction(113, 100)
                     + Fraction(8, 2 ** 53) * abs(mp_gelu(exact)) + Fraction(1, 2 ** 1000))
            g = mp_gelu(exact)
            if exact_rne_f16_signed(g - bound) == exact_rne_f16_signed(g + bound):
                pytest.fail(f"({i},{j}): oracle {got[i, j]:#06x} exact {want[i, j]:#06x}")
    ii, jj = np.divmod(np.arange(M * N), N)
    assert np.array_equal(oracle.gemm_bias_gelu_f16_points(A, B, bias, ii, jj), got.ravel())


def test_bias_is_per_column():
    # K = 0: every row of C is GELU(bias); A = I: C = GELU(B + bias) elementwise
    bias = f16_bits([-3.0, -0.5, 0.0, 0.25, 1.0, 2.5, 7.0])
    N = bias.size
    A0 = np.zeros((4, 0), dtype=np.uint16)
    B0 = np.zeros((0, N), dtype=np.uint16)
    C = oracle.gemm_bias_gelu_f16(A0, B0, bias)
    row = np.array([exact_rne_f16_signed(mp_gelu(exact_f16_value(int(b)))) for b in bias], dtype=np.uint16)
    assert np.array_equal(C, np.tile(row, (4, 1)))
    rng = np.random.default_rng(12)
    K = 5
    I = f16_bits(np.eye(K))
    B = rand_f16_bits(rng, (K, N))
    C = oracle.gemm_bias_gelu_f16(I, B, bias)
    want = np.array([[exact_rne_f16_signed(mp_gelu(exact_f16_value(int(B[i, j])) + exact_f16_value(int(bias[j]))))
                      for j in range(N)] for i in range(K)], dtype=np.uint16)
    assert np.array_equal(C, want)


def test_bias_gelu_zero_bias_and_sign_structure():
    # with bias 0, GELU(s) - GELU(-s) = s links C(A) and C(-A) to the plain sum
    a, b = workloads.make_inputs(6, 9, 40, dist="intsmall", seed=21)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    An = workloads.as_u16((-a).contiguous())
    z = np.zeros(9, dtype=np.uint16)
    gp, pre = oracle.gemm_bias_gelu_f16(A, B, z, want_pre=True)
    gn = oracle.gemm_bias_gelu_f16(An, B, z)
    s = a.numpy().astype(np.int64) @ b.numpy().astype(np.int64)
    assert np.array_equal(pre, s.astype(np.float64))
    vp = gp.view(np.float16).astype(np.float64)
    vn = gn.view(np.float16).astype(np.float64)
    # each fp16 result is within half an ulp of its value, so the identity holds to two half-ulps
    ulp = lambda v: np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -14))) - 10)
    assert np.all(np.abs((vp - vn) - s) <= 0.5 * ulp(vp) + 0.5 * ulp(vn) + 0.5 * ulp(s.astype(np.float64)))


BIAS_MUTANTS = {
    "bias_sign": ("const double pre = acc + oracle_f16_to_f64(bias[j]);",
                  "const double pre = acc - oracle_f16_to_f64(bias[j]);"),
    "bias_dropped": ("const double pre = acc + oracle_f16_to_f64(bias[j]);", "const double pre = acc;"),
    "bias_by_row": ("C[i * N + j] = finish(acc[j], bias, j,", "C[i * N + j] = finish(acc[j], bias, i % (N > 0 ? N : 1),"),
    "gelu_tanh_form": ("return x * (0.5 * erfc(-x / sqrt(2.0)));",
                       "return 0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)));"),
    "gelu_as_relu": ("return oracle_f64_to_f16_rne(oracle_gelu(pre));",
                     "return oracle_f64_to_f16_rne(pre > 0.0 ? pre : 0.0);"),
    "gelu_before_bias": ("const double pre = acc + oracle_f16_to_f64(bias[j]);",
                         "const double pre = oracle_gelu(acc) + oracle_f16_to_f64(bias[j]) - oracle_gelu(0.0) * 0.0;"),
}


def _bias_pin_suite(mod) -> list[str]:
    fails = []
    for x, phi in ((1.0, 0.841344746068543), (2.0, 0.977249868051821), (-1.0, 0.158655253931457)):
        if abs(float(mod.gelu(x)) - x * phi) > 2e-15 * abs(x):
            fails.append("textbook")
    for shape in ((3, 5, 2), (5, 17, 16), (2, 9, 0)):
        M, N, K = shape
        rng = np.random.default_rng(M * 7919 + N * 31 + K)
        A = rand_f16_bits(rng, (M, K))
        B = rand_f16_bits(rng, (K, N))
        bias = rand_f16_bits(rng, (N,))
        want, _ = _bias_gelu_exact(A, B, bias)
        if not np.array_equal(mod.gemm_bias_gelu_f16(A, B, bias), want):
            fails.append(f"brute{shape}")
    return fails


def test_bias_pins_pass_on_real_oracle():
    assert _bias_pin_suite(oracle) == []


@pytest.mark.parametrize("mutant", sorted(BIAS_MUTANTS))
def test_planted_bias_gelu_mistake_is_caught(mutant, tmp_path):
    import importlib.util
    src_dir = os.path.join(os.path.dirname(HERE), "oracle")
    old, new = BIAS_MUTANTS[mutant]
    text = open(os.path.join(src_dir, "gemm_relu_oracle.c")).read()
    assert text.count(old) >= 1, f"mutation anchor for {mutant} not found"
    dst = tmp_path / "oracle_mut"
    dst.mkdir()
    (dst / "gemm_relu_oracle.c").write_text(text.replace(old, new, 1))
    shutil.copy(os.path.join(src_dir, "__init__.py"), dst / "__init__.py")
    shutil.copy(os.path.join(src_dir, "attention_oracle.c"), dst / "attention_oracle.c")
    spec = importlib.util.spec_from_file_location(f"oracle_bmut_{mutant}", dst / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _bias_pin_suite(mod) != [], f"planted mistake {mutant} went unnoticed"


# ---------------------------------------------------------------------------
# 10. transposed operands: C = epilogue(op(A) @ op(B)), op = as stored or the
#     transpose of the stored matrix (the transpose_A / transpose_B flags of
#     the tile-level product in "Escribamos un GEMM")
# ---------------------------------------------------------------------------

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _stored(logical: np.ndarray, trans: bool) -> np.ndarray:
    """How a logical operand is laid out in memory under a transpose flag."""
    return np.ascontiguousarray(logical.T) if trans else logical


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (7, 2, 16), (5, 17, 3), (16, 3, 17)])
def test_transposed_brute_force_exact(ta, tb, M, N, K):
    # the exact rational sums of the logical product, with the stored layout
    # made by numpy's transpose: a wrong index in the oracle's transposed
    # reads shows up as a different value
    rng = np.random.default_rng(M * 1009 + N * 101 + K + 7 * ta + 13 * tb)
    A = rand_f16_bits(rng, (M, K))
    B = rand_f16_bits(rng, (K, N))
    want, sums = exact_gemm_relu(A, B)
    As, Bs = _stored(A, ta), _stored(B, tb)
    got, pre, absdot = oracle.gemm_relu_f16(As, Bs, want_pre=True, want_absdot=True, trans_a=ta, trans_b=tb)
    assert got.shape == (M, N)
    for i in range(M):
        for j in range(N):
            bound = Fraction(K) * Fraction(1, 2 ** 53) * Fraction(absdot[i, j])
            assert abs(Fraction(pre[i, j]) - sums[i][j]) <= bound
            if got[i, j] != want[i, j]:
                lo = exact_rne_f16(max(sums[i][j] - bound, Fraction(0)))
                hi = exact_rne_f16(max(sums[i][j] + bound, Fraction(0)))
                assert lo != hi, f"({i},{j}) layout {ta},{tb}"
    ii, jj = np.divmod(np.arange(M * N), N)
    pts = oracle.gemm_relu_f16_points(As, Bs, ii, jj, trans_a=ta, trans_b=tb)
    assert np.array_equal(pts, got.ravel())


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_transposed_integer_exact(ta, tb):
    # integer-valued inputs: every double sum is exact, so the result is the
    # int64 matrix product of the logical operands, bit for bit
    M, N, K = 19, 23, 40
    a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=5)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    s = a.numpy().astype(np.int64) @ b.numpy().astype(np.int64)
    want = np.maximum(s, 0).astype(np.float16).view(np.uint16)
    got = oracle.gemm_relu_f16(_stored(A, ta), _stored(B, tb), trans_a=ta, trans_b=tb)
    assert np.array_equal(got, want)
    # rows and points of the bias + GELU form read the operands the same way
    bias = f16_bits(np.linspace(-3, 3, N))
    full = oracle.gemm_bias_gelu_f16(A, B, bias)
    part = oracle.gemm_bias_gelu_f16(_stored(A, ta), _stored(B, tb), bias, rows=(4, 11), trans_a=ta, trans_b=tb)
    assert np.array_equal(part, full[4:11])
    ii = np.array([0, 18, 7, 3]); jj = np.array([22, 0, 11, 5])
    pts = oracle.gemm_bias_gelu_f16_points(_stored(A, ta), _stored(B, tb), bias, ii, jj, trans_a=ta, trans_b=tb)
    assert np.array_equal(pts, full[ii, jj])


def test_transposed_shapes_checked():
    A = np.zeros((4, 3), dtype=np.uint16)   # stored K x M with trans_a: M = 3, K = 4
    B = np.zeros((5, 4), dtype=np.uint16)   # stored N x K with trans_b: N = 5
    assert oracle.gemm_relu_f16(A, B, trans_a=True, trans_b=True).shape == (3, 5)
    with pytest.raises(ValueError):
        oracle.gemm_relu_f16(A, B, trans_a=True)   # op(B) would be 5 x 4: K differs


TRANS_MUTANTS = {
    "at_read_as_stored": ("return op_a ? A[k * M + i] : A[i * K + k];", "return op_a ? A[i * K + k] : A[i * K + k];"),
    "at_wrong_stride": ("return op_a ? A[k * M + i] : A[i * K + k];", "return op_a ? A[(k * K + i) % (M * K)] : A[i * K + k];"),
    "bt_read_as_stored": ("return op_b ? B[j * K + k] : B[k * N + j];", "return op_b ? B[k * N + j] : B[k * N + j];"),
    "bt_wrong_stride": ("return op_b ? B[j * K + k] : B[k * N + j];", "return op_b ? B[(j * N + k) % (N * K)] : B[k * N + j];"),
}


def _trans_pin_suite(mod) -> list[str]:
    fails = []
    for ta, tb in LAYOUTS:
        for M, N, K in ((3, 5, 7), (6, 4, 9)):
            a, b = workloads.make_inputs(M, N, K, dist="intsmall", seed=M + N + K + 2 * ta + tb)
            A, B = workloads.as_u16(a), workloads.as_u16(b)
            s = a.numpy().astype(np.int64) @ b.numpy().astype(np.int64)
            want = np.maximum(s, 0).astype(np.float16).view(np.uint16)
            try:
                got = mod.gemm_relu_f16(_stored(A, ta), _stored(B, tb), trans_a=ta, trans_b=tb)
            except Exception as e:  # a crash counts as caught
                fails.append(f"{ta}{tb}:{e}")
                continue
            if not np.array_equal(got, want):
                fails.append(f"{ta}{tb}{(M, N, K)}")
    return fails


def test_transposed_pins_pass_on_real_oracle():
    assert _trans_pin_suite(oracle) == []


@pytest.mark.parametrize("mutant", sorted(TRANS_MUTANTS))
def test_planted_transpose_mistake_is_caught(mutant, tmp_path):
    import importlib.util
    src_dir = os.path.join(os.path.dirname(HERE), "oracle")
    old, new = TRANS_MUTANTS[mutant]
    text = open(os.path.join(src_dir, "gemm_relu_oracle.c")).read()
    assert text.count(old) == 1, f"mutation anchor for {mutant} not found"
    dst = tmp_path / "oracle_mut"
    dst.mkdir()
    (dst / "gemm_relu_oracle.c").write_text(text.replace(old, new, 1))
    shutil.copy(os.path.join(src_dir, "__init__.py"), dst / "__init__.py")
    shutil.copy(os.path.join(src_dir, "attention_oracle.c"), dst / "attention_oracle.c")
    spec = importlib.util.spec_from_file_location(f"oracle_tmut_{mutant}", dst / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _trans_pin_suite(mod) != [], f"planted mistake {mutant} went unnoticed"



# ---------------------------------------------------------------------------
# 11. the error-scale output: absdot[i][j] = sum_k |A[i][k]| |B[k][j]|
# ---------------------------------------------------------------------------
# The GPU parity tests bound each output's fp32 accumulation error by
# K 2^-24 absdot, so absdot must be the true sum of absolute products: a
# value too large would loosen that bound without any test noticing. These
# pins tie it to exact rational sums, to integer products, and to the
# oracle's own signed sum of |A| and |B| (a separate code path).

def exact_absdot(A_bits: np.ndarray, B_bits: np.ndarray) -> list:
    M, K = A_bits.shape
    _, N = B_bits.shape
    Af = [[abs(exact_f16_value(int(A_bits[i, k]))) for k in range(K)] for i in range(M)]
    Bf = [[abs(exact_f16_value(int(B_bits[k, j]))) for j in range(N)] for k in range(K)]
    return [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]


def abs_bits(X: np.ndarray) -> np.ndarray:
    return X & np.uint16(0x7FFF)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (5, 1, 16), (3, 17, 7), (7, 3, 17), (16, 5, 2)])
def test_absdot_matches_exact_rational_sum(M, N, K):
    rng = np.random.default_rng(M * 7919 + N * 104729 + K)
    A = rand_f16_bits(rng, (M, K))
    B = rand_f16_bits(rng, (K, N))
    ex = exact_absdot(A, B)
    _, sab = oracle.gemm_relu_f16(A, B, want_absdot=True)
    ii, jj = np.divmod(np.arange(M * N), N)
    _, sab_pts = oracle.gemm_relu_f16_points(A, B, ii, jj, want_absdot=True)
    for i in range(M):
        for j in range(N):
            # K non-negative terms, each exact in double: relative error <= K 2^-53
            bound = Fraction(K) * Fraction(1, 2 ** 53) * ex[i][j]
            assert abs(Fraction(sab[i, j]) - ex[i][j]) <= bound, (i, j)
            assert abs(Fraction(sab_pts[i * N + j]) - ex[i][j]) <= bound, (i, j)


def test_absdot_integer_inputs_exact():
    # integer-valued inputs: every term and partial sum is exact
    a, b = workloads.make_inputs(13, 21, 37, dist="intsmall", seed=8)
    A, B = workloads.as_u16(a), workloads.as_u16(b)
    want = np.abs(a.numpy().astype(np.int64)) @ np.abs(b.numpy().astype(np.int64))
    _, sab = oracle.gemm_relu_f16(A, B, want_absdot=True)
    assert np.array_equal(sab, want.astype(np.float64))
    _, sab_r = oracle.gemm_relu_f16(A, B, want_absdot=True, rows=(3, 11))
    assert np.array_equal(sab_r, want[3:11].astype(np.float64))


def test_absdot_sign_invariance_and_signed_sum_of_abs():
    rng = np.random.default_rng(31)
    A = rand_f16_bits(rng, (9, 33))
    B = rand_f16_bits(rng, (33, 12))
    _, s0 = oracle.gemm_relu_f16(A, B, want_absdot=True)
    _, s1 = oracle.gemm_relu_f16(A ^ np.uint16(0x8000), B, want_absdot=True)
    _, s2 = oracle.gemm_relu_f16(A, B ^ np.uint16(0x8000), want_absdot=True)
    assert np.array_equal(s0, s1) and np.array_equal(s0, s2)
    # the signed sum of |A| @ |B| follows the same k order, so it is the same double
    _, pre_abs = oracle.gemm_relu_f16(abs_bits(A), abs_bits(B), want_pre=True)
    assert np.array_equal(s0, pre_abs)
    # it bounds the signed sum, with equality where all products share a sign
    _, pre = oracle.gemm_relu_f16(A, B, want_pre=True)
    assert (np.abs(pre) <= s0 * (1 + 33 * 2.0 ** -52)).all()


def test_absdot_same_for_every_epilogue_and_layout():
    rng = np.random.default_rng(32)
    A = rand_f16_bits(rng, (6, 19))
    B = rand_f16_bits(rng, (19, 10))
    bias = rand_f16_bits(rng, (10,))
    _, s0 = oracle.gemm_relu_f16(A, B, want_absdot=True)
    _, sg = oracle.gemm_bias_gelu_f16(A, B, bias, want_absdot=True)
    assert np.array_equal(s0, sg)  # the bias is not part of the product's error scale
    for ta, tb in LAYOUTS:
        _, st = oracle.gemm_relu_f16(_stored(A, ta), _stored(B, tb), want_absdot=True, trans_a=ta, trans_b=tb)
        assert np.array_equal(st, s0), (ta, tb)


ABSDOT_MUTANTS = {
    "absdot_no_abs_b": ("sab[j] += aa * fabs(brow[j]);", "sab[j] += aa * brow[j];"),
    "absdot_drop_last_k": ("sab[j] += aa * fabs(brow[j]);", "if (k + 1 < K) sab[j] += aa * fabs(brow[j]);"),
    "absdot_doubled": ("if (sab) absdot[i * N + j] = sab[j];", "if (sab) absdot[i * N + j] = 2.0 * sab[j];"),
    "absdot_points_no_abs_a": ("s += fabs(a) * fabs(b);", "s += a * fabs(b);"),
    "absdot_points_extra_term": ("s += fabs(a) * fabs(b);", "s += fabs(a) * fabs(b) + (k == 0 ? fabs(a) : 0.0);"),
}


def _absdot_pin_suite(mod) -> list[str]:
    global oracle
    checks = [
        ("exact", lambda: test_absdot_matches_exact_rational_sum(3, 17, 7)),
        ("exact_k1", lambda: test_absdot_matches_exact_rational_sum(1, 1, 1)),
        ("integer", test_absdot_integer_inputs_exact),
        ("signs", test_absdot_sign_invariance_and_signed_sum_of_abs),
        ("layouts", test_absdot_same_for_every_epilogue_and_layout),
    ]
    saved, fails = oracle, []
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


def test_absdot_pins_pass_on_real_oracle():
    assert _absdot_pin_suite(oracle) == []


@pytest.mark.parametrize("mutant", sorted(ABSDOT_MUTANTS))
def test_planted_absdot_mistake_is_caught(mutant, tmp_path):
    import importlib.util
    src_dir = os.path.join(os.path.dirname(HERE), "oracle")
    old, new = ABSDOT_MUTANTS[mutant]
    text = open(os.path.join(src_dir, "gemm_relu_oracle.c")).read()
    assert text.count(old) == 1, f"mutation anchor for {mutant} not found"
    dst = tmp_path / "oracle_mut"
    dst.mkdir()
    (dst / "gemm_relu_oracle.c").write_text(text.replace(old, new, 1))
    shutil.copy(os.path.join(src_dir, "__init__.py"), dst / "__init__.py")
    shutil.copy(os.path.join(src_dir, "attention_oracle.c"), dst / "attention_oracle.c")
    spec = importlib.util.spec_from_file_location(f"oracle_smut_{mutant}", dst / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _absdot_pin_suite(mod) != [], f"planted mistake {mutant} went unnoticed"
