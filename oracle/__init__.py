"""CPU oracle for C = ReLU(A @ B) and C = GELU(A @ B + bias) (fp16 in, fp16
out), and for row softmax and the attention forward pass -- TEST
INFRASTRUCTURE.

Only ``tests/``, the package smoke check in ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never imports it and shares no code
with it.

The arithmetic lives in ``gemm_relu_oracle.c`` and ``attention_oracle.c``
(plain C, built with gcc); this
module builds it on demand and marshals numpy arrays of fp16 bit patterns
(``uint16``) through ctypes. What each function computes, and the passage of
the TileLang pages it follows, is stated in the C source.

Parity is pinned by ``tests/test_oracle.py``: exhaustive fp16 decode/encode
checks, exact rational brute force on tiny shapes, identity / zero / K=1 closed
forms, integer-exact sums and the C >= 0 invariant.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_relu_oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "attention_oracle.c")]
# ORACLE_SANITIZE=1 selects the build with gcc's AddressSanitizer and
# UndefinedBehaviorSanitizer (the process must preload gcc's libasan)
_SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liboracle_gemm_relu_asan.so" if _SANITIZE else "liboracle_gemm_relu.so")
_lock = threading.Lock()
_lib = None
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math; with the
    sanitizers when ORACLE_SANITIZE=1). Returns the .so path."""
    if not force and os.path.exists(_LIB) and all(os.path.getmtime(_LIB) >= os.path.getmtime(f) for f in _SRCS):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", *(SANITIZE_FLAGS if _SANITIZE else []), *_SRCS, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build()
        lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_f16_rne.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16_rne.restype = ctypes.c_uint16
        lib.oracle_decode_f16.argtypes = [p, p, i64]
        lib.oracle_decode_f16.restype = None
        lib.oracle_encode_f16.argtypes = [p, p, i64]
        lib.oracle_encode_f16.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_gemm_relu_f16.argtypes = [i64, i64, i64, p, p, p, p, p]
        lib.oracle_gemm_relu_f16.restype = ctypes.c_int
        lib.oracle_gemm_relu_f16_rows.argtypes = [i64, i64, i64, p, p, p, p, p, i64, i64]
        lib.oracle_gemm_relu_f16_rows.restype = ctypes.c_int
        lib.oracle_gemm_relu_f16_points.argtypes = [i64, i64, i64, p, p, i64, p, p, p, p, p]
        lib.oracle_gemm_relu_f16_points.restype = ctypes.c_int
        lib.oracle_gelu.argtypes = [ctypes.c_double]
        lib.oracle_gelu.restype = ctypes.c_double
        lib.oracle_gemm_bias_gelu_f16_rows.argtypes = [i64, i64, i64, p, p, p, p, p, p, i64, i64]
        lib.oracle_gemm_bias_gelu_f16_rows.restype = ctypes.c_int
        lib.oracle_gemm_bias_gelu_f16_points.argtypes = [i64, i64, i64, p, p, p, i64, p, p, p, p, p]
        lib.oracle_gemm_bias_gelu_f16_points.restype = ctypes.c_int
        i32 = ctypes.c_int
        lib.oracle_gemm_f16_rows_t.argtypes = [i64, i64, i64, p, i32, p, i32, p, p, p, p, i64, i64]
        lib.oracle_gemm_f16_rows_t.restype = ctypes.c_int
        lib.oracle_gemm_f16_points_t.argtypes = [i64, i64, i64, p, i32, p, i32, p, i64, p, p, p, p, p]
        lib.oracle_gemm_f16_points_t.restype = ctypes.c_int
        lib.oracle_softmax_rows_f16.argtypes = [i64, i64, p, p, p]
        lib.oracle_softmax_rows_f16.restype = ctypes.c_int
        lib.oracle_attention_rows_f16.argtypes = [i64, i64, i64, i64, p, p, p, ctypes.c_double, i32, i64, p, p,
                                                  p, p, p, p]
        lib.oracle_attention_rows_f16.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(x: np.ndarray, shape) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("oracle inputs are fp16 bit patterns (numpy uint16)")
    if x.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {x.shape}")
    return x


def f16_to_f64(bits) -> np.ndarray:
    """Decode fp16 bit patterns (uint16 array) to float64."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode_f16(_ptr(b), _ptr(out), b.size)
    return out


def f64_to_f16(x) -> np.ndarray:
    """Encode float64 values to fp16 bit patterns, round to nearest even."""
    v = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_encode_f16(_ptr(v), _ptr(out), v.size)
    return out


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def gelu(x) -> np.ndarray:
    """GELU(x) = x * Phi(x) in float64, element by element."""
    lib = _load()
    v = np.asarray(x, dtype=np.float64)
    return np.vectorize(lib.oracle_gelu, otypes=[np.float64])(v)


def _dims(A, B, trans_a, trans_b):
    """M, N, K of op(A) @ op(B) from the stored shapes: A is [M, K], or [K, M]
    when trans_a; B is [K, N], or [N, K] when trans_b."""
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    return M, N, K


def _rows(A, B, bias, want_pre, want_absdot, rows, trans_a=False, trans_b=False):
    M, N, K = _dims(A, B, trans_a, trans_b)
    A = _u16(A, A.shape)
    B = _u16(B, B.shape)
    if bias is not None:
        bias = _u16(bias, (N,))
    r0, r1 = (0, M) if rows is None else rows
    # the C routine indexes C, pre and absdot as full [M, N] arrays; only the
    # requested rows are touched, so offset the base pointers accordingly
    nr = r1 - r0
    C = np.zeros((nr, N), dtype=np.uint16)
    pre = np.zeros((nr, N), dtype=np.float64) if want_pre else None
    sab = np.zeros((nr, N), dtype=np.float64) if want_absdot else None

    def base(arr, itemsize):
        if arr is None:
            return None
        return ctypes.c_void_p(arr.ctypes.data - r0 * N * itemsize)

    lib = _load()
    if trans_a or trans_b:
        rc = lib.oracle_gemm_f16_rows_t(M, N, K, _ptr(A), int(trans_a), _ptr(B), int(trans_b), _ptr(bias),
                                        base(C, 2), base(pre, 8), base(sab, 8), r0, r1)
    elif bias is None:
        rc = lib.oracle_gemm_relu_f16_rows(M, N, K, _ptr(A), _ptr(B), base(C, 2), base(pre, 8), base(sab, 8), r0, r1)
    else:
        rc = lib.oracle_gemm_bias_gelu_f16_rows(M, N, K, _ptr(A), _ptr(B), _ptr(bias), base(C, 2), base(pre, 8),
                                                base(sab, 8), r0, r1)
    if rc != 0:
        raise RuntimeError("oracle rows routine failed")
    out = [C]
    if want_pre:
        out.append(pre)
    if want_absdot:
        out.append(sab)
    return out[0] if len(out) == 1 else tuple(out)


def _points(A, B, bias, ii, jj, want_pre, want_absdot, trans_a=False, trans_b=False):
    M, N, K = _dims(A, B, trans_a, trans_b)
    A = _u16(A, A.shape)
    B = _u16(B, B.shape)
    if bias is not None:
        bias = _u16(bias, (N,))
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape or ii.ndim != 1:
        raise ValueError("ii and jj must be 1-D of equal length")
    out = np.zeros(ii.shape, dtype=np.uint16)
    pre = np.zeros(ii.shape, dtype=np.float64) if want_pre else None
    sab = np.zeros(ii.shape, dtype=np.float64) if want_absdot else None
    lib = _load()
    if trans_a or trans_b:
        rc = lib.oracle_gemm_f16_points_t(M, N, K, _ptr(A), int(trans_a), _ptr(B), int(trans_b), _ptr(bias),
                                          ii.size, _ptr(ii), _ptr(jj), _ptr(out), _ptr(pre), _ptr(sab))
    elif bias is None:
        rc = lib.oracle_gemm_relu_f16_points(M, N, K, _ptr(A), _ptr(B), ii.size, _ptr(ii), _ptr(jj), _ptr(out),
                                             _ptr(pre), _ptr(sab))
    else:
        rc = lib.oracle_gemm_bias_gelu_f16_points(M, N, K, _ptr(A), _ptr(B), _ptr(bias), ii.size, _ptr(ii),
                                                  _ptr(jj), _ptr(out), _ptr(pre), _ptr(sab))
    if rc != 0:
        raise RuntimeError("oracle points routine failed")
    res = [out]
    if want_pre:
        res.append(pre)
    if want_absdot:
        res.append(sab)
    return res[0] if len(res) == 1 else tuple(res)


def gemm_relu_f16(A: np.ndarray, B: np.ndarray, *, want_pre: bool = False,
                  want_absdot: bool = False, rows: tuple[int, int] | None = None,
                  trans_a: bool = False, trans_b: bool = False):
    """C = ReLU(op(A) @ op(B)) as fp16 bit patterns.

    A: uint16 [M, K] (or [K, M] stored, with trans_a), B: uint16 [K, N] (or
    [N, K] stored, with trans_b). With ``rows=(r0, r1)`` only those rows are
    computed and returned (shape [r1-r0, N]). Optionally also returns the
    float64 pre-activation sums and sum_k |a||b| for the same rows.
    """
    return _rows(A, B, None, want_pre, want_absdot, rows, trans_a, trans_b)


def gemm_relu_f16_points(A: np.ndarray, B: np.ndarray, ii, jj, *, want_pre: bool = False,
                         want_absdot: bool = False, trans_a: bool = False, trans_b: bool = False):
    """Elements C[ii[t], jj[t]] of ReLU(op(A) @ op(B)) as fp16 bit patterns."""
    return _points(A, B, None, ii, jj, want_pre, want_absdot, trans_a, trans_b)


def gemm_bias_gelu_f16(A: np.ndarray, B: np.ndarray, bias: np.ndarray, *, want_pre: bool = False,
                       want_absdot: bool = False, rows: tuple[int, int] | None = None,
                       trans_a: bool = False, trans_b: bool = False):
    """C = GELU(A @ B + bias) as fp16 bit patterns; bias: uint16 [N], one value per column.

    ``pre`` (if asked for) is the float64 value A @ B + bias before GELU.
    """
    return _rows(A, B, bias, want_pre, want_absdot, rows, trans_a, trans_b)


def gemm_bias_gelu_f16_points(A: np.ndarray, B: np.ndarray, bias: np.ndarray, ii, jj, *,
                              want_pre: bool = False, want_absdot: bool = False,
                              trans_a: bool = False, trans_b: bool = False):
    """Elements C[ii[t], jj[t]] of GELU(op(A) @ op(B) + bias) as fp16 bit patterns."""
    return _points(A, B, bias, ii, jj, want_pre, want_absdot, trans_a, trans_b)


def softmax_rows_f16(X: np.ndarray, *, want_double: bool = False):
    """Row softmax of fp16 bit patterns X [rows, cols]: fp16 bit patterns, and
    optionally the float64 values before the rounding."""
    X = np.ascontiguousarray(X)
    if X.dtype != np.uint16 or X.ndim != 2:
        raise ValueError("X must be a 2-D uint16 array of fp16 bit patterns")
    rows, cols = X.shape
    Y = np.zeros((rows, cols), dtype=np.uint16)
    yd = np.zeros((rows, cols), dtype=np.float64) if want_double else None
    if _load().oracle_softmax_rows_f16(rows, cols, _ptr(X), _ptr(Y), _ptr(yd)) != 0:
        raise RuntimeError("oracle softmax failed")
    return (Y, yd) if want_double else Y


def _bhsd(x, name):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16 or x.ndim != 4:
        raise ValueError(f"{name} must be a [B, H, S, D] uint16 array of fp16 bit patterns")
    return x


def attention_rows_f16(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, causal: bool, bh, qi, *,
                       want_double: bool = False, want_lse: bool = False, want_pv: bool = False):
    """Selected query rows of the attention forward pass.

    Q: [B, H, Sq, D], K and V: [B, H, Skv, D] (fp16 bit patterns). Row t is
    query qi[t] of batch-head bh[t] = b * H + h. Returns O rows [n, D] (fp16
    bit patterns) and, as asked for, their float64 values, the log-sum-exp per
    row and sum_j p_j |V[j][d]| per element.
    """
    Q, K, V = _bhsd(Q, "Q"), _bhsd(K, "K"), _bhsd(V, "V")
    B, H, Sq, D = Q.shape
    if K.shape[:2] != (B, H) or K.shape[3] != D or V.shape != K.shape:
        raise ValueError(f"shapes {Q.shape}, {K.shape}, {V.shape} do not match")
    Skv = K.shape[2]
    bh = np.ascontiguousarray(bh, dtype=np.int64)
    qi = np.ascontiguousarray(qi, dtype=np.int64)
    if bh.shape != qi.shape or bh.ndim != 1:
        raise ValueError("bh and qi must be 1-D of equal length")
    n = bh.size
    out = np.zeros((n, D), dtype=np.uint16)
    od = np.zeros((n, D), dtype=np.float64) if want_double else None
    lse = np.zeros(n, dtype=np.float64) if want_lse else None
    pv = np.zeros((n, D), dtype=np.float64) if want_pv else None
    rc = _load().oracle_attention_rows_f16(B * H, Sq, Skv, D, _ptr(Q), _ptr(K), _ptr(V), float(scale), int(causal), n,
                                           _ptr(bh), _ptr(qi), _ptr(out), _ptr(od), _ptr(lse), _ptr(pv))
    if rc != 0:
        raise RuntimeError("oracle attention failed")
    res = [out]
    if want_double:
        res.append(od)
    if want_lse:
        res.append(lse)
    if want_pv:
        res.append(pv)
    return res[0] if len(res) == 1 else tuple(res)


def attention_f16(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, causal: bool, **kw):
    """Every query row of the attention forward pass: O [B, H, Sq, D] (and the
    extras of attention_rows_f16, reshaped likewise)."""
    B, H, Sq, D = np.shape(Q)
    bh, qi = np.divmod(np.arange(B * H * Sq, dtype=np.int64), Sq)
    res = attention_rows_f16(Q, K, V, scale, causal, bh, qi, **kw)
    if not isinstance(res, tuple):
        return res.reshape(B, H, Sq, D)
    out = []
    for r in res:
        out.append(r.reshape(B, H, Sq) if r.ndim == 1 else r.reshape(B, H, Sq, D))
    return tuple(out)

