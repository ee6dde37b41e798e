"""ctypes binding of libgemm_relu.so (the C ABI in include/gemm_relu.h).

Argument marshalling only: every step of C = ReLU(A @ B) runs in the HIP
library. Torch is used for device memory and streams. There is no fallback: if
the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# GEMM_RELU_LIB selects another build of the same library (the host-sanitized
# one, for the CPU checks); the default is the in-tree build
LIB_PATH = os.environ.get("GEMM_RELU_LIB") or os.path.join(PKG, "libgemm_relu.so")

OK, EINVAL, EUNSUPPORTED, EHIP, ENOMEM, ETOOBIG = 0, 1, 2, 3, 4, 5
NOALLOC_MAX_TILES = 4096                      # GEMM_RELU_NOALLOC_MAX_TILES
NOALLOC_MAX_PARTIAL_BYTES = 2 * 1024 * 1024   # GEMM_RELU_NOALLOC_MAX_PARTIAL_BYTES
TILE_AUTO = -1
OP_N, OP_T = 0, 1  # operand as stored / stored transposed
ORDER_DEFAULT, ORDER_ROW_MAJOR = 0, 1


class GemmReluError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gemm_relu status {status}: {msg}")
        self.status = status


class Opts(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("block_order", ctypes.c_int32),
                ("group_m", ctypes.c_int32), ("reserved", ctypes.c_int32 * 5)]


FAMILY_PIPELINED, FAMILY_STAGED, FAMILY_SPLITK, FAMILY_SMALL = 0, 1, 2, 3


class TileDesc(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("waves_m", ctypes.c_int32), ("waves_n", ctypes.c_int32),
                ("waves_k", ctypes.c_int32), ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("default_group_m", ctypes.c_int32), ("family", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 4)]

    def as_dict(self) -> dict:
        return {f: int(getattr(self, f)) for f, _ in self._fields_ if f != "reserved"}


_lock = threading.Lock()
_lib = None

EXPORTED = ("gemm_relu_f16", "gemm_relu_f16_noalloc", "gemm_relu_f16_ex", "gemm_relu_f16_op", "gemm_bias_gelu_f16",
            "gemm_bias_gelu_f16_ex", "gemm_bias_gelu_f16_op", "gemm_relu_strerror", "gemm_relu_tile_count",
            "gemm_relu_tile_name", "gemm_relu_tile_info", "gemm_relu_default_order", "gemm_relu_select_tile",
            "gemm_relu_select_tile_op", "softmax_rows_f16", "flash_attn_fwd_f16")


def load():
    """Load the library, building it first only if it has never been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.gemm_relu_f16.argtypes = [i64, i64, i64, p, p, p, p]
        lib.gemm_relu_f16.restype = i32
        lib.gemm_relu_f16_noalloc.argtypes = [i64, i64, i64, p, p, p, p]
        lib.gemm_relu_f16_noalloc.restype = i32
        lib.gemm_relu_f16_ex.argtypes = [i64, i64, i64, p, p, p, p, ctypes.POINTER(Opts)]
        lib.gemm_relu_f16_ex.restype = i32
        lib.gemm_bias_gelu_f16.argtypes = [i64, i64, i64, p, p, p, p, p]
        lib.gemm_bias_gelu_f16.restype = i32
        lib.gemm_bias_gelu_f16_ex.argtypes = [i64, i64, i64, p, p, p, p, p, ctypes.POINTER(Opts)]
        lib.gemm_bias_gelu_f16_ex.restype = i32
        lib.gemm_relu_f16_op.argtypes = [i64, i64, i64, p, i32, p, i32, p, p, ctypes.POINTER(Opts)]
        lib.gemm_relu_f16_op.restype = i32
        lib.gemm_bias_gelu_f16_op.argtypes = [i64, i64, i64, p, i32, p, i32, p, p, p, ctypes.POINTER(Opts)]
        lib.gemm_bias_gelu_f16_op.restype = i32
        lib.gemm_relu_select_tile_op.argtypes = [i64, i64, i64, i32, i32, p, p, p]
        lib.gemm_relu_select_tile_op.restype = i32
        lib.softmax_rows_f16.argtypes = [i64, i64, p, p, p]
        lib.softmax_rows_f16.restype = i32
        lib.flash_attn_fwd_f16.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, ctypes.c_float, i32, p]
        lib.flash_attn_fwd_f16.restype = i32
        lib.gemm_relu_strerror.argtypes = [i32]
        lib.gemm_relu_strerror.restype = ctypes.c_char_p
        lib.gemm_relu_tile_count.argtypes = []
        lib.gemm_relu_tile_count.restype = i32
        lib.gemm_relu_tile_name.argtypes = [i32]
        lib.gemm_relu_tile_name.restype = ctypes.c_char_p
        lib.gemm_relu_tile_info.argtypes = [i32, ctypes.POINTER(TileDesc)]
        lib.gemm_relu_tile_info.restype = i32
        lib.gemm_relu_default_order.argtypes = [i32, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        lib.gemm_relu_default_order.restype = i32
        lib.gemm_relu_select_tile.argtypes = [i64, i64, i64, p, p, p]
        lib.gemm_relu_select_tile.restype = i32
        _lib = lib
        return lib


def strerror(status: int) -> str:
    return load().gemm_relu_strerror(int(status)).decode()


def _check(status: int) -> None:
    if status != OK:
        raise GemmReluError(status, strerror(status))


def make_opts(tile: int | None = None, block_order: int = ORDER_DEFAULT, group_m: int = 0) -> Opts:
    o = Opts()
    o.tile = TILE_AUTO if tile is None else int(tile)
    o.block_order = int(block_order)
    o.group_m = int(group_m)
    return o


def gemm_relu_f16(M: int, N: int, K: int, A: int, B: int, C: int, stream: int = 0) -> int:
    """Raw C-ABI call with integer device pointers; returns the status code."""
    return load().gemm_relu_f16(M, N, K, A or None, B or None, C or None, stream or None)


def gemm_relu_f16_noalloc(M: int, N: int, K: int, A: int, B: int, C: int, stream: int = 0) -> int:
    """Raw C-ABI call of the allocation-free variant of gemm_relu_f16 (its
    split-K scratch is the library's fixed per-GPU array); returns the status
    code."""
    return load().gemm_relu_f16_noalloc(M, N, K, A or None, B or None, C or None, stream or None)


def gemm_relu_f16_ex(M: int, N: int, K: int, A: int, B: int, C: int, stream: int = 0,
                     opts: Opts | None = None) -> int:
    """Raw C-ABI call with launch options; returns the status code."""
    return load().gemm_relu_f16_ex(M, N, K, A or None, B or None, C or None, stream or None,
                                   ctypes.byref(opts) if opts is not None else None)


def gemm_bias_gelu_f16(M: int, N: int, K: int, A: int, B: int, bias: int, C: int, stream: int = 0) -> int:
    """Raw C-ABI call of C = GELU(A @ B + bias) with integer device pointers; returns the status code."""
    return load().gemm_bias_gelu_f16(M, N, K, A or None, B or None, bias or None, C or None, stream or None)


def gemm_bias_gelu_f16_ex(M: int, N: int, K: int, A: int, B: int, bias: int, C: int, stream: int = 0,
                          opts: Opts | None = None) -> int:
    """Raw C-ABI call of C = GELU(A @ B + bias) with launch options; returns the status code."""
    return load().gemm_bias_gelu_f16_ex(M, N, K, A or None, B or None, bias or None, C or None, stream or None,
                                        ctypes.byref(opts) if opts is not None else None)


def gemm_relu_f16_op(M: int, N: int, K: int, A: int, op_a: int, B: int, op_b: int, C: int, stream: int = 0,
                     opts: Opts | None = None) -> int:
    """Raw C-ABI call of C = ReLU(op(A) @ op(B)); returns the status code."""
    return load().gemm_relu_f16_op(M, N, K, A or None, int(op_a), B or None, int(op_b), C or None, stream or None,
                                   ctypes.byref(opts) if opts is not None else None)


def gemm_bias_gelu_f16_op(M: int, N: int, K: int, A: int, op_a: int, B: int, op_b: int, bias: int, C: int,
                          stream: int = 0, opts: Opts | None = None) -> int:
    """Raw C-ABI call of C = GELU(op(A) @ op(B) + bias); returns the status code."""
    return load().gemm_bias_gelu_f16_op(M, N, K, A or None, int(op_a), B or None, int(op_b), bias or None,
                                        C or None, stream or None, ctypes.byref(opts) if opts is not None else None)


def tile_count() -> int:
    return int(load().gemm_relu_tile_count())


def tile_name(tile: int) -> str:
    return load().gemm_relu_tile_name(int(tile)).decode()


def tile_info(tile: int) -> dict:
    """Launch parameters of a compiled tile (see gemm_relu_tile_desc)."""
    d = TileDesc()
    _check(load().gemm_relu_tile_info(int(tile), ctypes.byref(d)))
    return d.as_dict()


def default_order(tile: int, M: int, N: int) -> tuple[int, int]:
    """(block_order, group_m) of a launch of `tile` over an M x N output whose
    opts leave both at their defaults."""
    order, group = ctypes.c_int32(), ctypes.c_int32()
    _check(load().gemm_relu_default_order(int(tile), int(M), int(N), ctypes.byref(order), ctypes.byref(group)))
    return int(order.value), int(group.value)


def select_tile(M: int, N: int, K: int, A: int = 0, B: int = 0, C: int = 0, *, trans_a: bool = False,
                trans_b: bool = False) -> int:
    return int(load().gemm_relu_select_tile_op(M, N, K, int(trans_a), int(trans_b), A or None, B or None,
                                               C or None))


def _check_operands(a, b, out, trans_a=False, trans_b=False):
    """a is the stored A ([M, K], or [K, M] with trans_a); b the stored B ([K, N],
    or [N, K] with trans_b)."""
    import torch

    if a.dtype != torch.float16 or b.dtype != torch.float16:
        raise TypeError("a and b must be float16")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be matrices")
    M, K = (a.shape[1], a.shape[0]) if trans_a else (a.shape[0], a.shape[1])
    K2, N = (b.shape[1], b.shape[0]) if trans_b else (b.shape[0], b.shape[1])
    if K != K2:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} do not chain "
                         f"(trans_a={trans_a}, trans_b={trans_b})")
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("a and b must be on the same GPU")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous row-major")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.device)
    else:
        if out.dtype != torch.float16 or tuple(out.shape) != (M, N) or out.device != a.device:
            raise ValueError("out must be float16 [M, N] on the inputs' device")
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    return M, N, K, out


def gemm_relu(a, b, out=None, *, trans_a: bool = False, trans_b: bool = False, tile: int | None = None,
              block_order: int = ORDER_DEFAULT, group_m: int = 0, stream=None):
    """C = ReLU(op(a) @ op(b)) for fp16 CUDA(HIP) tensors; returns out[M,N].

    a is [M, K] (or [K, M] with trans_a, op(a) = a.T), b is [K, N] (or [N, K]
    with trans_b). Enqueued on torch's current stream (or ``stream``); does not
    synchronise.
    """
    import torch

    M, N, K, out = _check_operands(a, b, out, trans_a, trans_b)
    s = stream if stream is not None else torch.cuda.current_stream(a.device)
    opts = make_opts(tile, block_order, group_m)
    with torch.cuda.device(a.device):
        _check(gemm_relu_f16_op(M, N, K, a.data_ptr(), int(trans_a), b.data_ptr(), int(trans_b), out.data_ptr(),
                                s.cuda_stream, opts))
    return out


def gemm_bias_gelu(a, b, bias, out=None, *, trans_a: bool = False, trans_b: bool = False,
                   tile: int | None = None, block_order: int = ORDER_DEFAULT, group_m: int = 0, stream=None):
    """C = GELU(op(a) @ op(b) + bias) for fp16 tensors (layouts as gemm_relu), bias[N]; returns out[M,N].

    Enqueued on torch's current stream (or ``stream``); does not synchronise.
    """
    import torch

    M, N, K, out = _check_operands(a, b, out, trans_a, trans_b)
    if bias.dtype != torch.float16 or bias.dim() != 1 or bias.shape[0] != N:
        raise ValueError(f"bias must be float16 [{N}]")
    if not bias.is_cuda or bias.device != a.device or not bias.is_contiguous():
        raise ValueError("bias must be contiguous on the inputs' device")
    s = stream if stream is not None else torch.cuda.current_stream(a.device)
    opts = make_opts(tile, block_order, group_m)
    with torch.cuda.device(a.device):
        _check(gemm_bias_gelu_f16_op(M, N, K, a.data_ptr(), int(trans_a), b.data_ptr(), int(trans_b),
                                     bias.data_ptr(), out.data_ptr(), s.cuda_stream, opts))
    return out


def softmax_rows_f16(rows: int, cols: int, X: int, Y: int, stream: int = 0) -> int:
    """Raw C-ABI call of the row softmax; returns the status code."""
    return load().softmax_rows_f16(rows, cols, X or None, Y or None, stream or None)


def flash_attn_fwd_f16(B: int, H: int, Sq: int, Skv: int, D: int, Q: int, K: int, V: int, O: int, lse: int,
                       scale: float, causal: int, stream: int = 0) -> int:
    """Raw C-ABI call of the attention forward pass; returns the status code."""
    return load().flash_attn_fwd_f16(B, H, Sq, Skv, D, Q or None, K or None, V or None, O or None, lse or None,
                                     float(scale), int(causal), stream or None)


def softmax_rows(x, out=None, *, stream=None):
    """Row softmax of a 2-D fp16 CUDA(HIP) tensor; returns out (may be x itself)."""
    import torch

    if x.dtype != torch.float16 or x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D float16 GPU tensor")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError("out must match x")
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        _check(softmax_rows_f16(x.shape[0], x.shape[1], x.data_ptr(), out.data_ptr(), s.cuda_stream))
    return out


def flash_attn_fwd(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, return_lse: bool = False,
                   stream=None):
    """Attention forward for fp16 tensors q [B, H, Sq, D], k and v [B, H, Skv, D]
    (contiguous, D = 64 or 128); scale defaults to 1/sqrt(D). Returns out
    [B, H, Sq, D] (and the fp32 log-sum-exp [B, H, Sq] with return_lse)."""
    import torch

    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.float16 or t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D float16 GPU tensor")
    B, H, Sq, D = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != D or v.shape != k.shape or k.device != q.device or v.device != q.device:
        raise ValueError(f"shapes {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)} do not match")
    Skv = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must match q")
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    sc = (1.0 / D ** 0.5) if scale is None else float(scale)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        _check(flash_attn_fwd_f16(B, H, Sq, Skv, D, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr() if lse is not None else 0, sc, int(causal), s.cuda_stream))
    return (out, lse) if return_lse else out

