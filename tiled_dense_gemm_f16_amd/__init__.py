"""MI355X (gfx950) fp16 GEMM with a fused ReLU: C = ReLU(A @ B) (and with a
fused bias + GELU epilogue: C = GELU(A @ B + bias)).

The computation is the GEMM + ReLU example of "Writing high-performance
kernels in TileLang" (section "Escribamos un GEMM"), implemented as
hand-written HIP for CDNA4 behind the C ABI in ``include/gemm_relu.h``.
This package is the thin Python binding of that ABI.
"""
from ._binding import (  # noqa: F401
    EHIP, EINVAL, ENOMEM, ETOOBIG, EUNSUPPORTED, EXPORTED, FAMILY_PIPELINED, FAMILY_SMALL, FAMILY_SPLITK, FAMILY_STAGED, LIB_PATH, OK,
    OP_N, OP_T, ORDER_DEFAULT, ORDER_ROW_MAJOR, TILE_AUTO, GemmReluError, Opts, TileDesc, default_order, gemm_bias_gelu,
    gemm_bias_gelu_f16, gemm_bias_gelu_f16_ex, gemm_bias_gelu_f16_op, gemm_relu, gemm_relu_f16, gemm_relu_f16_ex,
    gemm_relu_f16_noalloc, gemm_relu_f16_op, load, make_opts, NOALLOC_MAX_PARTIAL_BYTES, NOALLOC_MAX_TILES, select_tile, strerror, tile_count, tile_info, tile_name, softmax_rows,
    softmax_rows_f16, flash_attn_fwd, flash_attn_fwd_f16,
)
