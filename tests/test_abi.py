"""Host-side checks of the C ABI (no GPU needed, no compute call).

The library must load, export every entry point that include/gemm_relu.h
declares, and reject bad arguments before it makes any HIP runtime call.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import sys

import pytest

import tiled_dense_gemm_f16_amd as gr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gemm_relu.h", "attention.h")]


def declared_functions() -> list[str]:
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert "gemm_relu_f16" in names and "gemm_relu_f16_ex" in names
    assert "gemm_bias_gelu_f16" in names and "gemm_bias_gelu_f16_ex" in names
    assert "softmax_rows_f16" in names and "flash_attn_fwd_f16" in names
    assert set(names) == set(gr.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = gr.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", gr.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name


def test_library_targets_gfx950_only(tmp_path):
    fatbin = tmp_path / "fatbin.bin"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", gr.LIB_PATH, str(fatbin)],
                   check=True)
    out = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o",
                          f"--input={fatbin}"], capture_output=True, text=True, check=True)
    targets = [t for t in out.stdout.split() if "amdgcn" in t]
    assert targets and all("gfx950" in t for t in targets), targets


def test_strerror_and_tiles():
    assert gr.strerror(gr.OK) == "success"
    for s in (gr.EINVAL, gr.EUNSUPPORTED, gr.EHIP, gr.ENOMEM):
        assert gr.strerror(s) and gr.strerror(s) != "success"
    assert gr.strerror(999) == "unknown status"
    n = gr.tile_count()
    assert n >= 4
    names = [gr.tile_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    assert "128x128x64" in names[1]  # the pages' tile is kept as a named entry
    assert gr.tile_name(-1) == "" and gr.tile_name(n) == ""


def test_tile_selection_is_host_only():
    # the cost model's choices on shapes where the offline sweep's winner is
    # clear: few rows -> split-K tiles; otherwise the largest tile that still
    # fills the 256 compute units
    name = lambda *s: gr.tile_name(gr.select_tile(*s))  # noqa: E731
    # 256x256 with A stored M x K loaded two steps at a time (whole lines)
    assert name(4096, 4096, 4096) == "256x256x32s4_w2x2_mfma32x32x16_lds-dma-a2"
    assert name(16, 8192, 8192).startswith("splitk_16x")
    assert name(1, 8192, 8192).startswith("splitk_16x")
    assert name(4096, 64, 4096).startswith("32x64x64s4_w1x2")  # narrow: 128 tiles of 32x64
    assert name(32, 8192, 8192).startswith("splitk_16x")     # few rows: split-K only
    assert name(64, 8192, 8192).startswith("32x64x64s4_w1x2")
    assert name(3072, 3072, 3072).startswith("256x256x32s4_w2x2")  # 144 tiles of 256x256
    assert name(2560, 2560, 2560).startswith("128x256")  # 200 tiles
    assert name(2048, 2048, 2048).startswith("64x256")  # 256 tiles
    assert name(1024, 1024, 1024).startswith("64x64x64s4_w2x2_mfma32x32x16_lds-small")  # 256 tiles of 64x64
    assert name(1536, 1536, 1536).startswith("64x64x64s4_w2x2_mfma32x32x16_lds-small")  # 2.25 per compute unit
    # rows of A and B that are not whole 128-byte lines cost the small tiles more L2 requests
    assert name(1000, 1016, 1000).startswith("splitk_32x")
    assert name(512, 4096, 8192).startswith("splitk_64x")  # 256 tiles of 64x128
    assert name(256, 256, 256).startswith("32x64x64s4_w1x2")  # latency-bound: the most workgroups
    assert name(512, 512, 512).startswith("32x64x64s4_w1x2")
    # transposed layouts have their own rates: with A stored K x M the split-K
    # tiles (element-wise A reads) lose to the pipelined ones at mid sizes
    tname = lambda *s, **kw: gr.tile_name(gr.select_tile(*s, **kw))  # noqa: E731
    assert tname(1024, 1024, 1024, trans_a=True).startswith("64x256")
    assert tname(512, 4096, 8192, trans_a=True).startswith("64x256")
    # B stored N x K: the 64 x 256 tile that loads A two steps at a time
    # beats the 128 x 128 staged one (no transpose of B) at 2048^3
    assert tname(2048, 2048, 2048, trans_b=True) == "64x256x32s4_w1x2_mfma32x32x16_lds-dma-a2"
    for ta in (False, True):
        for tb in (False, True):
            assert tname(16, 8192, 8192, trans_a=ta, trans_b=tb).startswith("splitk_16x")  # few rows
            # the paired-A tile where A is stored M x K, the plain one where it is K x M
            assert gr.select_tile(4096, 4096, 4096, trans_a=ta, trans_b=tb) == (0 if ta else 14)
    # the split-K kernel's 32-bit A offsets: M*K*2 must stay below 2^31
    assert "splitk" not in name(65536, 256, 16384)
    # K or N not a multiple of 8 -> the generic element-wise path
    assert gr.select_tile(64, 64, 7) == -1
    assert gr.select_tile(64, 9, 64) == -1
    # misaligned pointers -> generic path
    assert gr.select_tile(64, 64, 64, 0x1000, 0x2002, 0x3000) == -1
    assert gr.select_tile(64, 64, 64, 0x1000, 0x2000, 0x3000) >= 0


def test_tile_info_describes_every_tile():
    # the tuner's search space: each compiled tile's parameters agree with its
    # name, and every tile fits the 160 KiB of LDS of a gfx950 compute unit
    for t in range(gr.tile_count()):
        d = gr.tile_info(t)
        name = gr.tile_name(t)
        assert d["lds_bytes"] <= 160 * 1024, name
        assert d["threads"] == 64 * d["waves_m"] * d["waves_n"] * d["waves_k"], name
        assert f"{d['bm']}x{d['bn']}" in name, name
        assert d["family"] in (gr.FAMILY_PIPELINED, gr.FAMILY_STAGED, gr.FAMILY_SPLITK, gr.FAMILY_SMALL)
        assert bool(d["split_k"]) == ("splitk" in name) == (d["family"] == gr.FAMILY_SPLITK), name
        assert ("lds-small" in name) == (d["family"] == gr.FAMILY_SMALL), name
        if d["family"] in (gr.FAMILY_PIPELINED, gr.FAMILY_SMALL):
            assert f"x{d['bk']}s{d['stages']}_w{d['waves_m']}x{d['waves_n']}" in name, name
            assert d["lds_bytes"] == d["stages"] * (d["bm"] + d["bn"]) * d["bk"] * 2, name
        elif d["family"] == gr.FAMILY_STAGED:
            assert d["lds_bytes"] == 2 * (d["bm"] + d["bn"]) * d["bk"] * 2, name
    lib = gr.load()
    d = gr.TileDesc()
    assert lib.gemm_relu_tile_info(gr.tile_count(), ctypes.byref(d)) == gr.EUNSUPPORTED
    assert lib.gemm_relu_tile_info(-1, ctypes.byref(d)) == gr.EUNSUPPORTED
    assert lib.gemm_relu_tile_info(0, None) == gr.EINVAL


def test_tuner_candidates():
    from tiled_dense_gemm_f16_amd import tune

    c = tune.candidates(4096, 4096, 4096)
    tiles = {x["tile"] for x in c}
    assert tiles == set(range(gr.tile_count()))
    for x in c:
        d = gr.tile_info(x["tile"])
        if x["block_order"] == gr.ORDER_ROW_MAJOR:
            assert x["group_m"] == 0 and not d["split_k"]
        assert x["group_m"] <= -(-4096 // d["bm"])
    # the library's own group is always timed (384 x 6144: 6 tile-rows of 64,
    # default group 8 -> 4)
    c384 = tune.candidates(384, 6144, 6144)
    t64 = next(t for t in range(gr.tile_count()) if gr.tile_name(t).startswith("64x64x64s4"))
    g_def = gr.default_order(t64, 384, 6144)[1]
    assert g_def == 4
    assert any(x["tile"] == t64 and x["block_order"] == gr.ORDER_DEFAULT and x["group_m"] == g_def for x in c384)
    # a grid one tile-row high has no block order to choose
    assert all(x["group_m"] == 0 and x["block_order"] == gr.ORDER_DEFAULT for x in tune.candidates(16, 8192, 8192))
    # a tighter LDS budget prunes the big tiles
    small = tune.candidates(1024, 1024, 1024, lds_limit=64 * 1024)
    assert small and all(gr.tile_info(x["tile"])["lds_bytes"] <= 64 * 1024 for x in small)


def _tile_named(prefix):
    return next(t for t in range(gr.tile_count()) if gr.tile_name(t).startswith(prefix))


def test_default_group_rule():
    # (tile default, tile-rows) -> group: a power of two, at least two groups
    # from four tile-rows on (tile-columns do not matter)
    tiles = {8: _tile_named("64x64x64s4"), 4: _tile_named("256x256x32s4_w2x2"), 1: _tile_named("16x64x64")}
    cases = {(8, 16): 8, (8, 8): 4, (8, 6): 4, (8, 4): 2, (8, 3): 2, (8, 2): 2, (8, 1): 1,
             (4, 16): 4, (4, 4): 2, (4, 5): 4, (1, 16): 1}
    for (g, tm), want in cases.items():
        t = tiles[g]
        d = gr.tile_info(t)
        assert d["default_group_m"] == g
        for N in (64, 8192):
            assert gr.default_order(t, tm * d["bm"], N)[1] == want, (g, tm, N)
        # a ragged last tile-row counts as a row
        assert gr.default_order(t, (tm - 1) * d["bm"] + 1, 64)[1] == want, (g, tm)


def test_default_order_rule():
    # row-major only on grids of one round (<= 256 tiles) of tiles under 256
    # rows, two tile-rows or more, a multiple of 4 tile-columns and at most
    # twice as many tile-rows as tile-columns
    t64, t32 = _tile_named("64x64x64s4"), _tile_named("32x64x64s4")
    t256, t64x256 = _tile_named("256x256x32s4_w2x2"), _tile_named("64x256x32s5")
    tsk = _tile_named("splitk_64x128")
    RM, G = gr.ORDER_ROW_MAJOR, gr.ORDER_DEFAULT
    cases = [(t64, 1024, 1024, RM), (t64, 1024, 512, RM), (t64, 1088, 512, G), (t64, 4096, 4096, G),
             (t64, 960, 960, G), (t64, 64, 8192, G), (t64, 128, 8192, RM), (t64, 2560, 640, G),
             (t32, 256, 256, RM), (t32, 512, 512, RM), (t256, 1024, 1024, G), (t256, 4096, 4096, G),
             (t64x256, 2048, 2048, G), (t64x256, 1024, 4096, RM), (t64x256, 4096, 1024, G), (tsk, 64, 1024, G),
             (t64, 0, 0, G)]
    for t, M, N, want in cases:
        assert gr.default_order(t, M, N)[0] == want, (gr.tile_name(t), M, N)
    lib = gr.load()
    o, g = ctypes.c_int32(7), ctypes.c_int32(7)
    assert lib.gemm_relu_default_order(gr.tile_count(), 64, 64, ctypes.byref(o), ctypes.byref(g)) == gr.EUNSUPPORTED
    assert lib.gemm_relu_default_order(-1, 64, 64, ctypes.byref(o), ctypes.byref(g)) == gr.EUNSUPPORTED
    assert lib.gemm_relu_default_order(0, -1, 64, ctypes.byref(o), ctypes.byref(g)) == gr.EINVAL
    assert lib.gemm_relu_default_order(0, 64, 64, None, ctypes.byref(g)) == gr.EINVAL
    assert lib.gemm_relu_default_order(0, 64, 64, ctypes.byref(o), None) == gr.EINVAL
    assert (o.value, g.value) == (7, 7)


def test_timing_rotation_covers_the_last_level_cache():
    from tiled_dense_gemm_f16_amd import tune

    MiB = 1 << 20
    # 4096^3: 64 MiB of inputs, 12 copies fit in one graph of 20
    assert tune.rotation(64 * MiB, 20) == 12
    # 1024^3: 4 MiB; 192 copies, rounded up to 10 graphs of 20
    assert tune.rotation(4 * MiB, 20) == 200
    assert tune.rotation(4 * MiB, 0) == 192
    # every copy count covers 768 MiB, up to the cap (then whole graphs past it)
    for in_bytes in (1, 3 * MiB + 5, 100 * MiB, 800 * MiB):
        for batch in (0, 10, 20):
            n = tune.rotation(in_bytes, batch)
            assert n >= tune.MAX_COPIES or n * in_bytes >= tune.DEFAULT_ROTATE_BYTES
            assert batch == 0 or n <= batch or n % batch == 0

    # the graphs cycle once through every copy, in order
    class FakeGraph:
        log = []

        def __enter__(self):
            FakeGraph.log.append([])

        def __exit__(self, *a):
            return False

    import types
    fake_torch = types.SimpleNamespace(cuda=types.SimpleNamespace(CUDAGraph=object, graph=lambda g, stream: FakeGraph()))
    saved = sys.modules.get("torch")
    sys.modules["torch"] = fake_torch
    try:
        gs = tune.capture_rotation(lambda i: FakeGraph.log[-1].append(i), 60, 20, None)
    finally:
        if saved is not None:
            sys.modules["torch"] = saved
    assert len(gs) == 3 and FakeGraph.log == [list(range(0, 20)), list(range(20, 40)), list(range(40, 60))]


def test_tuner_table_roundtrip(tmp_path):
    from tiled_dense_gemm_f16_amd import tune

    path = str(tmp_path / "tuned.json")
    res = {"shape": [64, 128, 256], "epilogue": "relu", "arch": "gfx950",
           "results": [{"ok": True}], "best": {"tile": 2, "tile_name": gr.tile_name(2), "block_order": 0,
                                             "group_m": 2, "us": 3.0}}
    tune.save(res, path)
    assert tune.lookup(path, "gfx950", "relu", 64, 128, 256) == {"tile": 2, "block_order": 0, "group_m": 2}
    assert tune.lookup(path, "gfx950", "bias_gelu", 64, 128, 256) is None
    assert tune.lookup(path, "gfx942", "relu", 64, 128, 256) is None
    # an entry whose tile id now names a different kernel is not applied
    res["best"]["tile_name"] = "no-such-tile"
    res["shape"] = [1, 2, 3]
    tune.save(res, path)
    assert tune.lookup(path, "gfx950", "relu", 1, 2, 3) is None


FAKE = 0x10000  # never dereferenced: these calls must fail validation first


@pytest.mark.parametrize("M,N,K", [(-1, 4, 4), (4, -1, 4), (4, 4, -1)])
def test_negative_sizes_rejected(M, N, K):
    assert gr.gemm_relu_f16(M, N, K, FAKE, FAKE * 2, FAKE * 3) == gr.EINVAL


def test_null_pointers_rejected():
    assert gr.gemm_relu_f16(4, 4, 4, 0, FAKE, FAKE * 3) == gr.EINVAL
    assert gr.gemm_relu_f16(4, 4, 4, FAKE, 0, FAKE * 3) == gr.EINVAL
    assert gr.gemm_relu_f16(4, 4, 4, FAKE, FAKE * 2, 0) == gr.EINVAL


def test_oversized_and_misaligned_rejected():
    assert gr.gemm_relu_f16(2 ** 31, 4, 4, FAKE, FAKE * 2, FAKE * 3) == gr.EUNSUPPORTED
    assert gr.gemm_relu_f16(4, 4, 4, FAKE + 1, FAKE * 2, FAKE * 3) == gr.EUNSUPPORTED


def test_overlap_rejected():
    # C overlapping A (4x4 fp16 = 32 bytes)
    assert gr.gemm_relu_f16(4, 4, 4, FAKE, FAKE * 2, FAKE + 16) == gr.EINVAL
    assert gr.gemm_relu_f16(4, 4, 4, FAKE, FAKE * 2, FAKE * 2 - 16) == gr.EINVAL


def test_bad_opts_rejected():
    o = gr.make_opts(tile=gr.tile_count())
    assert gr.gemm_relu_f16_ex(4, 4, 4, FAKE, FAKE * 2, FAKE * 3, 0, o) == gr.EUNSUPPORTED
    o = gr.make_opts(block_order=7)
    assert gr.gemm_relu_f16_ex(4, 4, 4, FAKE, FAKE * 2, FAKE * 3, 0, o) == gr.EINVAL
    o = gr.make_opts()
    o.reserved[2] = 1
    assert gr.gemm_relu_f16_ex(4, 4, 4, FAKE, FAKE * 2, FAKE * 3, 0, o) == gr.EINVAL


def test_bias_gelu_arguments_rejected():
    # no bias with columns to write, an odd bias address, a bias overlapping C
    assert gr.gemm_bias_gelu_f16(4, 4, 4, FAKE, FAKE * 2, 0, FAKE * 3) == gr.EINVAL
    assert gr.gemm_bias_gelu_f16(4, 4, 4, FAKE, FAKE * 2, FAKE * 4 + 1, FAKE * 3) == gr.EUNSUPPORTED
    assert gr.gemm_bias_gelu_f16(4, 4, 4, FAKE, FAKE * 2, FAKE * 3 + 8, FAKE * 3) == gr.EINVAL
    assert gr.gemm_bias_gelu_f16(-1, 4, 4, FAKE, FAKE * 2, FAKE * 4, FAKE * 3) == gr.EINVAL
    # nothing to write: a no-op without touching the device
    assert gr.gemm_bias_gelu_f16(0, 5, 5, 0, FAKE, FAKE * 4, 0) == gr.OK


def test_transposed_operand_arguments():
    # op values other than N (0) and T (1) are rejected before any HIP call
    for op_a, op_b in ((2, 0), (0, -1), (7, 7)):
        assert gr.gemm_relu_f16_op(4, 4, 4, FAKE, op_a, FAKE * 2, op_b, FAKE * 3) == gr.EINVAL
        assert gr.gemm_bias_gelu_f16_op(4, 4, 4, FAKE, op_a, FAKE * 2, op_b, FAKE * 4, FAKE * 3) == gr.EINVAL
    # the usual checks apply to every layout
    for op_a in (gr.OP_N, gr.OP_T):
        for op_b in (gr.OP_N, gr.OP_T):
            assert gr.gemm_relu_f16_op(-1, 4, 4, FAKE, op_a, FAKE * 2, op_b, FAKE * 3) == gr.EINVAL
            assert gr.gemm_relu_f16_op(4, 4, 4, 0, op_a, FAKE * 2, op_b, FAKE * 3) == gr.EINVAL
            assert gr.gemm_relu_f16_op(4, 4, 4, FAKE, op_a, FAKE * 2, op_b, FAKE * 3 + 1) == gr.EUNSUPPORTED
            assert gr.gemm_relu_f16_op(0, 4, 4, 0, op_a, FAKE, op_b, 0) == gr.OK
    # the vector kernels need the stored leading dimensions to be multiples of
    # 8: K or M for A, N or K for B, and N for C
    assert gr.select_tile(60, 64, 64) >= 0
    assert gr.select_tile(60, 64, 64, trans_a=True) == -1
    assert gr.select_tile(64, 64, 60) == -1  # A's leading dimension is K
    assert gr.select_tile(64, 64, 60, trans_a=True) >= 0  # neither stored operand has K as leading dimension
    assert gr.select_tile(64, 64, 60, trans_a=True, trans_b=True) == -1  # B's is
    assert gr.select_tile(64, 60, 64, trans_b=True) == -1
    assert gr.select_tile(64, 64, 64, trans_a=True, trans_b=True) >= 0
    assert gr.load().gemm_relu_select_tile_op(64, 64, 64, 3, 0, None, None, None) == -1


def test_python_wrapper_shapes_with_transposes():
    import torch
    a = torch.zeros(6, 4, dtype=torch.float16)   # stored K x M with trans_a: M = 4, K = 6
    b = torch.zeros(5, 6, dtype=torch.float16)   # stored N x K with trans_b: K = 6
    with pytest.raises(ValueError, match="do not chain"):
        gr.gemm_relu(a, b)
    with pytest.raises(ValueError, match="do not chain"):
        gr.gemm_relu(a, b, trans_a=True)
    with pytest.raises(ValueError, match="same GPU"):  # shapes chain; CPU tensors are not device memory
        gr.gemm_relu(a, b, trans_a=True, trans_b=True)


def test_softmax_arguments_rejected():
    assert gr.softmax_rows_f16(-1, 4, FAKE, FAKE * 2) == gr.EINVAL
    assert gr.softmax_rows_f16(4, 4, 0, FAKE * 2) == gr.EINVAL
    assert gr.softmax_rows_f16(4, 4, FAKE + 1, FAKE * 2) == gr.EUNSUPPORTED
    assert gr.softmax_rows_f16(4, 4, FAKE, FAKE + 8) == gr.EINVAL  # partial overlap
    assert gr.softmax_rows_f16(2 ** 31, 4, FAKE, FAKE * 2) == gr.EUNSUPPORTED
    assert gr.softmax_rows_f16(0, 4, 0, 0) == gr.OK


def test_attention_arguments_rejected():
    f = gr.flash_attn_fwd_f16
    Q, K, V, O = FAKE, FAKE * 4, FAKE * 8, FAKE * 12
    assert f(-1, 1, 4, 4, 64, Q, K, V, O, 0, 0.1, 0) == gr.EINVAL
    assert f(1, 1, 4, 4, 64, Q, K, V, O, 0, 0.1, 2) == gr.EINVAL      # causal must be 0 or 1
    assert f(1, 1, 4, 4, 96, Q, K, V, O, 0, 0.1, 0) == gr.EUNSUPPORTED  # head dimension
    assert f(1, 1, 4, 4, 64, 0, K, V, O, 0, 0.1, 0) == gr.EINVAL
    assert f(1, 1, 4, 4, 64, Q + 8, K, V, O, 0, 0.1, 0) == gr.EUNSUPPORTED  # 16-byte alignment
    assert f(1, 1, 4, 4, 64, Q, K, V, O, FAKE * 16 + 2, 0.1, 0) == gr.EUNSUPPORTED  # lse alignment
    assert f(1, 1, 4, 4, 64, Q, K, V, Q, 0, 0.1, 0) == gr.EINVAL       # O overlaps Q
    assert f(1, 1, 2 ** 24, 4, 64, Q, K, V, O, 0, 0.1, 0) == gr.EUNSUPPORTED  # in-head offsets
    assert f(1, 1, 0, 4, 64, 0, K, V, 0, 0, 0.1, 0) == gr.OK            # nothing to write
    assert f(1, 1, 4, 4, 64, Q, K, V, O, 0, float("inf"), 0) == gr.EINVAL
    assert f(1, 1, 4, 4, 64, Q, K, V, O, 0, float("nan"), 0) == gr.EINVAL
    # scales whose scaled scores could overflow fp32 are refused, before any HIP call
    assert f(1, 1, 4, 4, 64, Q, K, V, O, 0, 1e30, 0) == gr.EUNSUPPORTED
    assert f(1, 1, 4, 4, 64, Q, K, V, O, 0, -3e38, 1) == gr.EUNSUPPORTED
    assert f(1, 1, 4, 4, 64, Q, K, V, O, 0, 2.0 ** 65, 0) == gr.EUNSUPPORTED


def test_empty_output_is_a_no_op():
    # M == 0 or N == 0: success without touching the device (NULL is fine then)
    assert gr.gemm_relu_f16(0, 5, 5, 0, FAKE, 0) == gr.OK
    assert gr.gemm_relu_f16(5, 0, 5, FAKE, 0, 0) == gr.OK


def test_python_wrapper_rejects_bad_tensors():
    import torch
    a = torch.zeros(4, 4, dtype=torch.float16)
    with pytest.raises((TypeError, ValueError)):
        gr.gemm_relu(a.float(), a)
    with pytest.raises(ValueError):
        gr.gemm_relu(a, torch.zeros(5, 4, dtype=torch.float16))
    with pytest.raises(ValueError):  # CPU tensors are not device memory
        gr.gemm_relu(a, a)


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "tiled_dense_gemm_f16_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".hpp", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_noalloc_refuses_oversized_scratch_before_any_hip_call():
    # 32 rows over 33 tiles of 32 x 128: 4 splits, 2.03 MiB of partial sums,
    # more than the fixed array holds; refused before the device is touched
    F = 1 << 32  # never dereferenced
    assert gr.tile_name(gr.select_tile(32, 4160, 8192)).startswith("splitk_32x128")
    assert 4 * 32 * 4160 * 4 > gr.NOALLOC_MAX_PARTIAL_BYTES
    assert gr.gemm_relu_f16_noalloc(32, 4160, 8192, F, 2 * F, 3 * F, 0) == gr.ETOOBIG
    assert "scratch" in gr.strerror(gr.ETOOBIG)
    # the same argument checks as gemm_relu_f16
    assert gr.gemm_relu_f16_noalloc(-1, 8, 8, F, 2 * F, 3 * F, 0) == gr.EINVAL
    assert gr.gemm_relu_f16_noalloc(8, 8, 8, 0, 2 * F, 3 * F, 0) == gr.EINVAL
    assert gr.gemm_relu_f16_noalloc(8, 8, 8, F + 1, 2 * F, 3 * F, 0) == gr.EUNSUPPORTED
    assert gr.gemm_relu_f16_noalloc(8, 8, 8, F, 2 * F, F, 0) == gr.EINVAL   # C overlaps A
    assert gr.gemm_relu_f16_noalloc(0, 8, 0, 0, 0, 0, 0) == gr.OK          # empty: no launch


def test_noalloc_scratch_is_a_fixed_device_array():
    # the array lives in the code object (a device symbol), not in a
    # runtime allocation
    out = subprocess.run(["nm", "-C", gr.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert any("scratch" in line for line in out.splitlines())
    src = open(os.path.join(os.path.dirname(gr.LIB_PATH), "csrc", "gemm_relu.hip")).read()
    assert "static __device__ __align__(256) char scratch[" in src
    assert "hipGetSymbolAddress" in src


def test_ordinary_build_has_no_timestamp_hook():
    # the per-workgroup timestamps exist only in the profiling build
    out = subprocess.run(["nm", "-D", "--defined-only", gr.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "gemm_relu_stamps_set" not in out


def test_stamps_summary_on_synthetic_rows():
    import numpy as np
    from tiled_dense_gemm_f16_amd import stamps
    # two dies, two workgroups each: start, first data, loop end, end (100 MHz ticks), -, die
    rows = np.array([[1000, 1100, 1500, 1600, 0, 0, 0, 0],
                     [1002, 1104, 1510, 1620, 0, 0, 0, 0],
                     [1001, 1101, 1520, 1700, 0, 1, 0, 0],
                     [1003, 1103, 1530, 1650, 0, 1, 0, 0],
                     [0, 0, 0, 0, 0, 0, 0, 0]], dtype=np.int64)  # a row nothing wrote
    s = stamps.summarise(rows)
    assert s["workgroups"] == 4 and s["span_ns"] == 7000
    assert s["first_data_after_start_ns"][0] == 1000 and s["main_loop_ns"][2] == 4270
    assert [d["die"] for d in s["per_die"]] == [0, 1] and s["per_die"][1]["end_ns_max"] == 7000
