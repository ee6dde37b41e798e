"""Offline tile sweep: which compiled configuration is fastest for a shape.

The pages' tuner ("Writing high-performance kernels in TileLang", sections
"GEMM con Tensor Cores y decisiones que cambian la velocidad" and "El ajuste
automático encuentra configuraciones específicas para cada GPU") enumerates
tile sizes, the K depth of a step, the pipeline depth and the thread count,
drops the configurations that do not fit the shared-memory budget, then runs,
times and validates each on the GEMM at hand and keeps the winner, so that the
search is not repeated. Here the kernels are compiled ahead of time for
gfx950, so the candidates are the library's compiled tiles (their parameters
come from gemm_relu_tile_info) crossed with the launch-order choices of
gemm_relu_opts: the group size of the XCD-aware grouped block order, and the
plain row-major order. The LDS budget is enforced when the library is
compiled; it is checked again here against the device's LDS per workgroup.

Each candidate's output is validated by a caller-supplied checker (`check`),
which receives the candidate's C and the inputs as fp16 bit patterns on the
host and returns the number of elements it rejects; the test suite passes
one built on its independent CPU reference. Without a checker the candidates are only
checked for agreement with the library's default launch, within the
contract's bound |c - ref| <= 1e-2 + 1e-2 |ref| (numpy on the host): that
catches a broken tile, not a fault every tile shares. The package itself
computes no reference product. It is timed as replays of HIP graphs of `graph` launches that
together cycle through copies of the inputs (at least `rotate_bytes` in all,
at most MAX_COPIES copies), so inputs come from HBM rather than the
last-level cache. The winners go into a
JSON table keyed by device architecture, epilogue and shape; `lookup` returns
the keyword arguments that pin the winner in gemm_relu / gemm_bias_gelu.

Usage: python -m tiled_dense_gemm_f16_amd.tune 4096x4096x4096 [MxNxK ...]
           [--epilogue relu|bias_gelu] [--table tuned.json]
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

from . import _binding as gr

LDS_PER_WORKGROUP = 160 * 1024  # gfx950
GROUP_SIZES = (1, 2, 4, 8, 16)
DEFAULT_ROTATE_BYTES = 768 << 20  # three times the 256 MB last-level cache
MAX_COPIES = 4096


def rotation(in_bytes: int, batch: int, rotate_bytes: int = DEFAULT_ROTATE_BYTES) -> int:
    """Number of input copies a timing loop cycles through so that a launch's
    inputs were last touched at least `rotate_bytes` of other inputs ago (at
    most MAX_COPIES). With graphs of `batch` launches and more copies than
    that, the count is rounded up to a whole number of graphs."""
    n = max(1, min(MAX_COPIES, -(-rotate_bytes // max(in_bytes, 1))))
    if batch > 0 and n > batch:
        n = -(-n // batch) * batch
    return n


def capture_rotation(call, copies: int, batch: int, stream) -> list:
    """HIP graphs of `batch` launches of call(copy) that, replayed in turn,
    cycle through all `copies`: graph j runs copies j * batch .. j * batch +
    batch - 1 (modulo copies), ceil(copies / batch) graphs (one when copies
    <= batch; exactly once through when copies is a multiple of batch, as
    rotation() makes it). Nothing is allocated inside the graphs."""
    import torch

    graphs = []
    for j in range(-(-copies // batch) if copies > batch else 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(batch):
                st = call((j * batch + i) % copies)
                # a refused call records nothing: the graph would time an
                # empty launch, so fail instead
                if st is not None and st != gr.OK:
                    raise RuntimeError(f"call refused while capturing a graph: {gr.strerror(st)}")
        graphs.append(g)
    return graphs


def _tiles(M: int, N: int, bm: int, bn: int) -> tuple[int, int]:
    return -(-M // bm), -(-N // bn)


def candidates(M: int, N: int, K: int, lds_limit: int = LDS_PER_WORKGROUP) -> list[dict]:
    """Every (tile, block order, group size) the library can launch for this
    shape, minus tiles over the LDS budget. The block order only matters when
    the grid has several tile-rows and tile-columns, so other grids get the
    default order alone."""
    out = []
    for t in range(gr.tile_count()):
        d = gr.tile_info(t)
        if d["lds_bytes"] > lds_limit:
            continue
        base = {"tile": t, "tile_name": gr.tile_name(t), "block_order": gr.ORDER_DEFAULT, "group_m": 0}
        tm, tn = _tiles(M, N, d["bm"], d["bn"])
        if d["split_k"] or tm < 2 or tn < 2:
            out.append(base)
            continue
        # the library's own group (clamped to the tile-rows) is always a candidate
        for g in sorted({g for g in GROUP_SIZES if g <= tm} | {gr.default_order(t, M, N)[1]}):
            out.append(dict(base, group_m=g))
        out.append(dict(base, block_order=gr.ORDER_ROW_MAJOR))
    return out


def _inputs(M, N, K, epilogue, seed, device, copies, trans_a=False, trans_b=False):
    """Seeded inputs in their stored layouts (A as K x M with trans_a, B as
    N x K with trans_b)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    a = torch.randn((K, M) if trans_a else (M, K), generator=gen, device=device, dtype=torch.float32).half()
    b = torch.randn((N, K) if trans_b else (K, N), generator=gen, device=device, dtype=torch.float32).half()
    bias = None
    if epilogue == "bias_gelu":
        bias = (torch.randn((N,), generator=gen, device=device, dtype=torch.float32) * K ** 0.5).half()
    a_s = [a] + [a.clone() for _ in range(copies - 1)]
    b_s = [b] + [b.clone() for _ in range(copies - 1)]
    return a_s, b_s, bias


def _host_bits(t) -> np.ndarray:
    """A device fp16 tensor's bit patterns, copied to the host."""
    import torch

    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def agreement_check(ref_bits: np.ndarray):
    """A checker that accepts outputs within 1e-2 + 1e-2 |ref| of `ref_bits`
    (fp16 bit patterns) element by element."""
    r = ref_bits.view(np.float16).astype(np.float64)

    def check(c_bits: np.ndarray, *_inputs) -> int:
        g = c_bits.view(np.float16).astype(np.float64)
        return int((~(np.abs(g - r) <= 1e-2 + 1e-2 * np.abs(r))).sum())

    return check


def tune(M: int, N: int, K: int, *, epilogue: str = "relu", seed: int = 0, graph: int = 20,
         replays: int = 5, rotate_bytes: int = DEFAULT_ROTATE_BYTES, device: int = 0,
         only: list[dict] | None = None, trans_a: bool = False, trans_b: bool = False,
         check=None) -> dict:
    """Validates and times every candidate for (M, N, K) with the operand
    layouts trans_a / trans_b (A stored K x M, B stored N x K); returns
    {"shape", "epilogue", "layout", "arch", "results": [...] fastest first, "best"}.
    Candidates whose output fails validation or whose call fails are kept in
    the results with "ok": False and never chosen.

    check(c_bits, a_bits, b_bits, bias_bits) -> number of rejected elements,
    all arguments fp16 bit patterns (numpy uint16) on the host, A and B in
    their stored layouts, bias None for the ReLU epilogue. None: agreement
    with the library's default launch (see the module docstring)."""
    import torch

    if epilogue not in ("relu", "bias_gelu"):
        raise ValueError(f"unknown epilogue {epilogue!r}")
    if M <= 0 or N <= 0:
        raise ValueError("M and N must be positive")
    dev = torch.device("cuda", device)
    in_bytes = 2 * (M * K + K * N)
    copies = rotation(in_bytes, graph, rotate_bytes)
    cands = only if only is not None else candidates(M, N, K)
    with torch.cuda.device(dev):
        a_s, b_s, bias = _inputs(M, N, K, epilogue, seed, dev, copies, trans_a, trans_b)
        c = torch.empty((M, N), dtype=torch.float16, device=dev)
        stream = torch.cuda.Stream(dev)
        host_in = (_host_bits(a_s[0]), _host_bits(b_s[0]), None if bias is None else _host_bits(bias))
        if check is None:
            # the library's default launch is the reference of the others
            def default_call():
                if epilogue == "bias_gelu":
                    return gr.gemm_bias_gelu_f16_op(M, N, K, a_s[0].data_ptr(), int(trans_a), b_s[0].data_ptr(),
                                                    int(trans_b), bias.data_ptr(), c.data_ptr(), stream.cuda_stream,
                                                    None)
                return gr.gemm_relu_f16_op(M, N, K, a_s[0].data_ptr(), int(trans_a), b_s[0].data_ptr(),
                                           int(trans_b), c.data_ptr(), stream.cuda_stream, None)
            with torch.cuda.stream(stream):
                st = default_call()
                stream.synchronize()
            if st != gr.OK:
                raise RuntimeError(f"the default launch failed: {gr.strerror(st)}")
            check = agreement_check(_host_bits(c))
        results = []
        for cand in cands:
            opts = gr.make_opts(cand["tile"], cand["block_order"], cand["group_m"])

            def call(i, opts=opts):
                if epilogue == "bias_gelu":
                    return gr.gemm_bias_gelu_f16_op(M, N, K, a_s[i].data_ptr(), int(trans_a), b_s[i].data_ptr(),
                                                    int(trans_b), bias.data_ptr(), c.data_ptr(), stream.cuda_stream,
                                                    opts)
                return gr.gemm_relu_f16_op(M, N, K, a_s[i].data_ptr(), int(trans_a), b_s[i].data_ptr(), int(trans_b),
                                           c.data_ptr(), stream.cuda_stream, opts)

            res = dict(cand)
            torch.cuda.synchronize(dev)
            with torch.cuda.stream(stream):
                c.fill_(float("nan"))
                st = call(0)
                stream.synchronize()
                if st != gr.OK:
                    results.append(dict(res, ok=False, error=gr.strerror(st)))
                    continue
                bad = int(check(_host_bits(c), *host_in))
                res["violations"] = bad
                if bad:
                    results.append(dict(res, ok=False, error=f"{bad} elements outside 1e-2 + 1e-2|ref|"))
                    continue
                for i in range(3):
                    call(i % copies)
                stream.synchronize()
                gs = capture_rotation(call, copies, graph, stream)
                for g in gs:  # every copy once before timing
                    g.replay()
                times = []
                for r in range(max(replays, len(gs))):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    gs[r % len(gs)].replay()
                    e1.record(stream)
                    e1.synchronize()
                    times.append(e0.elapsed_time(e1) * 1e3 / graph)
                del gs
            times.sort()
            res.update(ok=True, us=times[len(times) // 2], us_min=times[0])
            results.append(res)
    results.sort(key=lambda r: (not r["ok"], r.get("us", float("inf"))))
    best = results[0] if results and results[0]["ok"] else None
    arch = torch.cuda.get_device_properties(dev).gcnArchName.split(":")[0]
    layout = ("t" if trans_a else "n") + ("t" if trans_b else "n")
    return {"shape": [M, N, K], "epilogue": epilogue, "layout": layout, "arch": arch, "copies": copies,
            "graph": graph, "results": results, "best": best,
            "default": _default_of(M, N, K, results, trans_a, trans_b)}


def _default_of(M, N, K, results, trans_a=False, trans_b=False):
    """The result of the launch the library makes without opts, if it was timed."""
    auto = gr.select_tile(M, N, K, trans_a=trans_a, trans_b=trans_b)
    if auto < 0:
        return None
    order, g = gr.default_order(auto, M, N)
    for r in results:
        if r["tile"] != auto:
            continue
        if r["block_order"] == order == gr.ORDER_ROW_MAJOR:
            return r
        if r["block_order"] == order == gr.ORDER_DEFAULT and r["group_m"] in (0, g):
            return r
    return None


def _key(arch: str, epilogue: str, M: int, N: int, K: int, layout: str = "nn") -> str:
    return f"{arch}/{epilogue}/{M}x{N}x{K}" + ("" if layout == "nn" else f"/{layout}")


def save(result: dict, path: str) -> None:
    """Adds (or replaces) the winner of `result` in the JSON table at `path`."""
    table = {}
    if os.path.exists(path):
        with open(path) as f:
            table = json.load(f)
    if result["best"] is None:
        raise ValueError("no candidate passed validation")
    b = result["best"]
    table[_key(result["arch"], result["epilogue"], *result["shape"], result.get("layout", "nn"))] = {
        "tile": b["tile"], "tile_name": b["tile_name"], "block_order": b["block_order"], "group_m": b["group_m"],
        "us": round(b["us"], 3), "candidates": len(result["results"])}
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    os.replace(tmp, path)


def lookup(path: str, arch: str, epilogue: str, M: int, N: int, K: int, layout: str = "nn") -> dict | None:
    """Keyword arguments (tile, block_order, group_m) of the stored winner, or
    None. The tile is checked by name, so a table written for another build
    of the library is not applied to different kernels."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        e = json.load(f).get(_key(arch, epilogue, M, N, K, layout))
    if e is None or not (0 <= e["tile"] < gr.tile_count()) or gr.tile_name(e["tile"]) != e["tile_name"]:
        return None
    return {"tile": e["tile"], "block_order": e["block_order"], "group_m": e["group_m"]}


def format_result(r: dict, top: int = 0) -> str:
    M, N, K = r["shape"]
    lay = r.get("layout", "nn")
    auto = gr.select_tile(M, N, K, trans_a=lay[0] == "t", trans_b=lay[1] == "t")
    lines = [f"{r['epilogue']} {lay} {M}x{N}x{K} on {r['arch']}: {len(r['results'])} candidates, "
             f"{r['copies']} input copies, graphs of {r['graph']}; library default tile {auto} "
             f"({gr.tile_name(auto) if auto >= 0 else 'generic'})"]
    d, b = r.get("default"), r["best"]
    if d is not None and d.get("ok") and b is not None:
        lines.append(f"  best {b['us']:.2f} us; library default {d['us']:.2f} us "
                     f"({d['us'] / b['us']:.3f}x the best)")
    rows = r["results"][:top] if top else r["results"]
    for x in rows:
        order = "row-major" if x["block_order"] == gr.ORDER_ROW_MAJOR else f"grouped g={x['group_m'] or 'def'}"
        if x["ok"]:
            lines.append(f"  {x['us']:10.2f} us (min {x['us_min']:.2f})  tile {x['tile']:2d} {x['tile_name']:42s} {order}")
        else:
            lines.append(f"  {'failed':>10s}     tile {x['tile']:2d} {x['tile_name']:42s} {order}: {x['error']}")
    return "\n".join(lines)


def _shape(s: str) -> tuple[int, int, int]:
    parts = s.lower().split("x")
    if len(parts) != 3:
        raise argparse.ArgumentTypeError(f"shape {s!r} is not MxNxK")
    return tuple(int(p) for p in parts)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description="time and validate every compiled tile on the given shapes")
    ap.add_argument("shapes", nargs="+", type=_shape, metavar="MxNxK")
    ap.add_argument("--epilogue", choices=("relu", "bias_gelu"), default="relu")
    ap.add_argument("--layout", choices=("nn", "nt", "tn", "tt"), default="nn",
                    help="A stored K x M (t first) and/or B stored N x K (t second)")
    ap.add_argument("--table", default=None, help="JSON table to add the winners to")
    ap.add_argument("--graph", type=int, default=20)
    ap.add_argument("--replays", type=int, default=5)
    ap.add_argument("--top", type=int, default=0, help="print only the fastest N candidates")
    ap.add_argument("--json", default=None, help="write every result to this file")
    args = ap.parse_args(argv)
    everything = []
    for M, N, K in args.shapes:
        r = tune(M, N, K, epilogue=args.epilogue, graph=args.graph, replays=args.replays,
                 trans_a=args.layout[0] == "t", trans_b=args.layout[1] == "t")
        print(format_result(r, args.top), flush=True)
        everything.append(r)
        if args.table and r["best"] is not None:
            save(r, args.table)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(everything, f, indent=1)
    return 0 if all(r["best"] is not None for r in everything) else 1


if __name__ == "__main__":
    sys.exit(main())
