"""Where a launch's time goes, workgroup by workgroup (profiling tool).

Runs the timestamp build of the library (``python -m
tiled_dense_gemm_f16_amd.build --stamps`` writes libgemm_relu_stamps.so), in
which the pipelined, small-tile and split-K kernels record the GPU's 100 MHz
realtime counter at their start, when the first tile's data has arrived, at
the end of the main loop and when the last store is acknowledged (split-K
workgroups also after counting their partial sums), with the die each
workgroup ran on. The launches are replayed back to back from a HIP graph, as
the benchmark times them, and the stamps of the last one are summarised per
die:

    python -m tiled_dense_gemm_f16_amd.stamps --workload gemm_relu_f16_1024x1024x1024_normal

Only this tool loads the timestamp build; the library and its tests never do.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

from . import _binding
from .build import STAMPS_LIB

WORDS = 8  # kStampWords


def load(path: str = STAMPS_LIB):
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with python -m tiled_dense_gemm_f16_amd.build --stamps")
    lib = ctypes.CDLL(path)
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.gemm_relu_stamps_set.argtypes = [p, i64]
    lib.gemm_relu_stamps_set.restype = i32
    lib.gemm_relu_f16_ex.argtypes = [i64, i64, i64, p, p, p, p, ctypes.POINTER(_binding.Opts)]
    lib.gemm_relu_f16_ex.restype = i32
    return lib


def summarise(t: np.ndarray) -> dict:
    """Per-die and overall phase times (ns) from one launch's stamp rows."""
    ok = t[:, 0] > 0
    t = t[ok]
    t0 = int(t[:, 0].min())
    ns = lambda col: (t[:, col].astype(np.int64) - t0) * 10  # noqa: E731
    start, first, loop_end, end = ns(0), ns(1), ns(2), ns(3)
    q = lambda x: [int(v) for v in np.percentile(x, [0, 50, 100])]  # noqa: E731
    out = {"workgroups": int(ok.sum()), "span_ns": int(end.max()),
           "start_ns": q(start), "first_data_after_start_ns": q(first - start),
           "main_loop_ns": q(loop_end - first), "after_loop_ns": q(end - loop_end), "end_ns": q(end),
           "per_die": []}
    if (t[:, 4] > 0).any():
        counted = ns(4)
        out["partials_counted_after_loop_ns"] = q(counted - loop_end)
    for x in sorted(set(int(v) for v in t[:, 5])):
        m = t[:, 5] == x
        out["per_die"].append({"die": x, "workgroups": int(m.sum()), "start_ns": int(np.median(start[m])),
                               "loop_end_ns": int(np.median(loop_end[m])), "end_ns_max": int(end[m].max())})
    return out


def main(argv=None) -> int:
    import torch

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import workloads

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default=workloads.SQUARE_1024.name, choices=sorted(workloads.BY_NAME))
    ap.add_argument("--tile", type=int, default=None)
    ap.add_argument("--launches", type=int, default=20, help="launches per graph replay")
    ap.add_argument("--rotate", type=int, default=1, help="input copies the launches cycle through")
    ap.add_argument("--json", default=None)
    args = ap.parse_args(argv)
    lib = load()
    w = workloads.BY_NAME[args.workload]
    a, b = workloads.workload_inputs(w)
    ads = [a.cuda() for _ in range(args.rotate)]
    bds = [b.cuda() for _ in range(args.rotate)]
    c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    max_wg = 1 << 16
    buf = torch.zeros(max_wg * WORDS, dtype=torch.int64, device="cuda")
    if lib.gemm_relu_stamps_set(buf.data_ptr(), max_wg) != 0:
        raise RuntimeError("gemm_relu_stamps_set failed")
    opts = _binding.make_opts(args.tile)
    s = torch.cuda.Stream()

    def call(i):
        st = lib.gemm_relu_f16_ex(w.M, w.N, w.K, ads[i].data_ptr(), bds[i].data_ptr(), c.data_ptr(), s.cuda_stream,
                                  ctypes.byref(opts))
        if st != 0:
            raise RuntimeError(f"launch refused: status {st}")

    with torch.cuda.stream(s):
        for i in range(args.rotate):
            call(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(args.launches):
                call(i % args.rotate)
        for _ in range(20):
            g.replay()
        buf.zero_()
        g.replay()
        torch.cuda.synchronize()
    lib.gemm_relu_stamps_set(None, 0)
    rows = buf.view(max_wg, WORDS).cpu().numpy()
    rows = rows[rows[:, 0] > 0]
    res = {"workload": w.name, "tile": _binding.tile_name(args.tile) if args.tile is not None else "auto",
           "launches_per_replay": args.launches, "input_copies": args.rotate, **summarise(rows)}
    print(json.dumps(res), flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
