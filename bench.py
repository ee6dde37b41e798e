"""Throughput of C = ReLU(A @ B) (fp16 in, fp32 accumulate, fp16 out) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--graph G] [--no-cpu-baseline]

A step is one call of gemm_relu_f16 on one batch of synthetic input that is
already resident in HBM: the whole hot path (tile loads, MFMA main loop, ReLU,
fp16 store) in one kernel. Exactly K timed steps follow the untimed warm-up,
bracketed by stream synchronisation; the calls are captured min(G, K) at a
time into HIP graphs and replayed (--graph 0 launches them one by one). The
warm-up runs the same work back to back for at least W launches and at least
--steady-ms milliseconds, so that the timed region sees the clock the chip
settles at under this load; the shader clock is sampled and reported with the
device's name and architecture. The line printed on stdout is one JSON
object. Extra per-workload lines (``--all``) go to stderr.

The CPU baseline leg times the oracle (plain C, all host threads) on a bounded
slice of the same workload -- leading rows of C -- and scales it to TFLOP/s.

    python bench.py --op attention [--batch B --heads H --seq S --head-dim D --causal]
    python bench.py --op softmax [--rows R --cols C]

time the second workload the same way (graph replay, rotated inputs): the
attention forward pass against the fp16 MFMA roofline, the row softmax
against HBM bandwidth; each prints its own JSON line, with the oracle on
sampled rows as its CPU baseline.

    python bench.py --vs-torch [--all]

adds, on stderr, torch.matmul (hipBLASLt, no ReLU) timed the same way on the
same operands, as context.

    python bench.py --sustain SECONDS [--sustain-op gemm|torch|attention]

only runs one operation back to back on fixed inputs and prints its rate each
second: the load under which board power and clocks are read with amd-smi.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

PEAK_FP16_TFLOPS = 2516.6   # MI355X dense fp16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "TFLOP/s and % of MI355X dense FP16 MFMA peak, fp16 GEMM+ReLU 4096³"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
CSRC = os.path.join(ROOT, "tiled_dense_gemm_f16_amd", "csrc")


def kernel_sources(tile: str) -> list[str]:
    """Device sources of the kernel family that runs a tile (or, for the
    second workload, the attention and softmax kernels: "attn_fwd_d128",
    "softmax_rows")."""
    if tile.startswith(("attn", "softmax")):
        # the kernels and their launch configuration (waves per workgroup)
        return [os.path.join(CSRC, "common.hpp"), os.path.join(CSRC, "attention.hpp"),
                os.path.join(CSRC, "attention.hip")]
    family = ("small.hpp" if "lds-small" in tile else "pipelined.hpp" if "lds-dma" in tile
              else "splitk.hpp" if "splitk" in tile else "staged.hpp")
    return [os.path.join(CSRC, "common.hpp"), os.path.join(CSRC, family)]


def source_hash(tile: str) -> str:
    h = hashlib.sha256()
    for p in kernel_sources(tile):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, tile: str, layout: str = "nn", epilogue: str = "relu") -> float | None:
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current source of the kernel that runs `tile`, with the
    same operand layout and epilogue (entries without those keys are "nn" and
    "relu"); otherwise None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    cur = source_hash(tile)
    entries, entry = [], {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, _, v = line.partition(":")
        k, v = k.strip(), v.strip()
        if k == "workload" and entry:
            entries.append(entry)
            entry = {}
        entry[k] = v
    if entry:
        entries.append(entry)
    for e in entries:
        if (e.get("workload") == workload and e.get("tile") == tile and e.get("kernel_source_sha256") == cur
                and e.get("layout", "nn") == layout and e.get("epilogue", "relu") == epilogue):
            try:
                return float(e["traffic_bytes_per_launch"])
            except (KeyError, ValueError):
                return None
    return None


ROTATE_BYTES = 768 << 20  # well above the 256 MB last-level (MALL) cache
STEADY_MS = 500.0         # back-to-back work before the timed region


def _sclk_file() -> str | None:
    """The sysfs file whose line marked '*' is the GPU's current shader clock
    (the only card on a one-GPU machine; else the first that has the file)."""
    import glob
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    return paths[0] if paths else None


class ClockSampler:
    """Samples the current shader clock (MHz) every `period` seconds on a
    thread, with host timestamps, so that the clock the chip held during a
    timed region can be reported next to the time."""

    def __init__(self, period: float = 0.005):
        import threading
        self.path = _sclk_file()
        self.period = period
        self.samples: list[tuple[float, float]] = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self) -> float | None:
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append((time.perf_counter(), v))
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()
        return False

    def summary(self, t0: float, t1: float) -> dict:
        """Median, min and max of the samples taken in [t0, t1] (host clock)."""
        v = sorted(x for t, x in self.samples if t0 <= t <= t1)
        if not v:
            return {"samples": 0, "source": self.path}
        return {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "samples": len(v), "source": self.path}


def _sysfs_device() -> dict:
    """Product name and PCI ids of the card behind the clock file, from sysfs
    (empty where the files are missing)."""
    out = {}
    path = _sclk_file()
    if not path:
        return out
    d = os.path.dirname(path)
    for key, name in (("product_name", "product_name"), ("vendor", "pci_vendor"), ("device", "pci_device")):
        try:
            with open(os.path.join(d, key)) as f:
                v = f.read().strip()
        except OSError:
            continue
        if v:
            out[name] = v
    return out


def device_identity() -> dict:
    import torch
    p = torch.cuda.get_device_properties(0)
    sysfs = _sysfs_device()
    name = torch.cuda.get_device_name(0) or sysfs.get("product_name", "")
    if not name and "pci_device" in sysfs:
        name = f"PCI {sysfs.get('pci_vendor', '?')}:{sysfs['pci_device']}"
    out = {"gpu_name": name, "gfx_arch": p.gcnArchName.split(":")[0],
           "compute_units": p.multi_processor_count, "hbm_gib": round(p.total_memory / 2 ** 30, 1)}
    if "pci_device" in sysfs:
        out["pci_id"] = f"{sysfs.get('pci_vendor', '?')}:{sysfs['pci_device']}"
    return out


def time_launches(calls, steps: int, warmup: int, graph_batch: int, stream, steady_ms: float = STEADY_MS,
                  singles: int = 200) -> dict:
    """Times exactly `steps` launches on `stream`, bracketed by two events on
    that stream (and torch.cuda.synchronize() on both sides). calls[i]() makes
    the launch on input copy i and returns its status.

    * Every copy is called once first, untimed (this creates any split-K
      workspace, so nothing is allocated or cleared inside a graph).
    * With graph_batch = G > 0 the launches are captured min(G, steps) at a
      time into HIP graphs that cycle through the copies, plus one graph for
      the remainder, so the timed region holds exactly `steps` launches
      without the host's per-call cost; G = 0 launches them one by one.
    * Before the timed region the same graphs (or calls) run back to back for
      at least `warmup` launches and at least `steady_ms` milliseconds, so
      that the chip's clock has settled under this load whatever `warmup`
      says; the shader clock is sampled throughout.
    * After it, `singles` launches each between their own pair of events give
      the duration of one launch under the same load."""
    import torch
    from tiled_dense_gemm_f16_amd import tune
    import tiled_dense_gemm_f16_amd as gr

    rot = len(calls)

    def checked(i):
        st = calls[i]()
        if st is not None and st != gr.OK:
            raise RuntimeError(f"launch refused: {gr.strerror(st)}")

    torch.cuda.synchronize()
    with ClockSampler() as clk, torch.cuda.stream(stream):
        for i in range(rot):
            checked(i)
        torch.cuda.synchronize()
        batch = min(graph_batch, steps) if graph_batch > 0 else 0
        if batch:
            graphs = tune.capture_rotation(lambda i: calls[i](), rot, batch, stream)
            rem = steps % batch
            tail = None
            if rem:
                # the remainder: one graph of the first `rem` copies
                tail = tune.capture_rotation(lambda i: calls[i](), min(rot, rem), rem, stream)[0]

            def run_steps():
                for r in range(steps // batch):
                    graphs[r % len(graphs)].replay()
                if tail is not None:
                    tail.replay()

            def warm_chunk(r):
                graphs[r % len(graphs)].replay()
                return batch
        else:
            def run_steps():
                for i in range(steps):
                    calls[i % rot]()

            def warm_chunk(r):
                for i in range(16):
                    calls[(16 * r + i) % rot]()
                return 16
        torch.cuda.synchronize()
        # steady state: the same work back to back, the host kept close
        # behind the device by a synchronisation every few chunks
        tw0 = time.perf_counter()
        done, r = 0, 0
        while done < warmup or (time.perf_counter() - tw0) * 1e3 < steady_ms:
            done += warm_chunk(r)
            r += 1
            if r % 4 == 0:
                stream.synchronize()
        torch.cuda.synchronize()
        tw1 = time.perf_counter()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        t0.record(stream)
        run_steps()
        t1.record(stream)
        torch.cuda.synchronize()
        h1 = time.perf_counter()
        total_ms = t0.elapsed_time(t1)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(singles)]
        for i, (e0, e1) in enumerate(evs):
            e0.record(stream)
            calls[i % rot]()
            e1.record(stream)
        torch.cuda.synchronize()
        h2 = time.perf_counter()
    per = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    timed = clk.summary(h0, h1)
    if timed["samples"] < 3:
        # a short timed region: the clock over the last 100 ms of the same work before it as well
        timed = dict(clk.summary(max(tw0, tw1 - 0.1), h1), window="last 100 ms of warm-up + timed region")
    else:
        timed["window"] = "timed region"
    return {"total_ms": total_ms, "steps": steps, "ms_per_step": total_ms / steps,
            "launch_ms_mean": float(per.mean()), "launch_ms_median": float(np.median(per)),
            "launch_ms_min": float(per.min()), "rotation": rot, "graph_batch": batch,
            "warmup_launches": done, "warmup_ms": round((tw1 - tw0) * 1e3, 1),
            "sclk_mhz": timed, "sclk_mhz_single_launches": clk.summary(h1, h2)}


def time_gpu(w, steps: int, warmup: int, tile=None, graph_batch: int = 0, epilogue: str = "relu",
             layout: str = "nn", rotate_bytes: int = ROTATE_BYTES, steady_ms: float = STEADY_MS):
    """Times `steps` launches of the GEMM on workload w (time_launches).
    Successive launches cycle through R copies of (A, B) with R * (|A| + |B|)
    >= rotate_bytes (at most 4096 copies: the 256^3 shape falls short of
    768 MiB), so with the default the inputs of a launch are not left in the
    256 MB last-level cache by the previous ones: every launch reads its
    inputs from HBM. rotate_bytes = 0 reuses one copy (inputs cached).

    `layout` ("nn", "nt", "tn", "tt") stores A as K x M (t in first place)
    and/or B as N x K (t in second place) and calls the transposed-operand
    entry points; the product is the same."""
    import torch
    import tiled_dense_gemm_f16_amd as gr
    from tiled_dense_gemm_f16_amd import tune

    a, b = workloads.workload_inputs(w)
    ta, tb = layout[0] == "t", layout[1] == "t"
    a_st = a.t().contiguous() if ta else a
    b_st = b.t().contiguous() if tb else b
    in_bytes = 2 * (w.M * w.K + w.K * w.N)
    rot = tune.rotation(in_bytes, min(graph_batch, steps), rotate_bytes) if rotate_bytes > 0 else 1
    ads = [a_st.cuda() for _ in range(rot)]
    bds = [b_st.cuda() for _ in range(rot)]
    c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    stream = torch.cuda.Stream()
    opts = gr.make_opts(tile)
    if epilogue == "bias_gelu":
        # the fused bias + GELU epilogue: a bias on the scale of the sums
        gen = torch.Generator(device="cpu")
        gen.manual_seed(w.seed + 1)
        bias = (torch.randn(w.N, generator=gen) * (w.K ** 0.5) * w.scale * w.scale).half().cuda()
        calls = [lambda i=i: gr.gemm_bias_gelu_f16_op(w.M, w.N, w.K, ads[i].data_ptr(), int(ta), bds[i].data_ptr(),
                                                      int(tb), bias.data_ptr(), c.data_ptr(), stream.cuda_stream, opts)
                 for i in range(rot)]
    else:
        calls = [lambda i=i: gr.gemm_relu_f16_op(w.M, w.N, w.K, ads[i].data_ptr(), int(ta), bds[i].data_ptr(), int(tb),
                                                 c.data_ptr(), stream.cuda_stream, opts) for i in range(rot)]
    r = time_launches(calls, steps, warmup, graph_batch, stream, steady_ms)
    tile_id = (gr.select_tile(w.M, w.N, w.K, ads[0].data_ptr(), bds[0].data_ptr(), c.data_ptr(), trans_a=ta,
                              trans_b=tb) if tile is None else tile)
    r.update({"tile": gr.tile_name(tile_id) if tile_id >= 0 else "generic", "epilogue": epilogue, "layout": layout,
              "c": c, "a": a, "b": b})
    return r


def cpu_baseline(w, gpu_c, target_s: float = 12.0):
    """The oracle as it stands, on leading rows of the same workload."""
    import oracle
    A, B = workloads.as_u16(gpu_c["a"]), workloads.as_u16(gpu_c["b"])
    threads = oracle.num_threads()
    # calibrate on a growing slice until one call takes at least 0.5 s (the
    # first call also pays for starting the thread pool)
    r_cal = min(w.M, max(threads, 8))
    while True:
        t = time.perf_counter()
        oracle.gemm_relu_f16(A, B, rows=(0, r_cal))
        t_cal = time.perf_counter() - t
        if t_cal >= 0.5 or r_cal >= w.M:
            break
        r_cal = min(w.M, r_cal * 4)
    rows = int(min(w.M, max(1, round(r_cal * target_s / max(t_cal, 1e-6)))))
    t = time.perf_counter()
    ora = oracle.gemm_relu_f16(A, B, rows=(0, rows))
    secs = time.perf_counter() - t
    flops = 2.0 * rows * w.N * w.K
    g = workloads.as_u16(gpu_c["c"][:rows].cpu()).view(np.float16).astype(np.float64)
    o = ora.view(np.float16).astype(np.float64)
    err = np.abs(g - o)
    viol = int((~(err <= 1e-2 + 1e-2 * np.abs(o))).sum())
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of C for {w.name} ({rows}x{w.N}x{w.K} multiply-adds, "
                      f"{secs:.1f} s on {threads} threads)",
            "seconds": secs, "parity_of_sample": {"max_abs_err": float(err.max()), "violations": viol}}


def timing_fields(r: dict) -> dict:
    """What every line reports about how its time was taken."""
    ratio = r["ms_per_step"] / r["launch_ms_mean"] if r["launch_ms_mean"] > 0 else None
    return {"graph_batch": r["graph_batch"],
            "single_launch_event_ms": {"mean": round(r["launch_ms_mean"], 5),
                                       "median": round(r.get("launch_ms_median", r["launch_ms_mean"]), 5),
                                       "min": round(r["launch_ms_min"], 5)},
            "timed_over_single_launch_mean": round(ratio, 4) if ratio else None,
            "steady_state": {"warmup_launches": r["warmup_launches"], "warmup_ms": r["warmup_ms"]},
            "sclk_mhz": r["sclk_mhz"], "sclk_mhz_single_launches": r["sclk_mhz_single_launches"],
            "device": device_identity()}


def result_line(w, r, steps, warmup, cpu=None):
    bound = "hbm" if 2 * w.M * w.N * w.K / w.min_bytes < 315 and w.M <= 64 else "mfma"
    value = w.flops / (r["ms_per_step"] * 1e-3) / 1e12
    # one launch per step: the kernel's average duration over the timed region
    launch_s = r["ms_per_step"] * 1e-3
    if bound == "mfma":
        achieved = w.flops / launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4)}
    else:
        achieved = w.min_bytes / launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(w.name, r["tile"], r["layout"], r["epilogue"])
    line = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": r["steps"],
            "warmup": warmup, "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16", "accum_dtype": "f32", "data": "synthetic",
            "pct_of_fp16_peak": round(100 * value / PEAK_FP16_TFLOPS, 2),
            "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "dist": w.dist,
                       "scale": w.scale, "seed": w.seed, "tile": r["tile"], "epilogue": r["epilogue"],
                       "layout": r["layout"],
                       "input_copies_rotated": r["rotation"],
                       "parallelism": "single GPU"},
            "roofline": roof,
            "kernel_ms_timed_region_mean": round(r["ms_per_step"], 5),
            **timing_fields(r),
            "hbm_gbs_at_min_bytes": round(w.min_bytes / (r["ms_per_step"] * 1e-3) / 1e9, 1),
            "kernel_source_sha256": source_hash(r["tile"])}
    if cpu is not None:
        line["cpu_baseline"] = cpu
    return line


def time_calls(calls, steps: int, warmup: int, graph_batch: int, stream) -> dict:
    """The second workload's timing: time_launches over `calls` (one per
    input copy)."""
    return time_launches(calls, steps, warmup, graph_batch, stream)


def cpu_sample(fn, total_rows: int, target_s: float) -> tuple[int, float]:
    """Times fn(n) (the oracle on n rows) on a growing n, then on about
    target_s seconds' worth; returns (rows, seconds)."""
    n = 8
    while True:
        t = time.perf_counter()
        fn(n)
        dt = time.perf_counter() - t
        if dt >= 0.5 or n >= total_rows:
            break
        n = min(total_rows, n * 4)
    rows = int(min(total_rows, max(1, round(n * target_s / max(dt, 1e-6)))))
    t = time.perf_counter()
    fn(rows)
    return rows, time.perf_counter() - t


def bench_attention(args) -> dict:
    import torch
    import tiled_dense_gemm_f16_amd as gr

    B, H, S, D = args.batch, args.heads, args.seq, args.head_dim
    Skv = args.seq_kv or S
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    mk = lambda s_: torch.randn((B, H, s_, D), generator=gen, device="cuda", dtype=torch.float32).half()  # noqa: E731
    rot = 2
    qs = [mk(S) for _ in range(rot)]
    ks = [mk(Skv) for _ in range(rot)]
    vs = [mk(Skv) for _ in range(rot)]
    o = torch.empty_like(qs[0])
    stream = torch.cuda.Stream()
    scale = 1.0 / D ** 0.5
    calls = [lambda i=i: gr.flash_attn_fwd_f16(B, H, S, Skv, D, qs[i].data_ptr(), ks[i].data_ptr(),
                                               vs[i].data_ptr(), o.data_ptr(), 0, scale, int(args.causal),
                                               stream.cuda_stream) for i in range(rot)]
    st = calls[0]()
    if st != gr.OK:
        raise RuntimeError(gr.strerror(st))
    r = time_calls(calls, args.steps, args.warmup, args.graph or 10, stream)
    # multiply-adds of Q K^T and P V over the visible (query, key) pairs
    pairs = sum(min(i + 1, Skv) for i in range(S)) if args.causal else S * Skv
    flops = 4.0 * B * H * D * pairs
    achieved = flops / (r["ms_per_step"] * 1e-3) / 1e12
    name = f"attention_fwd_f16_b{B}_h{H}_s{S}" + (f"_skv{Skv}" if Skv != S else "") + f"_d{D}" + \
        ("_causal" if args.causal else "")
    line = {"metric": "TFLOP/s of the attention forward pass (fp16 in, fp32 accumulate, fp16 out)",
            "value": round(achieved, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": r["steps"],
            "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16", "accum_dtype": "f32", "data": "synthetic",
            "config": {"workload": name, "batch": B, "heads": H, "seq_q": S, "seq_kv": Skv, "head_dim": D,
                       "causal": bool(args.causal), "dist": "normal", "input_copies_rotated": rot,
                       "parallelism": "single GPU"},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                         "traffic": measured_traffic(name, f"attn_fwd_d{D}")},
            "kernel_ms_timed_region_mean": round(r["ms_per_step"], 5), **timing_fields(r),
            "flops_per_launch": flops, "kernel_source_sha256": source_hash(f"attn_fwd_d{D}")}
    if not args.no_cpu_baseline:
        import oracle
        Q = workloads.as_u16(qs[0].cpu())
        Kc = workloads.as_u16(ks[0].cpu())
        Vc = workloads.as_u16(vs[0].cpu())
        rng = np.random.default_rng(0)
        total = B * H * S
        bh_all = rng.integers(0, B * H, total)
        qi_all = rng.integers(0, S, total)

        def run(n):
            oracle.attention_rows_f16(Q, Kc, Vc, scale, bool(args.causal), bh_all[:n], qi_all[:n])

        rows, secs = cpu_sample(run, total, args.cpu_seconds)
        qi = qi_all[:rows]
        row_pairs = np.minimum(qi + 1, Skv).sum() if args.causal else rows * Skv
        line["cpu_baseline"] = {"value": 4.0 * D * float(row_pairs) / secs / 1e12, "unit": "TFLOP/s",
                                "cores": oracle.num_threads(), "kind": "oracle",
                                "sample": f"{rows} random query rows of {name} ({secs:.1f} s)"}
    return line


def bench_softmax(args) -> dict:
    import torch
    import tiled_dense_gemm_f16_amd as gr

    R, C = args.rows, args.cols
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    nbytes = 2 * R * C
    rot = max(1, min(8, -(-ROTATE_BYTES // max(nbytes, 1))))
    xs = [torch.randn((R, C), generator=gen, device="cuda", dtype=torch.float32).half() for _ in range(rot)]
    y = torch.empty_like(xs[0])
    stream = torch.cuda.Stream()
    calls = [lambda i=i: gr.softmax_rows_f16(R, C, xs[i].data_ptr(), y.data_ptr(), stream.cuda_stream)
             for i in range(rot)]
    st = calls[0]()
    if st != gr.OK:
        raise RuntimeError(gr.strerror(st))
    r = time_calls(calls, args.steps, args.warmup, args.graph or 10, stream)
    moved = 2 * nbytes  # each element read once and written once
    gbs = moved / (r["ms_per_step"] * 1e-3) / 1e9
    name = f"softmax_rows_f16_{R}x{C}"
    line = {"metric": "GB/s of the row softmax (fp16 in and out, fp32 arithmetic)", "value": round(gbs, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": r["steps"], "warmup": args.warmup,
            "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16", "accum_dtype": "f32", "data": "synthetic",
            "config": {"workload": name, "rows": R, "cols": C, "dist": "normal", "input_copies_rotated": rot,
                       "parallelism": "single GPU"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(name, "softmax_rows")},
            "kernel_ms_timed_region_mean": round(r["ms_per_step"], 5), **timing_fields(r),
            "bytes_per_launch": moved}
    if not args.no_cpu_baseline:
        import oracle
        X = workloads.as_u16(xs[0].cpu())
        rows, secs = cpu_sample(lambda n: oracle.softmax_rows_f16(X[:n]), R, args.cpu_seconds)
        line["cpu_baseline"] = {"value": 4.0 * rows * C / secs / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
                                "kind": "oracle", "sample": f"rows 0..{rows - 1} of {name} ({secs:.1f} s)"}
    return line


def time_torch_matmul(w, steps: int, warmup: int, graph_batch: int) -> float:
    """Microseconds per launch of torch.matmul(a, b, out=c) (hipBLASLt; no
    ReLU) on the same operands as time_gpu, with the same rotation over input
    copies and the same graph replay: a context line, not part of the path."""
    import torch
    from tiled_dense_gemm_f16_amd import tune

    a, b = workloads.workload_inputs(w)
    rot = tune.rotation(2 * (w.M * w.K + w.K * w.N), graph_batch, ROTATE_BYTES)
    ads = [a.cuda() for _ in range(rot)]
    bds = [b.cuda() for _ in range(rot)]
    c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    stream = torch.cuda.Stream()

    def call(i):  # returns no status: capture_rotation checks only the library's
        torch.matmul(ads[i], bds[i], out=c)

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            call(i % rot)
        torch.cuda.synchronize()
        steps = max(graph_batch, steps // graph_batch * graph_batch)
        graphs = tune.capture_rotation(call, rot, graph_batch, stream)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for r in range(steps // graph_batch):
            graphs[r % len(graphs)].replay()
        t1.record(stream)
        torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / steps


def sustain(args) -> int:
    """Runs one operation back to back on the same inputs for args.sustain
    seconds (batches of 50 launches, each batch between two events) and
    prints the rate about once a second: the load under which board power and
    clocks are sampled (amd-smi / rocm-smi from another process). --sustain-op
    gemm is gemm_relu_f16 on --workload, torch is torch.matmul (hipBLASLt, no
    ReLU) on the same operands, attention is flash_attn_fwd_f16 on the
    --batch/--heads/--seq/--head-dim problem."""
    import torch
    import tiled_dense_gemm_f16_amd as gr

    stream = torch.cuda.Stream()
    if args.sustain_op == "attention":
        B, H, S, D = args.batch, args.heads, args.seq, args.head_dim
        gen = torch.Generator(device="cuda")
        gen.manual_seed(0)
        q, k, v = (torch.randn((B, H, S, D), generator=gen, device="cuda").half() for _ in range(3))
        o = torch.empty_like(q)
        pairs = S * (S + 1) // 2 if args.causal else S * S
        flops = 4.0 * B * H * D * pairs
        name = f"attention_fwd_f16_b{B}_h{H}_s{S}_d{D}" + ("_causal" if args.causal else "")

        def call():
            st = gr.flash_attn_fwd_f16(B, H, S, S, D, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 0,
                                       D ** -0.5, int(args.causal), stream.cuda_stream)
            if st != gr.OK:
                raise RuntimeError(gr.strerror(st))
    else:
        w = workloads.BY_NAME[args.workload]
        a, b = (x.cuda() for x in workloads.workload_inputs(w))
        c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
        flops = float(w.flops)
        name = w.name + (" torch.matmul" if args.sustain_op == "torch" else " gemm_relu_f16")

        def call():
            if args.sustain_op == "torch":
                torch.matmul(a, b, out=c)
                return
            st = gr.gemm_relu_f16(w.M, w.N, w.K, a.data_ptr(), b.data_ptr(), c.data_ptr(), stream.cuda_stream)
            if st != gr.OK:
                raise RuntimeError(gr.strerror(st))
    batch = 50
    end = time.time() + args.sustain
    with torch.cuda.stream(stream):
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        last, done, ms = time.time(), 0, 0.0
        while time.time() < end:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(batch):
                call()
            e1.record(stream)
            e1.synchronize()
            done += batch
            ms += e0.elapsed_time(e1)
            if time.time() - last >= 1.0:
                us = ms * 1e3 / done
                print(f"[sustain] {name}: {us:.1f} us per launch, {flops / (us * 1e-6) / 1e12:.1f} TFLOP/s "
                      f"({done} launches)", flush=True)
                last, done, ms = time.time(), 0, 0.0
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=workloads.SQUARE_4096.name, choices=sorted(workloads.BY_NAME))
    ap.add_argument("--tile", type=int, default=None, help="pin a tile id (default: library's choice)")
    ap.add_argument("--input-dist", choices=("normal", "uniform", "intsmall", "ones"), default=None,
                    help="ablation: draw the workload's inputs from another distribution (intsmall: integers "
                         "in [-2, 2]; ones: every element 1), to show how operand bit activity sets the "
                         "clock the chip holds; the line is then not the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--all", action="store_true", help="also time every workload (lines on stderr)")
    ap.add_argument("--floor", action="store_true",
                    help="also time each workload's launch with K = 64 on the same tile (one reduction step: "
                         "launch, first loads, epilogue and stores; lines on stderr)")
    ap.add_argument("--shards", action="store_true",
                    help="also time one GPU's share of the 4096^3 and 16x8192x8192 workloads under 2-, 4- "
                         "and 8-way column splits (lines on stderr)")
    ap.add_argument("--epilogue", choices=("relu", "bias_gelu"), default="relu",
                    help="relu: C = ReLU(A @ B) (the headline); bias_gelu: C = GELU(A @ B + bias)")
    ap.add_argument("--layout", choices=("nn", "nt", "tn", "tt"), default="nn",
                    help="operand layouts: A stored K x M (t first) and/or B stored N x K (t second)")
    ap.add_argument("--graph", type=int, default=50, metavar="G",
                    help="capture G launches per HIP graph and replay it (0: launch one by one from the host)")
    ap.add_argument("--op", choices=("gemm", "attention", "softmax"), default="gemm",
                    help="gemm (the headline), or the second workload: attention forward / row softmax")
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--heads", type=int, default=32)
    ap.add_argument("--seq", type=int, default=4096)
    ap.add_argument("--seq-kv", type=int, default=0, help="key/value length (default: --seq)")
    ap.add_argument("--head-dim", type=int, default=128, choices=(64, 128))
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--rows", type=int, default=16384)
    ap.add_argument("--cols", type=int, default=8192)
    ap.add_argument("--vs-torch", action="store_true",
                    help="also time torch.matmul (hipBLASLt, no ReLU) on the same operands (lines on stderr)")
    ap.add_argument("--sustain", type=float, default=0.0, metavar="SECONDS",
                    help="only run --sustain-op back to back for SECONDS, printing the rate each second")
    ap.add_argument("--sustain-op", choices=("gemm", "torch", "attention"), default="gemm")
    ap.add_argument("--rotate-mib", type=int, default=ROTATE_BYTES >> 20, metavar="MIB",
                    help="cycle the launches through copies of the inputs spanning at least MIB MiB "
                         "(default: three times the last-level cache, so inputs come from HBM; 0: one copy)")
    ap.add_argument("--steady-ms", type=float, default=STEADY_MS, metavar="MS",
                    help="run the timed work back to back for at least MS ms before the timed region")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run an element-wise copy (negation) of MIB MiB, 20 times: a kernel of known "
                         "traffic, used to scale the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards along M or N without communication, but no multi-GPU run is made.",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_probe:
        n = args.copy_probe << 20
        # an element-wise kernel that reads n bytes and writes n bytes (a plain
        # copy may be served by a DMA engine instead of a kernel)
        src = torch.ones(n // 2, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(20):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 20}), flush=True)
        return 0
    import tiled_dense_gemm_f16_amd as gr
    gr.load()
    if args.sustain > 0:
        return sustain(args)
    if args.op != "gemm":
        if args.graph == 50:
            args.graph = 10
        if args.steps == 2000 and args.warmup == 200:  # defaults sized for the GEMM
            args.steps, args.warmup = (40, 5) if args.op == "attention" else (200, 20)
        line = bench_attention(args) if args.op == "attention" else bench_softmax(args)
        print(f"[bench] {line['config']['workload']}: {line['ms_per_step'] * 1e3:.2f} us/step, "
              f"{line['value']} {line['unit']}", file=sys.stderr, flush=True)
        print(json.dumps(line), flush=True)
        return 0

    w = workloads.BY_NAME[args.workload]
    if args.input_dist:
        w = workloads.with_dist(w, args.input_dist)
    r = time_gpu(w, args.steps, args.warmup, args.tile, args.graph, args.epilogue, args.layout,
                 args.rotate_mib << 20, args.steady_ms)
    print(f"[bench] {w.name}: {r['ms_per_step'] * 1e3:.2f} us/step (graph batch {r['graph_batch']}), "
          f"single launches {r['launch_ms_mean'] * 1e3:.2f} us, tile {r['tile']}", file=sys.stderr, flush=True)

    def vs_torch(ww, rr, steps, warmup):
        if not args.vs_torch or args.layout != "nn":
            return
        t_us = time_torch_matmul(ww, steps, warmup, args.graph or 20)
        ours = rr["ms_per_step"] * 1e3
        print(json.dumps({"comparison": "torch.matmul (hipBLASLt, no ReLU), same operands and rotation",
                          "workload": ww.name, "torch_us": round(t_us, 2), "gemm_relu_f16_us": round(ours, 2),
                          "torch_over_ours": round(t_us / ours, 3)}), file=sys.stderr, flush=True)

    vs_torch(w, r, args.steps, args.warmup)
    if args.all:
        for ow in workloads.ALL:
            if ow is w:
                continue
            orr = time_gpu(ow, max(args.steps // 4, 50), max(args.warmup // 4, 10), None, args.graph, args.epilogue,
                           args.layout, args.rotate_mib << 20, args.steady_ms)
            print(json.dumps(result_line(ow, orr, max(args.steps // 4, 50), max(args.warmup // 4, 10))),
                  file=sys.stderr, flush=True)
            vs_torch(ow, orr, max(args.steps // 4, 50), max(args.warmup // 4, 10))
        # the pages' own tile (128 x 128 x 64) on 1024^3, for comparison
        pages_tile = next(t for t in range(gr.tile_count()) if gr.tile_name(t).startswith("128x128x64"))
        pw = workloads.SQUARE_1024
        prr = time_gpu(pw, max(args.steps // 4, 50), max(args.warmup // 4, 10), pages_tile, args.graph,
                       args.epilogue, args.layout, args.rotate_mib << 20, args.steady_ms)
        pl = result_line(pw, prr, max(args.steps // 4, 50), max(args.warmup // 4, 10))
        pl["note"] = "the pages' 128x128x64 tile pinned, for comparison with the library's choice"
        print(json.dumps(pl), file=sys.stderr, flush=True)
    if args.floor:
        # what a launch costs without its reduction: the same tile and grid
        # with one 64-deep step, so what remains is the launch, the first
        # loads' latency, the epilogue and the stores of C
        for fw in workloads.ALL:
            frr = r if fw is w else time_gpu(fw, max(args.steps // 4, 50), max(args.warmup // 4, 10), None, args.graph,
                                             args.epilogue, args.layout, args.rotate_mib << 20, args.steady_ms)
            tile_id = next(t for t in range(gr.tile_count()) if gr.tile_name(t) == frr["tile"])
            kw = workloads.Workload(fw.name.replace(f"x{fw.K}_", "x64_", 1) + "_floor", fw.M, fw.N, 64, fw.dist,
                                    fw.scale, fw.seed)
            krr = time_gpu(kw, max(args.steps // 4, 50), max(args.warmup // 4, 10), tile_id, args.graph, args.epilogue,
                           args.layout, args.rotate_mib << 20, args.steady_ms)
            print(json.dumps({"floor": kw.name, "tile": krr["tile"], "us_k64": round(krr["ms_per_step"] * 1e3, 3),
                              "workload": fw.name, "us_full": round(frr["ms_per_step"] * 1e3, 3),
                              "share_of_full": round(krr["ms_per_step"] / frr["ms_per_step"], 3)}),
                  file=sys.stderr, flush=True)
    if args.shards:
        # one GPU's share of a column split: no exchange is needed, so a
        # ways-GPU run would take this shard's time (C stays distributed)
        full = {w.name: r}
        for fw in (workloads.SQUARE_4096, workloads.SKINNY):
            if fw.name not in full:
                full[fw.name] = time_gpu(fw, max(args.steps // 4, 50), max(args.warmup // 4, 10), None, args.graph,
                                         args.epilogue, args.layout, args.rotate_mib << 20, args.steady_ms)
        for sw in workloads.SHARDS:
            base = workloads.SQUARE_4096 if sw.M == workloads.SQUARE_4096.M else workloads.SKINNY
            ways = base.N // sw.N
            srr = time_gpu(sw, max(args.steps // 4, 50), max(args.warmup // 4, 10), None, args.graph, args.epilogue,
                           args.layout, args.rotate_mib << 20, args.steady_ms)
            sl = result_line(sw, srr, max(args.steps // 4, 50), max(args.warmup // 4, 10))
            t_full = full[base.name]["ms_per_step"]
            sl["shard_of"] = {"workload": base.name, "ways": ways, "split": "columns of B and C",
                              "full_ms_per_step_one_gpu": t_full,
                              "speedup_if_each_gpu_runs_one_shard": round(t_full / srr["ms_per_step"], 3)}
            print(json.dumps(sl), file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline and args.epilogue == "relu" and args.layout == "nn":
        cpu = cpu_baseline(w, r, args.cpu_seconds)
    line = result_line(w, r, args.steps, args.warmup, cpu)
    if args.input_dist:
        line["note"] = (f"ablation: inputs drawn from {args.input_dist!r} instead of the workload's own; the "
                        "headline is the workload's own inputs")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
