#!/usr/bin/env python3
"""Benchmark of the W2A8 GEMV (M = 1) on one MI355X.

Workload: the eight (N, K) shapes of the benchmark page's test script
("如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？", section
"运行 test.py 做 GEMV 基准测试"), random int8 activations and ternary weights
(1/3 each), int32 output.  One step = one GEMV per shape (the whole sweep),
with the packed weights read cold: each step uses its own copy of every
matrix, rotating over enough copies (16 x 46 MB) that the 256 MB Infinity
Cache and the L2s never hold a copy when it is read again.  Inputs are
resident in HBM before timing starts.

Each step is one HIP graph of the eight launches.  Two events on the launch
stream bracket the K timed steps; their device time divided by the 8*K
launches is the average launch duration, so the roofline's `achieved` is the
algorithmic bytes of all launches over that device time (it includes the
short dispatch gaps between graph nodes).  The host clock around the K steps
gives the whole-job rate (`value`).  Algorithmic bytes per launch: N*K/4
(packed weights) + K (activations) + 4N (int32 output).  Events are not put
around single launches: a marker costs about as much as a small GEMV, and
markers captured inside a graph do not wait for the preceding kernel node.

Per-shape times ("detail") are measured the same way: one graph of 24
launches of one shape (rotating copies when cold), bracketed by two events.

Extras reported under "detail": per-shape times, the host-call latency of
one synchronised call (mean of 50, like the page's timeit(50)), the two
large shapes (5120x27648, 55296x5120; 60% zero weights) cold and warm, and a
device copy-bandwidth calibration.  The CPU baseline times the plain-C oracle
on the same eight GEMVs (single thread) and spot-checks the GPU outputs.

  python bench.py [--steps K] [--warmup W] [--mode cold|warm] [--no-cpu-baseline]
                  [--no-extra] [--eager]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W2A8 GEMV us/call and cold-cache HBM GB/s (% of peak) per (N,K), M=1"
PEAK_HBM_GBPS = 8000.0
PEAK_INT8_TOPS = 5000.0       # MI355X dense int8 MFMA, 5.0 POPS
ROTATE_BYTES = 700e6          # > 256 MB Infinity Cache + 8 x 4 MB L2, with margin
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_sweep_traffic.json")
COLDNESS_FILE = os.path.join(ROOT, "profiles", "gemv_sweep_coldness.json")
# Sources that decide what the GEMV kernels read and write: the ring and
# row-slice kernels and their launch plans (one file), and the shared helpers
# and launch struct.
GEMV_SRCS = [os.path.join(ROOT, "w2a8_gemv_amd", "csrc", f)
             for f in ("gemv_ring.hip", "common.h", "device.h")]


def gemv_sources_sha256():
    h = hashlib.sha256()
    for path in GEMV_SRCS:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()

# The page's A100 40GB numbers for the same shapes (host-timed mean of 50
# calls; another machine): context only.
A100_US = {(2560, 2560): 13.32, (3840, 2560): 14.90, (13824, 2560): 18.75, (2560, 6912): 14.49,
           (3200, 3200): 14.61, (4800, 3200): 13.09, (3200, 10240): 19.64,
           (20480, 3200): 30.99}


def algo_bytes(n, k):
    return n * k // 4 + k + 4 * n


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--mode", choices=["cold", "warm"], default="cold")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only the batched product on the prefill configs (counter runs); "
                         "prints detail.gemm as one JSON line")
    ap.add_argument("--no-detail", action="store_true",
                    help="skip the per-shape cold timings and read floors (counter runs)")
    ap.add_argument("--eager", action="store_true",
                    help="launch each GEMV from the host instead of replaying graphs")
    ap.add_argument("--steps-per-graph", type=int, default=16,
                    help="consecutive steps captured in one hipGraph (default 16, one "
                         "rotation of the weight copies)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="sweep the plain-read kernel over load width, loads in flight per "
                         "wave, waves per CU, non-temporal or plain loads and contiguous or "
                         "strided chunks, on cold 1 GiB, 71 MB and 35 MB buffers; prints one "
                         "JSON line with the table and exits")
    ap.add_argument("--launch-floor", action="store_true",
                    help="launch an empty kernel over 1 to 1024 workgroups and the int8 "
                         "quantizer at M = 1 to 256 (K = 2560), eagerly (kernel-trace runs) "
                         "and graph-timed; prints one JSON line and exits")
    ap.add_argument("--trace-summary", nargs="+", metavar="ARG",
                    help="KERNEL_TRACE_CSV [grid|kernel]: median, mean and minimum duration "
                         "per (kernel, grid, workgroup), or per kernel with its registers and "
                         "LDS, of a rocprofv3 --kernel-trace CSV; prints one JSON line and exits")
    ap.add_argument("--counter-summary", nargs=3, metavar=("TRACE_CSV", "A_CSV", "B_CSV"),
                    help="batched-product counters per launch shape from a kernel trace and "
                         "the two --pmc passes of `bench.py --gemm-only` (see "
                         "gemm_counter_summary); prints one JSON line and exits")
    ap.add_argument("--bf16-context", action="store_true",
                    help="also time the pages' bf16 torch.matmul comparison on the sweep "
                         "shapes (context only, off by default)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB device copy (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --steps 4 --warmup 1 --no-extra --no-detail "
                         "--no-cpu-baseline --calibrate-copy` into " + os.path.relpath(TRAFFIC_FILE, ROOT))
    ap.add_argument("--coldness-summary", nargs=2, metavar=("COLD_CSV", "WARM_CSV"),
                    help="summarise two rocprofv3 --pmc runs (TCC_HIT_sum TCC_MISS_sum "
                         "TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_DRAM_sum) of the traffic command, "
                         "cold and with --mode warm, into " + os.path.relpath(COLDNESS_FILE, ROOT))
    return ap.parse_args()


CALIB_BYTES = 256 << 20


# The plain GEMV's kernels, by the plan's kernel number (w2a8_gemv_plan).
GEMV_KERNELS = {2: "gemv_ring_kernel", 3: "gemv_slice_kernel"}


def gemv_dispatch_key(w2a8, n, k, cus):
    """(kernel with its depth, threads in the grid, threads per workgroup) of
    the plain GEMV's dispatch for (n, k): distinct for every sweep shape's plan
    (the grid alone is not)."""
    kern, wk, sg, d = w2a8.gemv_plan(n, k, cus)
    return (f"{GEMV_KERNELS[kern]}<{d}>", (-(-n // 32)) * sg * 64 * wk, 64 * wk)


def _gemv_row_key(r):
    """The same key for a counter row of a GEMV dispatch, else None."""
    name = _short_kernel_name(r["Kernel_Name"])
    if not any(name.startswith(g + "<") for g in GEMV_KERNELS.values()):
        return None
    return (name, int(r["Grid_Size"]), int(r["Workgroup_Size"]))


def _ring_dispatches(path, counters):
    """Per gemv_dispatch_key of the GEMV dispatches: the mean of each counter;
    and the largest copy dispatch's values (the 256 MiB calibration copy)."""
    import csv
    per, copy = {}, {}
    rows = list(csv.DictReader(open(path)))
    for r in rows:
        name, c, v = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
        if c not in counters:
            continue
        key = _gemv_row_key(r)
        if key is not None:
            per.setdefault(key, {}).setdefault(c, []).append(v)
        elif "copyBuffer" in name:
            copy[c] = max(copy.get(c, 0.0), v)
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in per.items()}, copy


def write_coldness_summary(cold_csv, warm_csv, cus=256):
    """L2 hit/miss and memory-side read requests of the sweep GEMVs, cold and
    warm.  Requests are converted to bytes with the request count of the
    256 MiB calibration copy of the same run."""
    import synth
    import w2a8_gemv_amd as w2a8
    names = ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_DRAM_sum")
    out = {"gemv_sources_sha256": gemv_sources_sha256(), "per_shape": [],
           "calibration": "bytes per memory-side read request = 256 MiB / the calibration "
                          "copy's TCC_EA0_RDREQ_DRAM_sum in the same run",
           "reading": "dram_read_bytes ~ packed bytes in both modes: every weight byte is "
                      "fetched past L2 on every launch.  The Infinity Cache (MALL) is on the "
                      "memory side and has no counter here; its coldness rests on the "
                      "rotation of >= 700 MB of weight copies and on the cold/warm timing gap.",
           "commands": [
               "rocprofv3 --pmc " + " ".join(names) + " --output-format csv -d <dir> -o tcc -- "
               "python -u bench.py --steps 4 --warmup 1 --no-extra --no-detail "
               "--no-cpu-baseline --calibrate-copy [--mode warm]",
               "python bench.py --coldness-summary <cold_counter_collection.csv> "
               "<warm_counter_collection.csv>"]}
    runs = {}
    for mode, path in (("cold", cold_csv), ("warm", warm_csv)):
        per, copy = _ring_dispatches(path, names)
        runs[mode] = (per, CALIB_BYTES / copy["TCC_EA0_RDREQ_DRAM_sum"])
        out["bytes_per_request_" + mode] = round(runs[mode][1], 2)
    for n, k in synth.SWEEP_SHAPES:
        key = gemv_dispatch_key(w2a8, n, k, cus)
        packed = -(-n // 32) * 32 * (-(-k // 128)) * 128 // 4
        row = {"n": n, "k": k, "packed_bytes": packed}
        for mode, (per, bpr) in runs.items():
            d = per[key]
            dram = d["TCC_EA0_RDREQ_DRAM_sum"] * bpr
            row[mode] = {"l2_hit_rate": round(d["TCC_HIT_sum"] / (d["TCC_HIT_sum"] +
                                                                  d["TCC_MISS_sum"]), 4),
                         "dram_read_bytes": round(dram),
                         "dram_over_packed": round(dram / packed, 4)}
        out["per_shape"].append(row)
    os.makedirs(os.path.dirname(COLDNESS_FILE), exist_ok=True)
    with open(COLDNESS_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    return out


def coldness_summary():
    """The committed coldness check, if the GEMV sources are unchanged since."""
    try:
        with open(COLDNESS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemv_sources_sha256") != gemv_sources_sha256():
        return None
    return {"dram_over_packed_cold": [r["cold"]["dram_over_packed"] for r in t["per_shape"]],
            "dram_over_packed_warm": [r["warm"]["dram_over_packed"] for r in t["per_shape"]],
            "source": os.path.relpath(COLDNESS_FILE, ROOT)}


def write_traffic_summary(fetch_csv, write_csv, cus=256):
    """Per-launch HBM traffic of the GEMV from two counter runs.

    Counter values are KiB per dispatch.  Each counter is scaled by what it
    reads for the 256 MiB calibration copy (the largest copy dispatch of the
    run), whose true read and write sizes are known."""
    import csv

    import synth
    import w2a8_gemv_amd as w2a8

    def load(path):
        rows = list(csv.DictReader(open(path)))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        factor = CALIB_BYTES / (max(copies) * 1024.0)
        per = {}
        for r in rows:
            key = _gemv_row_key(r)
            if key is not None:
                per.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        return factor, per

    ff, fetch = load(fetch_csv)
    wf, write = load(write_csv)
    shapes = []
    for n, k in synth.SWEEP_SHAPES:
        key = gemv_dispatch_key(w2a8, n, k, cus)
        f = sum(fetch[key]) / len(fetch[key]) * ff
        w = sum(write[key]) / len(write[key]) * wf
        shapes.append({"n": n, "k": k, "algorithmic_bytes": algo_bytes(n, k),
                       "fetch_bytes": round(f), "write_bytes": round(w),
                       "ratio": round((f + w) / algo_bytes(n, k), 4)})
    sha = gemv_sources_sha256()
    per_launch = sum(x["fetch_bytes"] + x["write_bytes"] for x in shapes) / len(shapes)
    algo = sum(x["algorithmic_bytes"] for x in shapes) / len(shapes)
    out = {"gemv_sources_sha256": sha, "bytes_per_launch": round(per_launch),
           "algorithmic_bytes_per_launch": round(algo),
           "ratio": round(per_launch / algo, 4),
           "fetch_scale": round(ff, 5), "write_scale": round(wf, 5),
           "calibration": "one 256 MiB device copy per run; scale = 256 MiB / counter",
           "per_shape": shapes,
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o fetch -- python -u "
               "bench.py --steps 4 --warmup 1 --no-extra --no-detail --no-cpu-baseline "
               "--calibrate-copy",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o write -- python -u "
               "bench.py --steps 4 --warmup 1 --no-extra --no-detail --no-cpu-baseline "
               "--calibrate-copy",
               "python bench.py --traffic-summary <fetch_counter_collection.csv> "
               "<write_counter_collection.csv>"]}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    return out


class Shape:
    """Device buffers of one GEMV shape (rotating weight copies)."""

    def __init__(self, torch, w2a8, n, k, x, w, slots, dev):
        self.n, self.k = n, k
        self.nbytes = algo_bytes(n, k)
        wp = w2a8.pack_ternary(torch.from_numpy(w)).to(dev)
        self.copies = [wp] + [wp.clone() for _ in range(slots - 1)]
        self.x = torch.from_numpy(x).to(dev)
        self.y = torch.empty(n, dtype=torch.int32, device=dev)
        self.ws = torch.zeros(max(256, w2a8.workspace_bytes(1, n, k)), dtype=torch.uint8,
                              device=dev)
        self.x_host = x

    def launcher(self, lib, stream):
        """A closure that enqueues the C-ABI GEMV on `stream` for copy `slot`."""
        xp, yp, wsp = (ctypes.c_void_p(self.x.data_ptr()), ctypes.c_void_p(self.y.data_ptr()),
                       ctypes.c_void_p(self.ws.data_ptr()))
        ptrs = [ctypes.c_void_p(c.data_ptr()) for c in self.copies]
        n, k, nws = self.n, self.k, self.ws.numel()
        one = ctypes.c_float(1.0)
        sp = ctypes.c_void_p(stream.cuda_stream)
        fn = lib.w2a8_gemv

        def launch(slot):
            rc = fn(ptrs[slot % len(ptrs)], xp, n, k, yp, None, one, None, wsp, nws, sp)
            if rc != 0:
                raise RuntimeError(f"w2a8_gemv failed with status {rc}")
        return launch


def make_shapes(torch, w2a8, synth, specs, mode, dev):
    total = sum(algo_bytes(n, k) for n, k, _, _ in specs)
    slots = 1 if mode == "warm" else max(2, int(-(-ROTATE_BYTES // total)) + 1)
    shapes = []
    for n, k, seed, sparse in specs:
        x, w = synth.gemv_case(n, k, seed, sparse=sparse)
        shapes.append(Shape(torch, w2a8, n, k, x, w, slots, dev))
        del w
    torch.cuda.synchronize()
    return shapes, slots


def _upload_graph(lib, g, stream):
    """Upload an instantiated graph to the device without running it
    (hipGraphUpload, resolved through the library's own HIP runtime, the one
    torch uses), so that its first replay carries no one-time setup.  Best
    effort: without the call the first replay does the upload."""
    try:
        up = lib.hipGraphUpload
        up.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        up.restype = ctypes.c_int
        up(ctypes.c_void_p(g.raw_cuda_graph_exec()), ctypes.c_void_p(stream.cuda_stream))
    except (AttributeError, RuntimeError):
        pass


def build_graphs(torch, shapes, lib, first, count, stream, per_graph):
    """Graphs of up to `per_graph` consecutive steps covering steps
    first .. first+count-1; step j reads copy j of every matrix.  Returns
    [(graph, steps)] and the launchers."""
    launchers = [s.launcher(lib, stream) for s in shapes]
    graphs = []
    with torch.cuda.stream(stream):
        for l in launchers:       # eager warm-up (device query, code object load)
            l(0)
    torch.cuda.synchronize()
    per_graph = max(1, per_graph)
    for start in range(first, first + count, per_graph):
        n = min(per_graph, first + count - start)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(start, start + n):
                for l in launchers:
                    l(j)
        _upload_graph(lib, g, stream)
        graphs.append((g, n))
    torch.cuda.synchronize()
    return graphs, launchers


def timed_steps(torch, graphs, warm_graphs, launchers, steps, warmup, eager, stream):
    """Exactly `warmup` untimed steps, then exactly `steps` timed ones (graph
    replays, or host launches when eager).  Returns (host seconds, device us
    of the timed steps)."""
    with torch.cuda.stream(stream):
        if eager:
            for j in range(warmup):
                for l in launchers:
                    l(j)
        else:
            for g, _ in warm_graphs:
                g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()                      # barrier (one rank)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        if eager:
            for j in range(steps):
                for l in launchers:
                    l(warmup + j)
        else:
            for g, _ in graphs:
                g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, e0.elapsed_time(e1) * 1e3


def kernel_times(torch, lib, shape, reps, stream, rounds=5):
    """Device time per launch (us) of one shape: a graph of launches (launch j
    reads copy j; at least one launch per copy, so a replay re-reads a copy
    only after all the others), replayed `rounds` times, two events per
    replay."""
    return graph_times(torch, shape.launcher(lib, stream), max(reps, len(shape.copies)), stream,
                       rounds)


# Plain-read configurations tried as the floor of each matrix: (waves per CU,
# width in bytes per lane, loads in flight per wave, non-temporal, strided).
# The best configurations of the --read-ceiling sweep on 35 MB and 71 MB
# (strided and contiguous), and a few neighbours.
READ_FLOOR_CONFIGS = [(4, 16, 12, 1, 1), (4, 16, 8, 1, 1), (3, 16, 12, 1, 1), (4, 16, 12, 1, 0),
                      (4, 16, 8, 1, 0), (12, 16, 4, 1, 0), (24, 8, 12, 1, 0), (8, 8, 8, 1, 1)]


def read_floor_times(torch, readref, shape, stream, rounds=5, configs=READ_FLOOR_CONFIGS):
    """The same cold rotation read by the plain-read kernel (no arithmetic, no
    output): per-launch device time of the fastest of `configs`, as a floor
    for the GEMV of that matrix size."""
    if readref is None:
        return None
    nbytes = shape.copies[0].numel()
    cus = torch.cuda.get_device_properties(shape.x.device).multi_processor_count
    best = None
    for cfg in configs:
        ts = read_times(torch, readref, shape.copies, nbytes, cus, cfg, stream, rounds)
        if best is None or sorted(ts)[len(ts) // 2] < sorted(best[1])[len(best[1]) // 2]:
            best = (cfg, ts)
    return best


def read_times(torch, readref, copies, nbytes, cus, cfg, stream, rounds=5, reps=None):
    """Per-launch device time (us) of the plain read of `nbytes` under `cfg`
    (waves per CU, width, depth, nt, strided), one launch per copy in a graph
    (at least 24 launches, or `reps`), so every launch reads a cold copy."""
    wpc, width, depth, nt, strided = cfg
    waves = cus * wpc
    ptrs = [ctypes.c_void_p(c.data_ptr()) for c in copies]
    out = torch.zeros(max(waves, 1), dtype=torch.int32, device=copies[0].device)
    op = ctypes.c_void_p(out.data_ptr())
    sp = ctypes.c_void_p(stream.cuda_stream)

    def launch(j):
        rc = readref.w2a8_readref_read(ptrs[j % len(ptrs)], nbytes, waves, width, depth, nt,
                                       strided, op, sp)
        if rc != 0:
            raise RuntimeError(f"plain read failed with status {rc}")
    return graph_times(torch, launch, reps or max(24, len(ptrs)), stream, rounds)


READ_CEILING_SIZES = [("1 GiB", 1 << 30), ("55296x5120 packed", 70778880),
                      ("5120x27648 packed", 35389440)]


def read_ceiling(torch, readref, stream, cus):
    """Sweep of the plain-read kernel on cold buffers of the READ_CEILING_SIZES:
    every (waves per CU, width, loads in flight, nt, strided) combination,
    per-launch device time from a graph with one launch per buffer copy
    (copies >= 700 MB in total, two for 1 GiB).  Also the per-launch time of
    an empty kernel (the dispatch floor of a graph of launches)."""
    import numpy as np
    wpcs = [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64]
    out = {"method": "per-launch device time of a graph with one launch per cold copy, median "
                     "of 5 replays (includes the dispatch gap between graph nodes)",
           "peak_GBps": PEAK_HBM_GBPS, "cus": cus, "sizes": []}
    dev = torch.device("cuda", torch.cuda.current_device())
    ob = torch.zeros(cus * 64, dtype=torch.int32, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    empty = {}
    for wpc in (1, 4, 16, 64):
        def el(j, w=cus * wpc):
            readref.w2a8_readref_empty(w, ctypes.c_void_p(ob.data_ptr()), sp)
        ts = graph_times(torch, el, 24, stream)
        empty[wpc] = round(float(np.median(ts)), 3)
    out["empty_kernel_us_by_waves_per_cu"] = empty
    for name, nbytes in READ_CEILING_SIZES:
        slots = max(2, int(-(-ROTATE_BYTES // nbytes)) + 1)
        copies = [torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32,
                                device=dev) for _ in range(slots)]
        torch.cuda.synchronize()
        rows = []
        for wpc in wpcs:
            print(f"# read ceiling {name}: {wpc} waves per CU", file=sys.stderr, flush=True)
            for width in (16, 8, 4):
                for depth in (2, 4, 8, 12, 16):
                    for nt in (1, 0):
                        for strided in (0, 1):
                            cfg = (wpc, width, depth, nt, strided)
                            ts = read_times(torch, readref, copies, nbytes, cus, cfg, stream,
                                            reps=max(8 if nbytes > (256 << 20) else 24, slots))
                            med = float(np.median(ts))
                            rows.append({"waves_per_cu": wpc, "width": width, "depth": depth,
                                         "nt": nt, "strided": strided, "median_us": round(med, 3),
                                         "min_us": round(min(ts), 3),
                                         "GBps": round(nbytes / med / 1e3, 1)})
        rows.sort(key=lambda r: r["median_us"])
        best = rows[0]
        out["sizes"].append({"name": name, "bytes": nbytes, "copies": slots,
                             "best": best, "best_pct_peak": round(best["GBps"] / PEAK_HBM_GBPS * 100, 1),
                             "top": rows[:25], "all": rows})
        print(f"# read ceiling {name}: best {best}", file=sys.stderr, flush=True)
        del copies
        torch.cuda.empty_cache()
    return out


def graph_times(torch, launch, reps, stream, rounds=5):
    """Device time per call (us): a graph of `reps` calls launch(0..reps-1),
    replayed `rounds` times after one warm-up replay, two events per replay."""
    with torch.cuda.stream(stream):
        launch(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for j in range(reps):
            launch(j)
    out = []
    for r in range(rounds + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        if r:
            out.append(e0.elapsed_time(e1) * 1e3 / reps)
    return out


LAUNCH_FLOOR_WGS = [1, 2, 4, 8, 16, 32, 128, 1024]
LAUNCH_FLOOR_QUANT_M = [1, 2, 8, 32, 128, 256]


def launch_floor(torch, w2a8, readref, stream, reps=50):
    """The fixed cost of a launch against the workgroups it spreads over the
    dies: an empty kernel (4 waves per workgroup, no memory access) over
    LAUNCH_FLOOR_WGS workgroups, and the int8 quantizer (one workgroup per
    row) at LAUNCH_FLOOR_QUANT_M rows of K = 2560.  Each is launched `reps`
    times eagerly with a synchronisation after each (so a kernel trace sees
    them one by one), then graph-timed (median per launch)."""
    import numpy as np
    dev = torch.device("cuda", torch.cuda.current_device())
    sp = ctypes.c_void_p(stream.cuda_stream)
    ob = torch.zeros(4 * max(LAUNCH_FLOOR_WGS), dtype=torch.int32, device=dev)
    out = {"method": "eager launches one by one (for the kernel trace), then the median "
                     "per-launch time of a graph of 24 launches over 5 replays",
           "empty_kernel": {}, "quant_act_int8_K2560": {}}

    def run(fn):
        for _ in range(reps):
            with torch.cuda.stream(stream):
                fn(0)
            torch.cuda.synchronize()
        return round(float(np.median(graph_times(torch, fn, 24, stream))), 3)

    for wgs in LAUNCH_FLOOR_WGS:
        def el(j, w=4 * wgs):
            rc = readref.w2a8_readref_empty(w, ctypes.c_void_p(ob.data_ptr()), sp)
            if rc != 0:
                raise RuntimeError(f"empty kernel launch failed ({rc})")
        out["empty_kernel"][str(wgs)] = run(el)
    K = 2560
    for m in LAUNCH_FLOOR_QUANT_M:
        xb = torch.randn(m, K, device=dev).to(torch.bfloat16)
        xq = torch.empty(m, K, dtype=torch.int8, device=dev)
        sa = torch.empty(m, dtype=torch.float32, device=dev)

        def ql(j, xb=xb, xq=xq, sa=sa):
            w2a8.quant_act_int8(xb, xq, sa)
        out["quant_act_int8_K2560"][str(m)] = run(ql)
    return out


def _short_kernel_name(name):
    """A kernel's name without its namespace noise and argument list."""
    name = name.replace("(anonymous namespace)::", "").replace("w2a8::", "")
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def _dispatch_size(r, name):
    if name in r:
        return int(r[name])
    return int(r[name + "_X"]) * int(r[name + "_Y"]) * int(r[name + "_Z"])


def trace_summary(path, by="grid"):
    """Dispatches of a rocprofv3 kernel trace, per (kernel, grid threads,
    workgroup threads) (by="grid") or per kernel (by="kernel", with its
    registers and LDS): launches and the median, mean and minimum duration
    (us)."""
    import csv
    import numpy as np
    per, info = {}, {}
    for r in csv.DictReader(open(path)):
        name = _short_kernel_name(r["Kernel_Name"])
        key = (name, _dispatch_size(r, "Grid_Size"), _dispatch_size(r, "Workgroup_Size"))
        if by == "kernel":
            key = (name,)
            info.setdefault(name, {"vgpr": int(r["VGPR_Count"]),
                                   "agpr": int(r.get("Accum_VGPR_Count", 0) or 0),
                                   "lds_bytes": int(r["LDS_Block_Size"]),
                                   "workgroup": _dispatch_size(r, "Workgroup_Size")})
        per.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = []
    for key, d in per.items():
        d = np.asarray(d)
        row = {"kernel": key[0][:70]}
        if by == "kernel":
            row.update(info[key[0]])
        else:
            row.update({"grid": key[1], "workgroup": key[2], "workgroups": key[1] // max(key[2], 1)})
        row.update({"launches": int(d.size), "median_us": round(float(np.median(d)), 3),
                    "mean_us": round(float(d.mean()), 3), "min_us": round(float(d.min()), 3)})
        rows.append(row)
    if by == "kernel":
        rows.sort(key=lambda r: -r["launches"] * r["mean_us"])
    else:
        rows.sort(key=lambda r: (r["kernel"], r["grid"]))
    return rows


def gemm_counter_summary(trace_csv, a_csv, b_csv, simds=1024, ghz=2.4):
    """Batched-product counters per launch shape from three rocprofv3 runs of
    `bench.py --gemm-only`: a kernel trace (durations) and two --pmc passes,
    (a) SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES
    SQ_INSTS_VALU_MFMA_I8 SQ_INSTS_VALU SQ_INSTS_LDS SQ_ACTIVE_INST_VALU and
    (b) SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_ANY
    SQ_ACTIVE_INST_ANY SQ_INSTS_SALU GRBM_GUI_ACTIVE GRBM_COUNT.  Counters are
    averaged over the dispatches of a (kernel, grid, workgroup); MFMA busy is
    SQ_VALU_MFMA_BUSY_CYCLES over all SIMD-cycles of the median duration."""
    import csv
    import numpy as np
    dur = {}
    for r in csv.DictReader(open(trace_csv)):
        key = (_short_kernel_name(r["Kernel_Name"]), _dispatch_size(r, "Grid_Size"),
               _dispatch_size(r, "Workgroup_Size"))
        dur.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counters(path):
        out = {}
        for r in csv.DictReader(open(path)):
            key = (_short_kernel_name(r["Kernel_Name"]), _dispatch_size(r, "Grid_Size"),
                   _dispatch_size(r, "Workgroup_Size"))
            out.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        return out
    ca, cb = counters(a_csv), counters(b_csv)
    rows = []
    for key, c in ca.items():
        if "gemm" not in key[0] or key not in cb:
            continue
        mean = {n: float(np.mean(v)) for n, v in list(c.items()) + list(cb[key].items())}
        mf = mean.get("SQ_INSTS_VALU_MFMA_I8", 0.0)
        if mf <= 0:
            continue
        med = float(np.median(dur[key])) if key in dur else None
        rows.append({"kernel": key[0], "grid": key[1], "workgroup": key[2],
                     "median_us": round(med, 3) if med else None,
                     "mfma": round(mf), "mfma_busy": round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                                           (simds * med * ghz * 1e3), 4) if med else None,
                     "busy_cycles_per_mfma": round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] / mf, 2),
                     "other_valu_per_mfma": round((mean["SQ_INSTS_VALU"] - mf) / mf, 2),
                     "lds_per_mfma": round(mean["SQ_INSTS_LDS"] / mf, 2),
                     "salu_per_mfma": round(mean["SQ_INSTS_SALU"] / mf, 2),
                     "lds_bank_conflicts": round(mean["SQ_LDS_BANK_CONFLICT"]),
                     "waves": round(mean["SQ_WAVES"])})
    rows.sort(key=lambda r: r["mfma"])
    return rows


def rotation(torch, wp, nbytes):
    """Copies of a packed matrix so that one graph of launches reads cold weights."""
    slots = max(2, int(-(-ROTATE_BYTES // max(1, nbytes))) + 1)
    return [wp] + [wp.clone() for _ in range(slots - 1)]


def gemm_extras(torch, w2a8, synth, lib, stream, cus):
    """The batched product on the prefill configs (M in GEMM_MS x GEMM_SHAPES),
    cold weights: int8 TOPS against the dense int8 MFMA peak, and GB/s."""
    out = []
    vp = ctypes.c_void_p
    for n, k in synth.GEMM_SHAPES:
        for m in synth.GEMM_MS:
            x, w = synth.gemm_case(m, n, k, synth.GEMM_SEEDS[((n, k), m)])
            wp = w2a8.pack_ternary(torch.from_numpy(w)).to(stream.device)
            copies = rotation(torch, wp, wp.numel())
            xd = torch.from_numpy(x).to(stream.device)
            y = torch.empty((m, n), dtype=torch.int32, device=stream.device)
            ws = torch.zeros(max(256, w2a8.workspace_bytes(m, n, k)), dtype=torch.uint8,
                             device=stream.device)
            ptrs = [vp(c.data_ptr()) for c in copies]
            args = (vp(xd.data_ptr()), m, n, k, vp(y.data_ptr()), None, ctypes.c_float(1.0),
                    None, vp(ws.data_ptr()), ws.numel(), vp(stream.cuda_stream))

            def launch(j, ptrs=ptrs, args=args):
                rc = lib.w2a8_gemm(ptrs[j % len(ptrs)], *args)
                if rc != 0:
                    raise RuntimeError(f"w2a8_gemm failed with status {rc}")
            ts = graph_times(torch, launch, max(12, len(ptrs)), stream)
            med = sorted(ts)[len(ts) // 2]
            ops = 2 * m * n * k
            nbytes = n * k // 4 + m * k + 4 * m * n
            out.append({"m": m, "n": n, "k": k, "median_us": round(med, 3),
                        "mean_us": round(sum(ts) / len(ts), 3),
                        "TOPS": round(ops / med / 1e6, 1),
                        "pct_int8_peak": round(100 * ops / med / 1e6 / PEAK_INT8_TOPS, 1),
                        "GBps": round(nbytes / med / 1e3, 1),
                        "pct_hbm_peak": round(100 * nbytes / med / 1e3 / PEAK_HBM_GBPS, 1),
                        "rotation_copies": len(copies)})
            del copies, wp, xd, y, ws
            torch.cuda.empty_cache()
    return out


def linear_extras(torch, w2a8, synth, lib, stream):
    """Activation quantizer alone, and the whole linear layer (quantize, then
    GEMV or GEMM with the fp32 epilogue) on the 13824 x 2560 layer, M = 1 and
    128, cold weights."""
    import numpy as np
    vp = ctypes.c_void_p
    n, k = 13824, 2560
    out = {}
    for m in (1, 128):
        xb, W = synth.linear_case(m, n, k, synth.LINEAR_SEEDS[m])
        wq, sw = w2a8.ternarize_absmean(torch.from_numpy(W))
        del W
        wp = w2a8.pack_ternary(wq).to(stream.device)
        copies = rotation(torch, wp, wp.numel())
        xd = torch.from_numpy(xb.view(np.int16)).to(stream.device)
        xq = torch.empty((m, k), dtype=torch.int8, device=stream.device)
        sa = torch.empty(m, dtype=torch.float32, device=stream.device)
        y = torch.empty((m, n), dtype=torch.float32, device=stream.device)
        ws = torch.zeros(max(256, w2a8.workspace_bytes(m, n, k)), dtype=torch.uint8,
                         device=stream.device)
        sp = vp(stream.cuda_stream)
        ptrs = [vp(c.data_ptr()) for c in copies]

        def quant(j):
            rc = lib.quant_act_int8(vp(xd.data_ptr()), m, k, vp(xq.data_ptr()),
                                    vp(sa.data_ptr()), sp)
            if rc != 0:
                raise RuntimeError(f"quant_act_int8 failed with status {rc}")

        def layer(j):
            quant(j)
            if m == 1:
                rc = lib.w2a8_gemv(ptrs[j % len(ptrs)], vp(xq.data_ptr()), n, k, None,
                                   vp(sa.data_ptr()), ctypes.c_float(float(sw)),
                                   vp(y.data_ptr()), vp(ws.data_ptr()), ws.numel(), sp)
            else:
                rc = lib.w2a8_gemm(ptrs[j % len(ptrs)], vp(xq.data_ptr()), m, n, k, None,
                                   vp(sa.data_ptr()), ctypes.c_float(float(sw)),
                                   vp(y.data_ptr()), vp(ws.data_ptr()), ws.numel(), sp)
            if rc != 0:
                raise RuntimeError(f"linear product failed with status {rc}")
        tq = graph_times(torch, quant, 24, stream)
        tl = graph_times(torch, layer, max(12, len(ptrs)), stream)
        mq, ml = sorted(tq)[len(tq) // 2], sorted(tl)[len(tl) // 2]
        qbytes = 3 * m * k + 4 * m
        lbytes = qbytes + n * k // 4 + m * k + 4 * m * n + 4 * m
        out[f"M={m}"] = {"quant_median_us": round(mq, 3),
                         "quant_GBps": round(qbytes / mq / 1e3, 1),
                         "layer_median_us": round(ml, 3),
                         "layer_GBps": round(lbytes / ml / 1e3, 1),
                         "layer_bytes": lbytes,
                         "layer": "quant_act_int8 + " + ("w2a8_gemv" if m == 1 else "w2a8_gemm")
                                  + " with fp32 epilogue, 13824 x 2560, two launches"}
        if m == 1:
            def fused(j):
                rc = lib.w2a8_linear_gemv(ptrs[j % len(ptrs)], vp(xd.data_ptr()), n, k,
                                          ctypes.c_float(float(sw)), vp(y.data_ptr()), None,
                                          vp(ws.data_ptr()), ws.numel(), sp)
                if rc != 0:
                    raise RuntimeError(f"w2a8_linear_gemv failed with status {rc}")
            tf = graph_times(torch, fused, max(24, len(ptrs)), stream)
            mf = sorted(tf)[len(tf) // 2]
            fbytes = 2 * k + n * k // 4 + 4 * n      # bf16 row, packed weights, fp32 out
            out["M=1"].update({"fused_median_us": round(mf, 3),
                               "fused_GBps": round(fbytes / mf / 1e3, 1),
                               "fused_bytes": fbytes,
                               "fused": "w2a8_linear_gemv: the same layer in one launch"})
        del copies, wp, xd, xq, sa, y, ws
        torch.cuda.empty_cache()
    return out


def linear_large_extras(torch, w2a8, synth, lib, stream):
    """The whole linear layer for one token on the two large matrices, cold:
    quant_act_int8 + w2a8_gemv (two launches) against w2a8_linear_gemv, and
    w2a4_linear_gemv (int4 activations), one launch each.  The fused outputs
    are checked bit for bit against the two-launch path."""
    import numpy as np
    vp, F = ctypes.c_void_p, ctypes.c_float
    sp = vp(stream.cuda_stream)
    out = []
    for n, k in ((5120, 27648), (55296, 5120)):
        xb, W = synth.linear_case(1, n, k, synth.LINEAR_SEEDS[1])
        wq, sw = w2a8.ternarize_absmean(torch.from_numpy(W))
        del W
        wp = w2a8.pack_ternary(wq).to(stream.device)
        copies = rotation(torch, wp, wp.numel())
        ptrs = [vp(c.data_ptr()) for c in copies]
        xd = torch.from_numpy(xb.view(np.int16)).to(stream.device)
        xq = torch.empty(k, dtype=torch.int8, device=stream.device)
        sa = torch.empty(1, dtype=torch.float32, device=stream.device)
        y2, yf, y4 = (torch.empty(n, dtype=torch.float32, device=stream.device) for _ in range(3))
        ws = torch.zeros(max(256, w2a8.workspace_bytes(1, n, k)), dtype=torch.uint8,
                         device=stream.device)

        def two(j):
            rc = lib.quant_act_int8(vp(xd.data_ptr()), 1, k, vp(xq.data_ptr()),
                                    vp(sa.data_ptr()), sp)
            if rc == 0:
                rc = lib.w2a8_gemv(ptrs[j % len(ptrs)], vp(xq.data_ptr()), n, k, None,
                                   vp(sa.data_ptr()), F(float(sw)), vp(y2.data_ptr()),
                                   vp(ws.data_ptr()), ws.numel(), sp)
            if rc != 0:
                raise RuntimeError(f"two-launch layer failed with status {rc}")

        def fused(j):
            rc = lib.w2a8_linear_gemv(ptrs[j % len(ptrs)], vp(xd.data_ptr()), n, k,
                                      F(float(sw)), vp(yf.data_ptr()), None,
                                      vp(ws.data_ptr()), ws.numel(), sp)
            if rc != 0:
                raise RuntimeError(f"w2a8_linear_gemv failed with status {rc}")

        def fused4(j):
            rc = lib.w2a4_linear_gemv(ptrs[j % len(ptrs)], vp(xd.data_ptr()), n, k,
                                      F(float(sw)), vp(y4.data_ptr()), None,
                                      vp(ws.data_ptr()), ws.numel(), sp)
            if rc != 0:
                raise RuntimeError(f"w2a4_linear_gemv failed with status {rc}")
        reps = max(24, len(ptrs))
        med = {}
        for nm, fn in (("two_launch_us", two), ("fused_us", fused), ("fused_int4_us", fused4)):
            t = graph_times(torch, fn, reps, stream)
            med[nm] = round(sorted(t)[len(t) // 2], 3)
        stream.synchronize()
        if not torch.equal(y2, yf):
            raise RuntimeError("w2a8_linear_gemv differs from quant_act_int8 + w2a8_gemv")
        fbytes = 2 * k + n * k // 4 + 4 * n
        out.append({"n": n, "k": k, **med, "rotation_copies": len(ptrs),
                    "fused_GBps": round(fbytes / med["fused_us"] / 1e3, 1)})
        del copies, ptrs, wp, xd, xq, sa, y2, yf, y4, ws
        torch.cuda.empty_cache()
    return out


# Decode projections of a 2560-wide layer that share one activation row:
# query/key/value (2560 + 640 + 640 rows) and gate/up (2 x 6912 rows).
GROUP_SETS = {"qkv": ([2560, 640, 640], 2560), "gate_up": ([6912, 6912], 2560)}


def grouped_extras(torch, w2a8, synth, lib, stream):
    """Several projections sharing x: one w2a8_gemv per projection against one
    grouped launch (int8 x), and quant_act_int8 + those GEMVs against one
    grouped linear launch (bf16 x), cold weights, fp32 outputs."""
    import numpy as np
    vp, F = ctypes.c_void_p, ctypes.c_float
    out = {}
    for name, (Ns, k) in GROUP_SETS.items():
        G = len(Ns)
        x, _ = synth.gemv_case(1, k, seed=50)
        xb, _ = synth.linear_case(1, 1, k, seed=51)
        wps = [w2a8.pack_ternary(torch.from_numpy(synth.gemv_case(n, k, seed=52 + g)[1]))
               .to(stream.device) for g, n in enumerate(Ns)]
        total = sum(w.numel() for w in wps)
        slots = max(2, int(-(-ROTATE_BYTES // total)) + 1)   # copies of the whole set
        sets = [wps] + [[w.clone() for w in wps] for _ in range(slots - 1)]
        xd = torch.from_numpy(x).to(stream.device)
        xbd = torch.from_numpy(xb.view(np.int16)).to(stream.device)
        xq = torch.empty(k, dtype=torch.int8, device=stream.device)
        sa = torch.full((1,), 0.02, dtype=torch.float32, device=stream.device)
        ys = [torch.empty(n, dtype=torch.float32, device=stream.device) for n in Ns]
        need = sum(w2a8.workspace_bytes(1, n, k) for n in Ns)
        ws = torch.zeros(max(256, need), dtype=torch.uint8, device=stream.device)
        sp = vp(stream.cuda_stream)
        sw = [0.01 * (g + 1) for g in range(G)]
        n_arr = (ctypes.c_int64 * G)(*Ns)
        sw_arr = (ctypes.c_float * G)(*sw)
        y_arr = (vp * G)(*[y.data_ptr() for y in ys])
        w_arrs = [(vp * G)(*[w.data_ptr() for w in s]) for s in sets]

        def gemvs(j, xp=None):
            for g in range(G):
                rc = lib.w2a8_gemv(vp(sets[j % slots][g].data_ptr()), xp or vp(xd.data_ptr()),
                                   Ns[g], k, None, vp(sa.data_ptr()), F(sw[g]),
                                   vp(ys[g].data_ptr()), vp(ws.data_ptr()), ws.numel(), sp)
                if rc != 0:
                    raise RuntimeError(f"w2a8_gemv failed with status {rc}")

        def grouped(j):
            rc = lib.w2a8_gemv_grouped(G, w_arrs[j % slots], n_arr, k, vp(xd.data_ptr()),
                                       vp(sa.data_ptr()), sw_arr, None, y_arr,
                                       vp(ws.data_ptr()), ws.numel(), sp)
            if rc != 0:
                raise RuntimeError(f"w2a8_gemv_grouped failed with status {rc}")

        def quant_gemvs(j):
            rc = lib.quant_act_int8(vp(xbd.data_ptr()), 1, k, vp(xq.data_ptr()),
                                    vp(sa.data_ptr()), sp)
            if rc != 0:
                raise RuntimeError(f"quant_act_int8 failed with status {rc}")
            gemvs(j, vp(xq.data_ptr()))

        def linear_grouped(j):
            rc = lib.w2a8_linear_gemv_grouped(G, w_arrs[j % slots], n_arr, k,
                                              vp(xbd.data_ptr()), sw_arr, y_arr, None,
                                              vp(ws.data_ptr()), ws.numel(), sp)
            if rc != 0:
                raise RuntimeError(f"w2a8_linear_gemv_grouped failed with status {rc}")

        med = {}
        for key, fn in (("separate", gemvs), ("grouped", grouped),
                        ("linear_separate", quant_gemvs), ("linear_grouped", linear_grouped)):
            ts = graph_times(torch, fn, max(12, slots), stream)
            med[key] = sorted(ts)[len(ts) // 2]
        wbytes = sum(n * k // 4 for n in Ns)
        ybytes = 4 * sum(Ns)
        out[name] = {"N": Ns, "K": k,
                     "separate_us": round(med["separate"], 3),
                     "grouped_us": round(med["grouped"], 3),
                     "grouped_GBps": round((wbytes + k + ybytes) / med["grouped"] / 1e3, 1),
                     "linear_separate_us": round(med["linear_separate"], 3),
                     "linear_grouped_us": round(med["linear_grouped"], 3),
                     "linear_grouped_GBps": round((wbytes + 2 * k + ybytes)
                                                  / med["linear_grouped"] / 1e3, 1),
                     "separate": f"{G} w2a8_gemv launches (linear: quant_act_int8 first)",
                     "grouped": "one w2a8_gemv_grouped launch (linear: one "
                                "w2a8_linear_gemv_grouped launch)"}
        del sets, wps, xd, xbd, xq, sa, ys, ws
        torch.cuda.empty_cache()
    return out


def a4_extras(torch, w2a8, synth, lib, stream):
    """W2A4 variant (int4 activations): per sweep shape and large shape, cold,
    the W2A4 GEMV and the W2A8 GEMV over the same rotation of weight copies
    (one launch per copy per graph), and the whole int4 layer at 13824 x 2560
    (quant_act_int4 + w2a4_gemv with the fp32 epilogue, then w2a4_linear_gemv
    in one launch)."""
    import numpy as np
    vp, F = ctypes.c_void_p, ctypes.c_float
    sp = vp(stream.cuda_stream)
    out = {"shapes": []}
    specs = [(n, k, False) for n, k in synth.SWEEP_SHAPES] + \
            [(n, k, True) for n, k in synth.LARGE_SHAPES]
    for n, k, sparse in specs:
        q, w = synth.gemv_a4_case(n, k, seed=60 + n % 97, sparse=sparse)
        x8 = torch.from_numpy(np.clip(q, -7, 7).astype(np.int8)).to(stream.device)
        x4 = w2a8.pack_act_int4(torch.from_numpy(q)).to(stream.device)
        wp = w2a8.pack_ternary(torch.from_numpy(w)).to(stream.device)
        del w
        copies = rotation(torch, wp, wp.numel())
        ptrs = [vp(c.data_ptr()) for c in copies]
        y = torch.empty(n, dtype=torch.int32, device=stream.device)
        ws = torch.zeros(max(256, w2a8.workspace_bytes(1, n, k)), dtype=torch.uint8,
                         device=stream.device)

        def a4(j):
            rc = lib.w2a4_gemv(ptrs[j % len(ptrs)], vp(x4.data_ptr()), n, k, vp(y.data_ptr()),
                               None, F(1.0), None, vp(ws.data_ptr()), ws.numel(), sp)
            if rc != 0:
                raise RuntimeError(f"w2a4_gemv failed with status {rc}")

        def a8(j):
            rc = lib.w2a8_gemv(ptrs[j % len(ptrs)], vp(x8.data_ptr()), n, k, vp(y.data_ptr()),
                               None, F(1.0), None, vp(ws.data_ptr()), ws.numel(), sp)
            if rc != 0:
                raise RuntimeError(f"w2a8_gemv failed with status {rc}")
        t4 = graph_times(torch, a4, max(24, len(ptrs)), stream)
        t8 = graph_times(torch, a8, max(24, len(ptrs)), stream)
        m4, m8 = sorted(t4)[len(t4) // 2], sorted(t8)[len(t8) // 2]
        b4 = n * k // 4 + x4.numel() + 4 * n
        out["shapes"].append({"n": n, "k": k, "w2a4_median_us": round(m4, 3),
                              "w2a4_GBps": round(b4 / m4 / 1e3, 1),
                              "w2a8_median_us": round(m8, 3), "rotation_copies": len(ptrs)})
        del copies, ptrs, wp, x4, x8, y, ws
        torch.cuda.empty_cache()
    # the whole int4 linear layer for one token at 13824 x 2560
    n, k = 13824, 2560
    xb, W = synth.linear_case(1, n, k, synth.LINEAR_SEEDS[1])
    wq, sw = w2a8.ternarize_absmean(torch.from_numpy(W))
    del W
    wp = w2a8.pack_ternary(wq).to(stream.device)
    copies = rotation(torch, wp, wp.numel())
    ptrs = [vp(c.data_ptr()) for c in copies]
    xd = torch.from_numpy(xb.view(np.int16)).to(stream.device)
    x4 = torch.empty(w2a8.act4_bytes(1, k), dtype=torch.uint8, device=stream.device)
    sa = torch.empty(1, dtype=torch.float32, device=stream.device)
    yf = torch.empty(n, dtype=torch.float32, device=stream.device)
    ws = torch.zeros(max(256, w2a8.workspace_bytes(1, n, k)), dtype=torch.uint8,
                     device=stream.device)

    def layer(j):
        rc = lib.quant_act_int4(vp(xd.data_ptr()), 1, k, vp(x4.data_ptr()), vp(sa.data_ptr()), sp)
        if rc == 0:
            rc = lib.w2a4_gemv(ptrs[j % len(ptrs)], vp(x4.data_ptr()), n, k, None,
                               vp(sa.data_ptr()), F(float(sw)), vp(yf.data_ptr()),
                               vp(ws.data_ptr()), ws.numel(), sp)
        if rc != 0:
            raise RuntimeError(f"int4 layer failed with status {rc}")
    tl = graph_times(torch, layer, max(12, len(ptrs)), stream)
    out["linear_13824x2560_layer_us"] = round(sorted(tl)[len(tl) // 2], 3)
    out["linear"] = "quant_act_int4 + w2a4_gemv with fp32 epilogue, two launches"
    yfu = torch.empty(n, dtype=torch.float32, device=stream.device)

    def fused(j):
        rc = lib.w2a4_linear_gemv(ptrs[j % len(ptrs)], vp(xd.data_ptr()), n, k, F(float(sw)),
                                  vp(yfu.data_ptr()), None, vp(ws.data_ptr()), ws.numel(), sp)
        if rc != 0:
            raise RuntimeError(f"w2a4_linear_gemv failed with status {rc}")
    tf = graph_times(torch, fused, max(12, len(ptrs)), stream)
    stream.synchronize()
    if not torch.equal(yf, yfu):
        raise RuntimeError("w2a4_linear_gemv differs from quant_act_int4 + w2a4_gemv")
    out["linear_13824x2560_fused_us"] = round(sorted(tf)[len(tf) // 2], 3)
    out["fused"] = "w2a4_linear_gemv: the same layer in one launch (bit-identical, checked)"
    del copies, ptrs, wp, xd, x4, sa, yf, yfu, ws
    torch.cuda.empty_cache()
    return out


def bf16_context(torch, synth, stream, per):
    """The pages' comparison on this device, context only: torch.matmul of a
    bf16 activation row [1, K] with bf16 weights [K, N] (cold rotation of
    weight copies), next to the W2A8 GEMV of the same shape
    (detail.per_shape_kernel_times).  The bf16 calls are captured in a graph
    (one call per copy) and the last replay is checked against an eager call;
    if they differ, the eager calls are timed instead."""
    out = []
    g = torch.Generator(device="cpu").manual_seed(90)
    for (n, k), p in zip(synth.SWEEP_SHAPES, per):
        w0 = (torch.randn(k, n, generator=g) * 0.02).to(torch.bfloat16).to(stream.device)
        x = torch.randn(1, k, generator=g).to(torch.bfloat16).to(stream.device)
        slots = max(2, int(-(-ROTATE_BYTES // (2 * n * k))) + 1)
        ws = [w0] + [w0.clone() for _ in range(slots - 1)]
        y = torch.empty(1, n, dtype=torch.bfloat16, device=stream.device)

        def mm(j):
            torch.matmul(x, ws[j % slots], out=y)
        with torch.cuda.stream(stream):
            ref = torch.matmul(x, ws[(slots - 1) % slots])
        torch.cuda.synchronize()
        how = "graph"
        try:
            ts = graph_times(torch, mm, max(24, slots), stream)
            torch.cuda.synchronize()
            if not torch.equal(y, ref):
                raise RuntimeError("graph replay differs from eager")
        except RuntimeError:
            how = "eager"
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                with torch.cuda.stream(stream):
                    e0.record(stream)
                    for j in range(max(24, slots)):
                        mm(j)
                    e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / max(24, slots))
        med = sorted(ts)[len(ts) // 2]
        out.append({"n": n, "k": k, "bf16_matmul_us": round(med, 3), "timing": how,
                    "w2a8_gemv_us": p["median_us"], "bf16_over_w2a8": round(med / p["median_us"], 2)})
        del ws, w0, x, y, ref
        torch.cuda.empty_cache()
    return out


def host_call_us(torch, launcher, reps=50):
    """Mean latency of one synchronised call (the page's timeit(50) style)."""
    launcher(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(reps):
        launcher(j)
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps * 1e6


def copy_bandwidth(torch, dev, nbytes=1 << 30):
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a.fill_(1)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    ts.sort()
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / ts[len(ts) // 2] / 1e9


def traffic_summary():
    """Measured HBM bytes per launch from the committed counter summary, if the
    GEMV kernel sources (kernel, helpers, launch plan) are unchanged since the
    counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        h = gemv_sources_sha256()
    except (OSError, ValueError):
        return None
    if t.get("gemv_sources_sha256") != h:
        return None
    return t.get("bytes_per_launch")


def host_cpu_info():
    """nproc and the CPU model name of this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "model_name": model}


def cpu_baseline(shapes, seconds=10.0, max_threads=16):
    """The oracle (plain C) on the same eight GEMVs, repeated for about
    `seconds` per leg: one thread, then all cores (the same C product on
    contiguous blocks of weight rows, one host thread each, at most
    `max_threads`, a one-GPU machine's CPU share).  Also checks the GPU's last
    outputs on sampled rows."""
    import numpy as np

    import oracle
    import synth

    ws = []
    for s in shapes:
        _, w = synth.gemv_case(s.n, s.k, s.seed, sparse=s.sparse)
        ws.append(w)
    # spot check: a sample of rows of every shape against the GPU result
    ok = True
    rng = np.random.default_rng(0)
    for s, w in zip(shapes, ws):
        rows = rng.choice(s.n, size=min(64, s.n), replace=False)
        ref = oracle.gemm_i32(s.x_host, w[rows])
        got = s.y.cpu().numpy()[rows]
        ok = ok and bool(np.array_equal(ref, got))

    def leg(threads):
        t0 = time.perf_counter()
        reps = 0
        while True:
            for s, w in zip(shapes, ws):
                if threads == 1:
                    oracle.gemm_i32(s.x_host, w)
                else:
                    oracle.gemm_i32_threads(s.x_host, w, threads)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
        return reps, dt, sum(s.nbytes for s in shapes) * reps / dt / 1e9

    info = host_cpu_info()
    nthreads = max(1, min(max_threads, info["nproc"] or 1))
    r1, d1, v1 = leg(1)
    rn, dn, vn = leg(nthreads)
    return {"value": round(v1, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the 8 sweep GEMVs in full (int8 weights unpacked), repeated {r1} times "
                      f"({d1:.1f} s), single thread; GB/s counts the same algorithmic bytes "
                      f"N*K/4+K+4N per GEMV", "ms_per_sweep": round(d1 / r1 * 1e3, 3),
            "all_cores": {"value": round(vn, 4), "unit": "GB/s", "cores": nthreads,
                          "sample": f"the same 8 GEMVs, repeated {rn} times ({dn:.1f} s), the "
                                    f"oracle's C product on {nthreads} host threads, each over "
                                    f"its own block of weight rows",
                          "ms_per_sweep": round(dn / rn * 1e3, 3)},
            "host": info, "gpu_rows_match": ok}


def load_readref():
    """The pure streaming-read helper library (measurement only), or None."""
    from w2a8_gemv_amd import build as b
    if not os.path.exists(b.READREF_PATH):
        return None
    L = ctypes.CDLL(b.READREF_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.w2a8_readref_read.argtypes = [P, ctypes.c_int64, I, I, I, I, I, P, P]
    L.w2a8_readref_read.restype = I
    L.w2a8_readref_empty.argtypes = [I, P, P]
    L.w2a8_readref_empty.restype = I
    return L


def shape_detail(torch, lib, readref, s, stream):
    """Per-launch GEMV time of one shape over its own rotation, and the
    pure-read floor of the same packed matrix over the same rotation."""
    p = summarize_times(s, kernel_times(torch, lib, s, 24, stream))
    p["rotation_copies"] = len(s.copies)
    fl = read_floor_times(torch, readref, s, stream)
    if fl is not None:
        cfg, ts = fl
        med = sorted(ts)[len(ts) // 2]
        p["read_floor"] = {"median_us": round(med, 3),
                           "config": dict(zip(("waves_per_cu", "width", "depth", "nt", "strided"),
                                              cfg)),
                           "packed_bytes": s.copies[0].numel(),
                           "gemv_over_floor": round(p["median_us"] / med, 3)}
    return p


def read_floor_sweep(per):
    """Sum of the per-shape GEMV medians against the sum of the pure-read
    floors of the same matrices (None if the floor was not measured)."""
    if not per or any("read_floor" not in p for p in per):
        return None
    g = sum(p["median_us"] for p in per)
    f = sum(p["read_floor"]["median_us"] for p in per)
    return {"gemv_sum_us": round(g, 3), "floor_sum_us": round(f, 3),
            "gemv_over_floor": round(g / f, 3)}


def summarize_times(s, d):
    """Per-launch times of one shape: GB/s and % of peak follow the median,
    as the reported time does; GBps_of_mean is the rate of the mean."""
    import numpy as np
    d = np.asarray(d, dtype=np.float64)
    return {"n": s.n, "k": s.k, "bytes": s.nbytes, "mean_us": round(float(d.mean()), 3),
            "median_us": round(float(np.median(d)), 3),
            "p10_us": round(float(np.percentile(d, 10)), 3),
            "p90_us": round(float(np.percentile(d, 90)), 3),
            "GBps": round(s.nbytes / float(np.median(d)) / 1e3, 1),
            "pct_peak": round(100 * s.nbytes / float(np.median(d)) / 1e3 / PEAK_HBM_GBPS, 1),
            "GBps_of_mean": round(s.nbytes / float(d.mean()) / 1e3, 1)}


def main():
    args = parse_args()
    if args.traffic_summary:
        print(json.dumps(write_traffic_summary(*args.traffic_summary), indent=1))
        return
    if args.coldness_summary:
        print(json.dumps(write_coldness_summary(*args.coldness_summary), indent=1))
        return
    if args.trace_summary:
        by = args.trace_summary[1] if len(args.trace_summary) > 1 else "grid"
        print(json.dumps({"trace_summary": trace_summary(args.trace_summary[0], by)}))
        return
    if args.counter_summary:
        print(json.dumps({"gemm_counters": gemm_counter_summary(*args.counter_summary)}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the W2A8 GEMV runs on a single MI355X and has no "
              "multi-GPU path (row-sharding across GPUs is a design note only). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w2a8_gemv_amd as w2a8

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    lib = w2a8.lib()
    stream = torch.cuda.Stream()
    if args.read_ceiling:
        rr = load_readref()
        if rr is None:
            raise RuntimeError("the plain-read measurement library is not built")
        print(json.dumps({"read_ceiling": read_ceiling(torch, rr, stream, cus)}), flush=True)
        return
    if args.launch_floor:
        rr = load_readref()
        if rr is None:
            raise RuntimeError("the plain-read measurement library is not built")
        print(json.dumps({"launch_floor": launch_floor(torch, w2a8, rr, stream)}), flush=True)
        return
    if args.gemm_only:
        print(json.dumps({"gemm": gemm_extras(torch, w2a8, synth, lib, stream, cus),
                          "gemm_peak_int8_TOPS": PEAK_INT8_TOPS}), flush=True)
        return

    specs = [(n, k, seed, False) for (n, k), seed in zip(synth.SWEEP_SHAPES, synth.SWEEP_SEEDS)]
    shapes, slots = make_shapes(torch, w2a8, synth, specs, args.mode, dev)
    for s, (_, _, seed, sparse) in zip(shapes, specs):
        s.seed, s.sparse = seed, sparse
    graphs, warm_graphs, launchers = [], [], [s.launcher(lib, stream) for s in shapes]
    if not args.eager:
        # Warm-up steps 0..W-1, timed steps W..W+K-1 (copy j of every matrix
        # in step j), each in graphs of up to --steps-per-graph steps.
        warm_graphs, launchers = build_graphs(torch, shapes, lib, 0, args.warmup, stream,
                                              args.steps_per_graph)
        graphs, launchers = build_graphs(torch, shapes, lib, args.warmup, args.steps, stream,
                                         args.steps_per_graph)
    secs, region_us = timed_steps(torch, graphs, warm_graphs, launchers, args.steps,
                                  args.warmup, args.eager, stream)
    step_bytes = sum(s.nbytes for s in shapes)
    ms_per_step = secs * 1e3 / args.steps
    value = step_bytes / (secs / args.steps) / 1e9
    dev_us = region_us / args.steps                      # device time of one step
    achieved = step_bytes / dev_us / 1e3                 # GB/s over all launches
    traffic = traffic_summary()
    readref = load_readref()
    per = []
    for s in ([] if args.no_detail else shapes):
        solo, _ = make_shapes(torch, w2a8, synth, [(s.n, s.k, s.seed, s.sparse)], args.mode, dev)
        p = shape_detail(torch, lib, readref, solo[0], stream)
        del solo
        warm, _ = make_shapes(torch, w2a8, synth, [(s.n, s.k, s.seed, s.sparse)], "warm", dev)
        wt = sorted(kernel_times(torch, lib, warm[0], 24, stream))
        p["warm_median_us"] = round(wt[len(wt) // 2], 3)
        p["warm_GBps"] = round(s.nbytes / p["warm_median_us"] / 1e3, 1)
        del warm
        per.append(p)
        torch.cuda.empty_cache()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "W2A8 GEMV M=1 over the 8 (N,K) shapes of the page's test script, "
                        + ("cold weights (rotating copies)" if args.mode == "cold" else "warm"),
            "shapes_nk": [[s.n, s.k] for s in shapes],
            "weights": "ternary, P(-1)=P(0)=P(1)=1/3, 2-bit packed",
            "activations": "int8 uniform [-127,127]",
            "rotation_copies": slots,
            "launch": "eager" if args.eager else
                      f"hipGraphs of up to {max(1, args.steps_per_graph)} steps "
                      f"({max(1, args.steps_per_graph) * len(shapes)} launches)",
            "bytes_per_step": step_bytes,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel": "w2a8::gemv_ring_kernel and w2a8::gemv_slice_kernel (all launches "
                      "of the timed region)",
            "avg_launch_us": round(dev_us / len(shapes), 3),
            "step_device_us": round(dev_us, 3),
        },
        "detail": {
            "device": f"{props.name} {props.gcnArchName} {cus} CUs",
            "per_shape_kernel_times": per,
            "per_shape_method": "each shape on its own rotation of >= 700 MB of weight copies "
                                "(cold mode); a graph of one launch per copy (at least 24), "
                                "warm: 24 launches on one copy (L2 / Infinity Cache resident), "
                                "device time per launch from two events per replay, median "
                                "of 5 replays (includes the graph's inter-node gaps). "
                                "read_floor: the plain-read kernel over the same rotation, "
                                "fastest of READ_FLOOR_CONFIGS (waves per CU, bytes per lane, "
                                "loads in flight, non-temporal, strided)",
            "read_floor_sweep": read_floor_sweep(per),
            "l2_coldness_counters": coldness_summary(),
            "plans": {f"{s.n}x{s.k}": list(w2a8.gemv_plan(s.n, s.k, cus)) for s in shapes},
            "a100_page_us_context": {f"{n}x{k}": v for (n, k), v in A100_US.items()},
        },
    }

    if not args.no_extra:
        out["detail"]["host_call_us_mean50"] = {
            f"{s.n}x{s.k}": round(host_call_us(torch, l), 2) for s, l in zip(shapes, launchers)}
        # the two large shapes, cold then warm
        large = []
        lspecs = [(n, k, seed, True) for (n, k), seed in zip(synth.LARGE_SHAPES, synth.LARGE_SEEDS)]
        for spec in lspecs:
            for mode in ("cold", "warm"):
                shp, sl = make_shapes(torch, w2a8, synth, [spec], mode, dev)
                p = shape_detail(torch, lib, readref if mode == "cold" else None, shp[0], stream)
                p.update({"mode": mode, "rotation_copies": sl,
                          "plan": list(w2a8.gemv_plan(spec[0], spec[1], cus))})
                large.append(p)
                del shp
                torch.cuda.empty_cache()
        out["detail"]["large_shapes"] = large
        # the pass bar: the two largest matrices, cold, against 8 TB/s and against the
        # best plain read of the same bytes on the same rotation
        out["largest_shapes_cold"] = [
            {"nk": f"{p['n']}x{p['k']}", "us": p["median_us"], "GBps": p["GBps"],
             "pct_peak": p["pct_peak"],
             "read_floor_us": p.get("read_floor", {}).get("median_us"),
             "over_read_floor": p.get("read_floor", {}).get("gemv_over_floor")}
            for p in large if p["mode"] == "cold"]
        # one GPU's share of each large matrix over 8 GPUs (cold)
        shard = []
        for (n, k), seed in zip(synth.SHARD_SHAPES, synth.SHARD_SEEDS):
            shp, sl = make_shapes(torch, w2a8, synth, [(n, k, seed, True)], "cold", dev)
            p = shape_detail(torch, lib, readref, shp[0], stream)
            p.update({"rotation_copies": sl, "plan": list(w2a8.gemv_plan(n, k, cus))})
            shard.append(p)
            del shp
            torch.cuda.empty_cache()
        out["detail"]["shard_shapes"] = shard
        out["detail"]["device_copy_GBps_read_plus_write"] = round(copy_bandwidth(torch, dev), 1)
        out["detail"]["gemm"] = gemm_extras(torch, w2a8, synth, lib, stream, cus)
        out["detail"]["gemm_peak_int8_TOPS"] = PEAK_INT8_TOPS
        out["detail"]["linear_13824x2560"] = linear_extras(torch, w2a8, synth, lib, stream)
        out["detail"]["linear_large"] = linear_large_extras(torch, w2a8, synth, lib, stream)
        out["detail"]["grouped_decode"] = grouped_extras(torch, w2a8, synth, lib, stream)
        out["detail"]["w2a4"] = a4_extras(torch, w2a8, synth, lib, stream)
        if per and args.bf16_context:
            out["detail"]["bf16_matmul_context"] = bf16_context(torch, synth, stream, per)

    if args.calibrate_copy:
        a = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shapes)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
