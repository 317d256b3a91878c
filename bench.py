#!/usr/bin/env python3
"""Decode-step benchmark of the fused W4 GEMV library on one MI355X.

One step = the 197 weight GEMVs of a Qwen2.5-1.5B decode step at batch 1 (28 layers x {q, k, v, o,
gate, up, down} + lm_head; Do Quantization and Sparsity make LLM Inference Faster?, "What we
did"), NF4 blocksize 64 with fp32 absmax and fp16 activations, every matrix distinct (872 MB of
packed weights and scales, more than the 256 MB last-level cache, so every step streams from
HBM).  Weights are synthetic N(0, 0.02), quantized on the GPU before timing; activations N(0, 1).
The step is captured once as a HIP graph and replayed.

Schedules of the same 197 GEMVs: "grouped" (default) launches each layer's q, k, v together and
its gate, up together through w4_gemm_smallbatch_grouped (the grouped fused GEMV at batch 1), as
a model whose projections share their input runs them (113 launches); "serial" launches every
GEMV on its own (197 launches); "dag" puts q|k|v and gate|up on parallel graph branches.  Every
schedule is timed and reported.

stdout: ONE JSON line (the driver contract).  Details go to stderr and to --report.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--fmt", default="nf4_f16",
                    choices=["nf4_f16", "nf4_bf16", "int4_f16", "int4_bf16", "fp4_f16", "fp4_bf16",
                             "int4a_f16", "int4a_bf16"])
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "splitk", "twopass", "mfma"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-table", action="store_true", help="skip the per-shape table")
    ap.add_argument("--no-large", action="store_true",
                    help="leave the hidden-8192 shapes out of the per-shape table")
    ap.add_argument("--trace-from", metavar="KT_DIR", default=None,
                    help="turn a rocprofv3 --kernel-trace run of this script into the stored "
                         "per-kernel traced durations, then exit")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="cap on the CPU time of the oracle's decode step")
    ap.add_argument("--suite", default="decode",
                    choices=["decode", "shapes", "counters", "steps", "prefill", "gptq", "sparse24"],
                    help="decode: the 197-GEMV step (the benchmark line); shapes: per-shape table; "
                         "counters: a few launches of each path, for rocprofv3 --pmc runs; "
                         "steps: the decode step in the other formats and at batch 8; "
                         "prefill: the 197 GEMMs of a 512-token prompt and a per-shape GEMM table")
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="graph replays per kernel class / shape kind when timing launches")
    ap.add_argument("--schedule", default="grouped", choices=["serial", "grouped", "dag"],
                    help="serial: one chain of 197 launches; grouped: one chain of 113 launches, "
                         "q|k|v and gate|up each in one grouped launch; dag: 197 launches with "
                         "q|k|v and gate|up as graph branches")
    ap.add_argument("--report", default=None, help="write a detailed JSON report here")
    ap.add_argument("--prefill-rows", default="512",
                    help="--suite prefill: activation-row counts of the per-shape table (comma list; "
                         "the step itself is always the 512-token prompt)")
    ap.add_argument("--prefill-steps", type=int, default=1,
                    help="--suite prefill: 0 skips the step timings (per-shape table only)")
    ap.add_argument("--counters-from", nargs="+", metavar="PMC_DIR", default=None,
                    help="CPU only: turn rocprofv3 --pmc runs of --suite counters into per-path "
                         "instruction counts (profiles/counters_paths.json), then exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="CPU only: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script into the stored per-kernel HBM traffic, then exit")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(fmt: str, n: int, k: int, b: int) -> int:
    """Bytes the method itself must move for one GEMV: packed weights + scales + x + y."""
    scale_bytes = {"nf4": n * k // 16, "fp4": n * k // 16, "int4": n * k // 64,
                   "int4a": n * k // 32}[fmt.split("_")[0]]
    return n * k // 2 + scale_bytes + 2 * b * k + 4 * b * n


GROUPS = {"q": ("q", "k", "v"), "gate": ("gate", "up")}  # projections that read the same x


def step_units(shapes, schedule):
    """Launch units of one step: tuples of GEMV indices that share one kernel launch.  "serial"
    and "dag" launch every GEMV on its own; "grouped" launches a layer's q, k and v together and
    its gate and up together (they read the same activations), 113 launches for the 197 GEMVs."""
    if schedule != "grouped":
        return [(i,) for i in range(len(shapes))]
    units, i = [], 0
    while i < len(shapes):
        members = GROUPS.get(shapes[i][0].split(".")[-1])
        if members and tuple(sh[0].split(".")[-1] for sh in shapes[i:i + len(members)]) == members:
            units.append(tuple(range(i, i + len(members))))
            i += len(members)
        else:
            units.append((i,))
            i += 1
    return units


class Step:
    """The 197 GEMVs with their inputs resident in HBM and prebuilt C-ABI arguments."""

    def __init__(self, fmt, b, path, dev, layers=None, on_weight=None):
        """`layers` decoder layers (all 28 by default) plus lm_head.  `on_weight(i, name, w)`, if
        given, sees each fp32 weight matrix on the device before it is quantized and freed."""
        import ctypes

        import torch

        import bit_weight_only_w4_amd as w4
        import synth_inputs

        self.w4, self.fmt, self.b, self.path = w4, fmt, b, path
        self.shapes = synth_inputs.decode_step_shapes(
            synth_inputs.QWEN15_LAYERS if layers is None else layers)
        self.fmt_id = w4.FORMATS[fmt]
        xdt = torch.float16 if fmt.endswith("_f16") else torch.bfloat16
        gen = torch.Generator(device=dev).manual_seed(7)
        self.x = {k: torch.randn(b, k, generator=gen, device=dev).to(xdt).contiguous()
                  for k in sorted({k for _, _, k in self.shapes})}
        self.mats, self.ys = [], []
        t0 = time.time()
        for i, (name, n, k) in enumerate(self.shapes):
            if name == "lm_head":
                seed = 999
            else:
                layer, j = i // 7, i % 7
                seed = 1000 + 8 * layer + j
            g = torch.Generator(device=dev).manual_seed(seed)
            w = torch.randn(n, k, generator=g, device=dev) * synth_inputs.QWEN15_SIGMA
            if on_weight is not None:
                on_weight(i, name, w)
            packed, scales = w4.quantize(fmt, w)
            del w
            self.mats.append((packed, scales))
            self.ys.append(torch.empty(b, n, device=dev))
        torch.cuda.synchronize()
        log(f"[bench] quantized {len(self.shapes)} matrices in {time.time() - t0:.1f}s")
        self.ws_bytes = max(w4.workspace_bytes(fmt, n, k, b, path) for _, n, k in self.shapes)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.plans = []
        vp = ctypes.c_void_p
        self.args = []
        for (name, n, k), (p, s), y in zip(self.shapes, self.mats, self.ys):
            ap, sk = w4.auto_path(fmt, n, k, b, self.ws_bytes) if path == "auto" else (path, 0)
            self.plans.append((ap, sk))
            self.args.append((vp(self.x[k].data_ptr()), vp(p.data_ptr()), vp(s.data_ptr()),
                              self.fmt_id, n, k, b, vp(y.data_ptr()), w4.PATHS[ap], sk,
                              vp(self.ws.data_ptr()), self.ws.numel()))
        self.bytes = [algorithmic_bytes(fmt, n, k, b) for _, n, k in self.shapes]
        self.group_args = {}

    def launch(self, i, stream_handle):
        r = self.w4.lib().w4_matmul_ex(*self.args[i], stream_handle)
        if r != 0:
            self.w4.check(r, f"gemv {self.shapes[i][0]}")

    def launch_unit(self, unit, stream_handle):
        if len(unit) == 1:
            self.launch(unit[0], stream_handle)
            return
        if unit not in self.group_args:
            k = self.shapes[unit[0]][2]
            arrays = self.w4.grouped_args(self.x[k], [self.mats[i][0] for i in unit],
                                          [self.mats[i][1] for i in unit],
                                          [self.ys[i] for i in unit])
            self.group_args[unit] = (self.args[unit[0]][0], len(unit)) + arrays + (
                self.fmt_id, k, self.b)
        # the automatic choice for the members' summed rows: the grouped fused GEMV at small B,
        # the MFMA kernel over every member's row tiles from the MFMA threshold on
        r = self.w4.lib().w4_gemm_smallbatch_grouped(*self.group_args[unit], stream_handle)
        if r != 0:
            self.w4.check(r, f"grouped gemv {[self.shapes[i][0] for i in unit]}")

    def launcher(self, unit, mats=None):
        """A callable(stream_handle) that launches `unit` exactly as launch_unit does, but on the
        matrices `mats` (a list of (packed, scales), one per member; default the step's own): the
        rotated timings launch clones of the step's matrices this way."""
        if mats is None:
            mats = [self.mats[i] for i in unit]
        L = self.w4.lib()
        if len(unit) == 1:
            import ctypes

            a = list(self.args[unit[0]])
            a[1] = ctypes.c_void_p(mats[0][0].data_ptr())
            a[2] = ctypes.c_void_p(mats[0][1].data_ptr())
            a = tuple(a)

            def run(stream_handle):
                r = L.w4_matmul_ex(*a, stream_handle)
                if r != 0:
                    self.w4.check(r, f"gemv {self.shapes[unit[0]][0]}")
            return run
        k = self.shapes[unit[0]][2]
        arrays = self.w4.grouped_args(self.x[k], [m[0] for m in mats], [m[1] for m in mats],
                                      [self.ys[i] for i in unit])
        a = (self.args[unit[0]][0], len(unit)) + arrays + (self.fmt_id, k, self.b)

        def run_group(stream_handle):
            r = L.w4_gemm_smallbatch_grouped(*a, stream_handle)
            if r != 0:
                self.w4.check(r, f"grouped gemv {[self.shapes[i][0] for i in unit]}")
        return run_group

    def unit_key(self, unit):
        """Name of the kernel instantiation a launch unit runs (the profiler's kernel names)."""
        if len(unit) == 1:
            _, n, k = self.shapes[unit[0]]
            path, sk = self.plans[unit[0]]
            return plan_kernel(self.w4, self.fmt, n, k, self.b, path, sk)[0]
        return grouped_kernel(self.w4, self.fmt, [self.shapes[i][1] for i in unit],
                              self.shapes[unit[0]][2], self.b)[0]

    def unit_kind(self, unit):
        return "|".join(self.shapes[i][0].split(".")[-1] for i in unit)

    def unit_bytes(self, unit):
        """Algorithmic bytes of one launch unit: every member's weights, scales and y, x once."""
        x_bytes = 2 * self.b * self.shapes[unit[0]][2]
        return sum(self.bytes[i] - x_bytes for i in unit) + x_bytes


def _gemv_name(fmt, b, iters, threads, grouped):
    fmt_i = {"nf4": 0, "int4": 1, "fp4": 2, "int4a": 3}[fmt.split("_")[0]]
    xt = 0 if fmt.endswith("_f16") else 1
    return f"gemv_kernel<{fmt_i}, {xt}, {b}, {iters}, {threads}, {'true' if grouped else 'false'}>"


def plan_kernel(w4, fmt, n, k, b, path, sk):
    """(kernel name, grid size in work-items) of one launch, from the library's own host-side plan.
    Names match the profiler's kernel names; the grid size is the profiler's Grid_Size."""
    if path in ("gemv", "splitk"):
        plan = w4.gemv_plan(fmt, n, k, b, max(sk, 1))
        key = _gemv_name(fmt, b, plan["iters"], plan["threads"], False)
        if path == "splitk":
            key += f"+splitk_reduce(S={sk})"
        return key, plan["grid_x"] * plan["threads"] * max(sk, 1)
    return path, None


def grouped_kernel(w4, fmt, ns, k, b):
    """(kernel name, grid size in work-items) of one grouped launch over members of ns rows: the
    grouped fused GEMV where the automatic choice for the summed rows is the GEMV, else the MFMA
    kernel (from the tiled batch on, members of 4096 rows and more as tiled launches)."""
    if b > 8 or w4.auto_path(fmt, sum(ns), k, b)[0] != "gemv":
        return ("tiled|mfma" if b >= 128 else "mfma"), None
    plan = w4.gemv_grouped_plan(fmt, ns, k, b)
    return (_gemv_name(fmt, b, plan["iters"], plan["threads"], True),
            plan["grid_x"] * plan["grid_z"] * plan["threads"])


def step_launch_mix(w4, fmt, b, path, schedule):
    """Per launch of the decode step: (kernel name, grid work-items, algorithmic bytes).  Host-only:
    the same units, path choice and plans as Step, without touching the GPU."""
    import synth_inputs

    shapes = synth_inputs.decode_step_shapes()
    ws = max(w4.workspace_bytes(fmt, n, k, b, path) for _, n, k in shapes)
    mix = []
    for unit in step_units(shapes, schedule):
        k = shapes[unit[0]][2]
        if len(unit) == 1:
            n = shapes[unit[0]][1]
            ap, sk = w4.auto_path(fmt, n, k, b, ws) if path == "auto" else (path, 0)
            key, grid = plan_kernel(w4, fmt, n, k, b, ap, sk)
            mix.append((key, grid, algorithmic_bytes(fmt, n, k, b)))
        else:
            ns = [shapes[i][1] for i in unit]
            key, grid = grouped_kernel(w4, fmt, ns, k, b)
            x_bytes = 2 * b * k
            mix.append((key, grid, sum(algorithmic_bytes(fmt, n, k, b) - x_bytes for n in ns) + x_bytes))
    return mix


def kernel_source_digest():
    """sha256 over the sources of the decode step's kernels (the fused GEMV, its launch planning
    and the build flags): a stored counter reading belongs to the kernels it was taken on and to
    nothing built since."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    pkg = os.path.join(root, "bit_weight_only_w4_amd")
    h = hashlib.sha256()
    files = [os.path.join("csrc", f) for f in sorted(os.listdir(os.path.join(pkg, "csrc")))
             if f.startswith("w4_gemv") or f in ("w4_common.h", "w4_api.cpp")]
    for rel in files + ["build.py"]:
        h.update(rel.encode())
        with open(os.path.join(pkg, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_path(fmt, b, path, schedule):
    root = os.path.dirname(os.path.abspath(__file__))
    return os.path.join(root, "profiles", f"traffic_decode_{fmt}_b{b}_{path}_{schedule}.json")


def traffic_from_counters(fetch_dir, write_dir, fmt, b, path, schedule, out):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, in KiB per
    dispatch) into HBM bytes per launch for every kernel of the decode step.

    Each counter is scaled by what it reads for the library's plain copy kernel (1 GiB read and
    1 GiB written per dispatch, launched by the same run); per kernel, the readings are averaged
    per grid size and weighted by how often the step launches that grid.  CPU-only."""
    import collections
    import csv

    import bit_weight_only_w4_amd as w4

    def load(d):
        agg = collections.defaultdict(list)
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                agg[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        return agg

    def mean(v):
        return sum(v) / len(v)

    fetch, write = load(fetch_dir), load(write_dir)
    copy_bytes = 1 << 30
    cf = [v for (n, _), vs in fetch.items() if "probe_copy" in n for v in vs]
    cw = [v for (n, _), vs in write.items() if "probe_copy" in n for v in vs]
    if not cf or not cw:
        raise SystemExit("traffic: the copy probe is missing from the counter runs")
    f_fac = copy_bytes / (mean(cf) * 1024)
    w_fac = copy_bytes / (mean(cw) * 1024)
    mix = step_launch_mix(w4, fmt, b, path, schedule)
    kernels = {}
    for key in sorted({m[0] for m in mix}):
        launches = [m for m in mix if m[0] == key]
        tot_f = tot_w = 0.0
        for _, grid, _ in launches:
            fv = [v for (n, g), vs in fetch.items() if key in n and g == grid for v in vs]
            wv = [v for (n, g), vs in write.items() if key in n and g == grid for v in vs]
            if not fv or not wv:
                raise SystemExit(f"traffic: no counter reading for {key} at grid {grid}")
            tot_f += mean(fv) * 1024 * f_fac
            tot_w += mean(wv) * 1024 * w_fac
        cnt = len(launches)
        kernels[key] = {"launches_per_step": cnt,
                        "fetch_bytes": round(tot_f / cnt), "write_bytes": round(tot_w / cnt),
                        "traffic_bytes": round((tot_f + tot_w) / cnt),
                        "algorithmic_bytes": round(sum(m[2] for m in launches) / cnt)}
        kernels[key]["traffic_over_algorithmic"] = round(
            kernels[key]["traffic_bytes"] / kernels[key]["algorithmic_bytes"], 4)
    rec = {"workload": f"decode step {fmt} batch {b} path {path} schedule {schedule}",
           "format": fmt, "batch": b, "path": path, "schedule": schedule,
           "sources_sha256": kernel_source_digest(),
           "calibration": {"copy_bytes_per_dispatch": copy_bytes,
                           "fetch_kib_per_copy": round(mean(cf), 3),
                           "write_kib_per_copy": round(mean(cw), 3),
                           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
           "kernels": kernels}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def trace_path(fmt, b, path, schedule):
    root = os.path.dirname(os.path.abspath(__file__))
    return os.path.join(root, "profiles", f"trace_decode_{fmt}_b{b}_{path}_{schedule}.json")


def trace_from(kt_dir, fmt, b, path, schedule, out):
    """Turn a rocprofv3 --kernel-trace run of this script into per-kernel execution times of the
    decode step's kernels: for every kernel and grid size of the step's launch mix, the count,
    mean and median of End - Start over all its traced dispatches (every bench phase that ran
    it), and per kernel the mean of those medians weighted by how often the step launches each
    grid.  CPU-only."""
    import collections
    import csv
    import statistics

    import bit_weight_only_w4_amd as w4

    durs = collections.defaultdict(list)
    with open(os.path.join(kt_dir, "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            durs[(r["Kernel_Name"], grid)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    mix = step_launch_mix(w4, fmt, b, path, schedule)
    kernels = {}
    for key in sorted({m[0] for m in mix}):
        launches = [m for m in mix if m[0] == key]
        by_grid = {}
        for grid in sorted({m[1] for m in launches}):
            d = [v for (n, g), vs in durs.items() if key in n and g == grid for v in vs]
            if not d:
                raise SystemExit(f"trace: no dispatch of {key} at grid {grid}")
            by_grid[str(grid)] = {"count": len(d), "mean_ns": round(statistics.fmean(d), 1),
                                  "median_ns": float(statistics.median(d)),
                                  "launches_per_step": sum(1 for m in launches if m[1] == grid)}
        w = sum(v["launches_per_step"] for v in by_grid.values())
        kernels[key] = {"by_grid": by_grid,
                        "step_weighted_median_ns": round(sum(
                            v["median_ns"] * v["launches_per_step"] for v in by_grid.values()) / w, 1),
                        "algorithmic_bytes": round(sum(m[2] for m in launches) / len(launches))}
    rec = {"workload": f"decode step {fmt} batch {b} path {path} schedule {schedule}",
           "sources_sha256": kernel_source_digest(), "kernels": kernels}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def stored_trace(fmt, b, path, schedule):
    """The stored kernel-trace summary of this configuration, or None when there is none or the
    library's sources have changed since it was taken."""
    p = trace_path(fmt, b, path, schedule)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    return rec if rec.get("sources_sha256") == kernel_source_digest() else None


def traced_entry(rec, key, dom):
    """The dominant kernel's traced execution time (no launch gaps) beside the live figure."""
    k = rec["kernels"].get(key)
    if not k:
        return None
    us = k["step_weighted_median_ns"] / 1e3
    gbs = dom["bytes"] / (us / 1e6) / 1e9
    return {"avg_launch_us": round(us, 3), "achieved": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "source": "rocprofv3 --kernel-trace of the default bench command: median End - Start "
                      "per grid size, weighted by the step's launches (kernel execution only, no "
                      "gap between graph nodes)",
            "by_grid": k["by_grid"]}


def stored_traffic(fmt, b, path, schedule, key):
    """HBM bytes per launch of kernel `key` from the stored counter reading, or None when there is
    none or the library's sources have changed since it was taken."""
    p = traffic_path(fmt, b, path, schedule)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("sources_sha256") != kernel_source_digest() or key not in rec.get("kernels", {}):
        return None
    return rec["kernels"][key]["traffic_bytes"]


def capture(step, dev, units, schedule="serial"):
    """Capture the launch units `units` (tuples of GEMV indices; see step_units) into one HIP graph.

    "serial" and "grouped": every launch depends on the previous one (one stream).
    "dag": the dependency structure of a real decode step -- q, k and v of a layer read the same
    activations and run on three branches, gate and up on two, everything else in order -- still
    one kernel launch per GEMV."""
    import torch

    units = list(units)
    s0 = torch.cuda.Stream(device=dev)
    s0.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s0):
        for u in units:  # warm every launch once on the capture stream
            step.launch_unit(u, s0.cuda_stream)
    torch.cuda.synchronize()
    side = [torch.cuda.Stream(device=dev) for _ in range(2)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s0):
        pos = 0
        while pos < len(units):
            group = [units[pos]]
            if schedule == "dag" and len(units[pos]) == 1:
                want = list(GROUPS.get(step.shapes[units[pos][0]][0].split(".")[-1], ())[1:])
                while want and pos + len(group) < len(units):
                    nxt = units[pos + len(group)]
                    if len(nxt) != 1 or step.shapes[nxt[0]][0].split(".")[-1] != want[0]:
                        break
                    group.append(nxt)
                    want.pop(0)
            if len(group) == 1:
                step.launch_unit(group[0], s0.cuda_stream)
            else:
                fork = torch.cuda.Event()
                fork.record(s0)
                for b, u in enumerate(group[1:]):
                    side[b].wait_event(fork)
                    step.launch_unit(u, side[b].cuda_stream)
                step.launch_unit(group[0], s0.cuda_stream)
                for b in range(len(group) - 1):
                    join = torch.cuda.Event()
                    join.record(side[b])
                    s0.wait_event(join)
            pos += len(group)
    torch.cuda.synchronize()
    return graph


def time_replays(graph, steps, warmup):
    """ms per replay: `warmup` untimed replays, then `steps` replays between two events on the
    current stream (the stream the graph's kernels run on)."""
    import torch

    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def graph_time(launchers, dev, reps):
    """us per launch of the launch closures `launchers`, captured in order as one HIP graph on a
    side stream (each launch depends on the previous one, as in the step) and replayed `reps`
    times between two HIP events on the stream the kernels run on."""
    import torch

    s0 = torch.cuda.Stream(device=dev)
    s0.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s0):
        for f in launchers:
            f(s0.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s0):
        for f in launchers:
            f(s0.cuda_stream)
    torch.cuda.synchronize()
    # Replay for about 20 ms before timing, so that the first shape of a table is not timed while
    # the clocks still ramp up from an idle device.
    warm = time_replays(g, 1, 1)
    ms = time_replays(g, reps, max(2, int(20.0 / max(warm, 1e-3))))
    del g
    return ms * 1e3 / len(launchers)


ROTATE_BYTES = 600 << 20  # > 2 x the 256 MB last-level cache


def time_kinds_rotated(step, dev, units, reps=10, min_bytes=ROTATE_BYTES):
    """Average launch time of every launch kind of the step (q|k|v, o, gate|up, down, lm_head, or
    one per projection when ungrouped), measured as the step runs it but on weights that stream
    from HBM: a graph of that kind's launches over the step's own distinct matrices, followed by
    launches on clones of them until the graph has read more than `min_bytes` (twice the
    last-level cache), timed with HIP events.  Returns {kind: {...}}."""
    import torch

    kinds = {}
    for u in units:
        kinds.setdefault(step.unit_kind(u), []).append(u)
    out = {}
    for kind, us in kinds.items():
        launchers = [step.launcher(u) for u in us]
        total = sum(step.unit_bytes(u) for u in us)
        clones = []
        j = 0
        while total < min_bytes:
            u = us[j % len(us)]
            mats = [(step.mats[i][0].clone(), step.mats[i][1].clone()) for i in u]
            clones.append(mats)
            launchers.append(step.launcher(u, mats))
            total += step.unit_bytes(u)
            j += 1
        t = graph_time(launchers, dev, reps)
        u0 = us[0]
        ab = step.unit_bytes(u0)
        out[kind] = {"n": sum(step.shapes[i][1] for i in u0), "k": step.shapes[u0[0]][2],
                     "count": len(us), "graph_launches": len(launchers), "us": t, "bytes": ab,
                     "gbs": ab / (t / 1e6) / 1e9,
                     "path": "grouped" if len(u0) > 1 else step.plans[u0[0]][0],
                     "kernel": step.unit_key(u0)}
        del clones, launchers
        torch.cuda.empty_cache()
    return out


def kernel_classes(step, units, kinds):
    """Per kernel instantiation of the step: launches per step, average launch time (the
    launch-weighted mean of its kinds' rotated times) and average algorithmic bytes per launch."""
    out = {}
    for u in units:
        kd = kinds[step.unit_kind(u)]
        c = out.setdefault(step.unit_key(u), {"launches": 0, "us_sum": 0.0, "bytes_sum": 0.0,
                                             "kinds": []})
        c["launches"] += 1
        c["us_sum"] += kd["us"]
        c["bytes_sum"] += step.unit_bytes(u)
        if step.unit_kind(u) not in c["kinds"]:
            c["kinds"].append(step.unit_kind(u))
    for c in out.values():
        c["us"] = c.pop("us_sum") / c["launches"]
        c["bytes"] = c.pop("bytes_sum") / c["launches"]
    return out


def measure_ceilings(dev, nbytes=2 << 30, reps=10):
    import torch

    import bit_weight_only_w4_amd as w4

    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    dst = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)
    w4.probe_read(src, sink)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        w4.probe_read(src, sink)
    e.record()
    torch.cuda.synchronize()
    read_gbs = nbytes * reps / (s.elapsed_time(e) / 1e3) / 1e9
    half = src[: nbytes // 2]
    w4.probe_copy(half, dst)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        w4.probe_copy(half, dst)
    e.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (nbytes // 2) * reps / (s.elapsed_time(e) / 1e3) / 1e9
    del src, dst
    return read_gbs, copy_gbs


def cpu_baseline(fmt, b, seconds):
    """The oracle (fp64 dequantize + dot products) timed on the host cores: the single 256 x 1536
    GEMV (W ~ N(0, 0.02), seed 0, quantized by the oracle), then one whole 197-GEMV decode step --
    every matrix, lm_head included, in chunks of at most 8192 rows to bound host memory.  The
    step's packed bytes and scales are random storage bits from synth_inputs (drawn untimed, one
    matrix at a time): the oracle's cost does not depend on the values.  The per-shape times are
    those of layer 0's matrices and lm_head within the step.  `seconds` caps the step: when the
    time runs out, the remaining matrices are scaled from the measured ones by weight count (the
    sample string says so)."""
    import numpy as np

    import oracle
    import synth_inputs

    try:
        from threadpoolctl import threadpool_info

        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        threads = 1
    wf = fmt.split("_")[0]
    xd = "f16" if fmt.endswith("_f16") else "bf16"
    quant = {"nf4": oracle.quantize_nf4, "int4": oracle.quantize_int4, "fp4": oracle.quantize_fp4,
             "int4a": oracle.quantize_int4_asym}[wf]
    # the single-GEMV workload
    w0, x0 = synth_inputs.single_gemv_case(seed=0, dtype=xd)
    p0, s0 = quant(w0)
    t0 = time.perf_counter()
    reps = 0
    while reps < 20 or time.perf_counter() - t0 < 0.5:
        oracle.gemv_reference(x0, xd, oracle.dequant(wf, p0, s0))
        reps += 1
    single_us = (time.perf_counter() - t0) / reps * 1e6
    # one decode step, matrix by matrix
    xs = {k: synth_inputs.activations(b, k, xd, seed=7) for k in (1536, 8960)}
    shapes = synth_inputs.decode_step_shapes()
    per_shape, done_s, done_w, total_w = {}, 0.0, 0, sum(n * k for _, n, k in shapes)
    chunk = 8192
    for i, (name, n, k) in enumerate(shapes):
        if done_s >= seconds and name != "lm_head":
            continue
        p, sc = synth_inputs.random_packed(wf, n, k, seed=5000 + i)
        t = time.perf_counter()
        for r0 in range(0, n, chunk):
            oracle.gemv_reference(xs[k], xd, oracle.dequant(wf, p[r0:r0 + chunk], sc[r0:r0 + chunk]))
        el = time.perf_counter() - t
        done_s += el
        done_w += n * k
        short = name.split(".")[-1]
        if name.startswith("L1.") or name == "lm_head":
            per_shape[short] = round(el * 1e6, 1)
        del p, sc
    step_s = done_s * total_w / done_w
    full = done_w == total_w
    try:
        model = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")][0]
    except Exception:
        model = "unknown"
    return {
        "value": round(b / step_s, 4),
        "unit": "tok/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"the 197-GEMV decode step at batch {b}, "
                   + ("every matrix timed" if full else
                      f"{done_w} of {total_w} weights timed, the rest scaled by weight count")
                   + f" (row chunks of {chunk}; random packed bytes and scales, value-independent "
                   f"cost): {step_s:.2f} s/step; the 256x1536 single GEMV {single_us:.0f} us; "
                   f"CPU {model}"),
        "step_s": round(step_s, 3),
        "single_gemv_256x1536_us": round(single_us, 1),
        "per_shape_us": per_shape,
    }


def rotated_mats(fmt, n, k, dev, min_bytes=ROTATE_BYTES, seed=None):
    """One [n, k] matrix W ~ N(0, 0.02) drawn and quantized on the device, plus clones of it until
    the copies together exceed `min_bytes` (so that launches rotating over them stream their
    weights from HBM; the kernels' cost does not depend on the values)."""
    import torch

    import bit_weight_only_w4_amd as w4

    wb = algorithmic_bytes(fmt, n, k, 0)
    copies = max(2, min(4096, -(-min_bytes // wb)))
    gen = torch.Generator(device=dev).manual_seed(n * 31 + k if seed is None else seed)
    w = torch.randn(n, k, generator=gen, device=dev) * 0.02
    p, s = w4.quantize(fmt, w)
    del w
    mats = [(p, s)] + [(p.clone(), s.clone()) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return mats


def time_shape(fmt, n, k, b, path, split_k, dev, mats=None, reps=5):
    """Average launch time of one (format, N, K, B, path) over rotated weight copies (together
    larger than twice the last-level cache, so the weights stream from HBM), as a HIP graph of
    launches timed with events.  Returns (us per launch, None) or (None, error text)."""
    import ctypes

    import torch

    import bit_weight_only_w4_amd as w4

    own = mats is None
    if own:
        mats = rotated_mats(fmt, n, k, dev)
    copies = len(mats)
    xdt = torch.float16 if fmt.endswith("_f16") else torch.bfloat16
    gen = torch.Generator(device=dev).manual_seed(b * 7 + k)
    x = torch.randn(b, k, generator=gen, device=dev).to(xdt)
    y = torch.empty(b, n, device=dev)
    wsb = w4.workspace_bytes(fmt, n, k, b, path, split_k) if path != "gemv" else 0
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    launches = max(copies, 16)
    vp = ctypes.c_void_p
    L = w4.lib()
    err = []

    def make(r):
        p_, s_ = mats[r % copies]
        a = (vp(x.data_ptr()), vp(p_.data_ptr()), vp(s_.data_ptr()), w4.FORMATS[fmt], n, k, b,
             vp(y.data_ptr()), w4.PATHS[path], split_k, vp(ws.data_ptr()), ws.numel())

        def run(stream_handle):
            st = L.w4_matmul_ex(*a, stream_handle)
            if st != 0:
                err.append(w4.status_string(st))
                raise RuntimeError(err[-1])
        return run

    try:
        us = graph_time([make(r) for r in range(launches)], dev, reps)
    except RuntimeError:
        return None, err[-1] if err else "launch failed"
    finally:
        del ws
        if own:
            del mats
        torch.cuda.empty_cache()
    return us, None


def time_read_probe(nbytes, dev, min_bytes=600 << 20, reps=5):
    """Size-matched streaming-read ceiling: the library's read probe over `nbytes` per launch,
    rotated over enough buffers to exceed the last-level cache, as a graph of launches timed like
    time_shape.  Returns us per launch."""
    import torch

    import bit_weight_only_w4_amd as w4

    nbytes = (nbytes + 15) // 16 * 16
    copies = max(1, min(4096, -(-min_bytes // nbytes)))
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    launches = max(copies, 16)
    s0 = torch.cuda.Stream(device=dev)
    s0.wait_stream(torch.cuda.current_stream())
    for r in range(launches):
        w4.probe_read(bufs[r % copies], sink, stream=s0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s0):
        for r in range(launches):
            w4.probe_read(bufs[r % copies], sink, stream=s0)
    ms = time_replays(g, reps, 2)
    del g, bufs
    torch.cuda.empty_cache()
    return ms * 1e3 / launches


# The per-shape table of the default run: the Qwen2.5-1.5B decode shapes at batches 1, 8, 32 and
# 128, the hidden-8192 model's shapes at 1, 4, 16 (its own batches) and 8, 32, 128, and the single
# 256 x 1536 GEMV, all on the automatic path over rotated copies.
TABLE_QWEN = (("q/o", 1536, 1536), ("k/v", 256, 1536), ("gate/up", 8960, 1536),
              ("down", 1536, 8960), ("lm_head", 151936, 1536))
TABLE_LARGE = (("q", 8192, 8192), ("kv", 1024, 8192), ("gate/up", 28672, 8192),
               ("down", 8192, 28672), ("lm_head", 128256, 8192))
# One GPU's share of the hidden-8192 model and of the Qwen lm_head under 8-way tensor
# parallelism: column-parallel matrices split N (q, gate/up, lm_head), the row-parallel down
# projection splits K.
TABLE_SHARD = (("q/8", 1024, 8192), ("gate/up/8", 3584, 8192), ("down/8", 8192, 3584),
               ("lm_head/8", 16032, 8192), ("qwen-lm/8", 18992, 1536))


def shape_table(fmt, dev, read_gbs, large=True):
    """Rows of (shape, B, path, us, GB/s, fractions of 8 TB/s and of the measured read ceiling,
    TFLOP/s and the fraction of the 2.5 PFLOP/s dense fp16/bf16 matrix-core peak from B = 32)."""
    import bit_weight_only_w4_amd as w4

    plan = [("single", "256x1536", 256, 1536, (1,))]
    plan += [("qwen2.5-1.5b", nm, n, k, (1, 8, 32, 128)) for nm, n, k in TABLE_QWEN]
    if large:
        plan += [("hidden-8192", nm, n, k, (1, 4, 8, 16, 32, 128)) for nm, n, k in TABLE_LARGE]
        plan += [("tp8-shard", nm, n, k, (1, 8, 32)) for nm, n, k in TABLE_SHARD]
    rows = []
    for group, name, n, k, bs in plan:
        mats = rotated_mats(fmt, n, k, dev)
        for b in bs:
            # the automatic choice given the workspace it asks for (time_shape passes it)
            path, sk = w4.auto_path(fmt, n, k, b, w4.workspace_bytes(fmt, n, k, b))
            us, err = time_shape(fmt, n, k, b, "auto", 0, dev, mats=mats)
            ab = algorithmic_bytes(fmt, n, k, b)
            r = {"group": group, "shape": name, "n": n, "k": k, "b": b, "path": path,
                 "split_k": sk}
            path = path + (f"/S{sk}" if sk > 1 else "")
            if us is None:
                r["error"] = err
            else:
                gbs = ab / us / 1e3
                tf = 2.0 * n * k * b / us / 1e6
                r.update({"us": round(us, 3), "gbs": round(gbs, 1),
                          "frac_8tbs": round(gbs / HBM_PEAK_GBS, 4),
                          "frac_read_ceiling": round(gbs / read_gbs, 4),
                          "tflops": round(tf, 2)})
                if b >= 32:
                    r["frac_mfma_peak"] = round(tf / MFMA_FP16_PEAK_TFLOPS, 4)
            rows.append(r)
            log(f"[table] {group:12s} {name:9s} {n:6d}x{k:5d} B={b:3d} {path:8s} "
                + (f"{r['us']:9.2f} us {r['gbs']:7.0f} GB/s ({100 * r['frac_8tbs']:5.1f}% of 8 TB/s, "
                   f"{100 * r['frac_read_ceiling']:5.1f}% of read ceiling) {r['tflops']:7.1f} TFLOP/s"
                   if us else f"ERR {err}"))
        del mats
    return rows


# Steps and the split-K table the default run also records (the grouped schedule; compact).
LINE_STEPS = [("int4_bf16", 1), ("int4_bf16", 8), ("nf4_f16", 8)]
LINE_SPLITK = [("int4_bf16", 1, "splitk"), ("int4_bf16", 8, "mfma")]


def line_extras(args, dev):
    """The decode step in INT4 x bf16 at B = 1 and 8 and in NF4 x fp16 at B = 8 (grouped schedule,
    automatic paths), and the down projection 1536 x 8960 in INT4 x bf16 at B = 1 (fused GEMV
    split-K) and B = 8 (MFMA split-K) for S = 1, 2, 4, 8, 16 against the automatic choice, each
    timed over rotated weights: the records the benchmark line carries besides its own step."""
    import torch

    import bit_weight_only_w4_amd as w4

    steps = []
    for fmt, b in LINE_STEPS:
        step = Step(fmt, b, "auto", dev)
        total = sum(step.bytes)
        g = capture(step, dev, step_units(step.shapes, "grouped"), "grouped")
        ms = time_replays(g, args.steps, max(args.warmup, 500))  # clocks settle over ~0.3 s
        del g
        steps.append({"format": fmt, "batch": b, "paths": sorted({p for p, _ in step.plans}),
                      "ms_per_step": round(ms, 5), "tok_s": round(b * 1e3 / ms, 2),
                      "gbs": round(total / (ms / 1e3) / 1e9, 1)})
        log(f"[extras] step {fmt} B={b} grouped: {ms * 1e3:.1f} us/step, {b * 1e3 / ms:.1f} tok/s")
        del step
        torch.cuda.empty_cache()
    splitk = []
    n, k = 1536, 8960
    for fmt, b, path in LINE_SPLITK:
        mats = rotated_mats(fmt, n, k, dev)
        ap, ask = w4.auto_path(fmt, n, k, b, w4.workspace_bytes(fmt, n, k, b))
        row = {"format": fmt, "n": n, "k": k, "b": b, "split_path": path, "auto": [ap, ask], "us": {}}
        for s in (1, 2, 4, 8, 16):
            p = ("gemv" if path == "splitk" else "mfma") if s == 1 else path
            us, err = time_shape(fmt, n, k, b, p, s if s > 1 else 0, dev, mats=mats)
            row["us"][str(s)] = round(us, 3) if us is not None else err
        us, err = time_shape(fmt, n, k, b, "auto", 0, dev, mats=mats)
        row["us"]["auto"] = round(us, 3) if us is not None else err
        splitk.append(row)
        log(f"[extras] down {fmt} B={b} {path}: " + ", ".join(f"S={s} {v}" for s, v in row["us"].items()))
        del mats
        torch.cuda.empty_cache()
    return {"steps": steps, "down_splitk": splitk}


# Decode steps besides the benchmark line's: (format, batch).
OTHER_STEPS = [("int4_bf16", 1), ("int4_bf16", 8), ("nf4_f16", 8), ("nf4_bf16", 1), ("int4_f16", 1),
               ("fp4_f16", 1), ("fp4_bf16", 1), ("fp4_f16", 8), ("int4a_bf16", 1), ("int4a_f16", 1),
               ("int4a_bf16", 8)]


def steps_suite(args, dev):
    """The 197-GEMV step in each OTHER_STEPS format and batch, automatic paths: the serial chain
    and the grouped schedule (q|k|v and gate|up in one launch each, on the kernel the automatic
    path picks for their summed rows).  Returns rows of ms per step and tok/s."""
    import torch

    rows = []
    for fmt, b in OTHER_STEPS:
        step = Step(fmt, b, "auto", dev)
        total = sum(step.bytes)
        r = {"format": fmt, "batch": b, "algorithmic_bytes_per_step": total,
             "paths": sorted({p for p, _ in step.plans})}
        scheds = ["serial", "grouped"]
        for sched in scheds:
            g = capture(step, dev, step_units(step.shapes, sched), sched)
            ms = time_replays(g, args.steps, args.warmup)
            del g
            r[sched] = {"ms_per_step": round(ms, 5), "tok_s": round(b * 1e3 / ms, 2),
                        "gbs": round(total / (ms / 1e3) / 1e9, 1),
                        "launches": len(step_units(step.shapes, sched))}
            log(f"[steps] {fmt} B={b} {sched}: {ms * 1e3:.1f} us/step, {b * 1e3 / ms:.1f} tok/s, "
                f"{total / (ms / 1e3) / 1e9:.0f} GB/s")
        rows.append(r)
        del step
        torch.cuda.empty_cache()
    return rows


PREFILL_TOKENS = 512
PREFILL_FMTS = ("nf4_f16", "int4_bf16", "nf4_bf16", "int4_f16", "fp4_f16", "fp4_bf16", "int4a_f16",
                "int4a_bf16")
MFMA_FP16_PEAK_TFLOPS = 2500.0


def prefill_suite(args, dev):
    """Prefill of a 512-token prompt (LLM Quantization on RTX 4060, "Why Only 16%", item 3): the
    197 matrix multiplications of one Qwen2.5-1.5B forward pass at B = 512 activation rows, through
    the automatic paths (tiled GEMM for the large-N matrices, MFMA for the rest), as one HIP graph
    per schedule; and a per-shape table at B = 512 of the tiled and MFMA paths, with the fp16 dense
    GEMM of the decoded matrix (torch.matmul on an fp16 copy, no 4-bit decode) as context.
    Returns dict(steps=[...], shapes=[...])."""
    import torch

    import bit_weight_only_w4_amd as w4
    import synth_inputs

    b = PREFILL_TOKENS
    out = {"tokens": b, "steps": [], "shapes": []}
    for fmt in (PREFILL_FMTS if args.prefill_steps else ()):
        step = Step(fmt, b, "auto", dev)
        flops = sum(2.0 * n * k * b for _, n, k in step.shapes)
        r = {"format": fmt, "tokens": b, "flop_per_step": flops,
             "paths": sorted({p for p, _ in step.plans})}
        for sched in ("serial", "grouped"):
            g = capture(step, dev, step_units(step.shapes, sched), sched)
            ms = time_replays(g, max(3, args.steps // 10), max(2, args.warmup // 5))
            del g
            r[sched] = {"ms_per_step": round(ms, 4), "tok_s": round(b * 1e3 / ms, 1),
                        "tflops": round(flops / (ms / 1e3) / 1e12, 1),
                        "frac_fp16_mfma_peak": round(flops / (ms / 1e3) / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
                        "launches": len(step_units(step.shapes, sched))}
            log(f"[prefill] {fmt} {b} tokens {sched}: {ms:.3f} ms/step, {b * 1e3 / ms:.0f} tok/s, "
                f"{flops / (ms / 1e3) / 1e12:.0f} TFLOP/s")
        out["steps"].append(r)
        del step
        torch.cuda.empty_cache()
    shapes = [("q/o", 1536, 1536), ("k/v", 256, 1536), ("gate/up", 8960, 1536), ("down", 1536, 8960),
              ("lm_head", 151936, 1536)] + [(f"L.{nm}", n, k) for nm, n, k in synth_inputs.LARGE_SHAPES
                                             if nm != "up"]
    rows_list = [int(v) for v in str(args.prefill_rows).split(",") if v]
    for fmt, b in [(f, r) for r in rows_list for f in ("nf4_f16", "int4_bf16")]:
        for name, n, k in shapes:
            ap, sk = w4.auto_path(fmt, n, k, b, w4.workspace_bytes(fmt, n, k, b))
            row = {"format": fmt, "shape": name, "n": n, "k": k, "b": b, "auto_path": ap,
                   "auto_split": sk}
            mats = rotated_mats(fmt, n, k, dev, min_bytes=256 << 20)
            # "auto": the automatic path with the workspace it asks for (the tiled GEMM over K
            # ranges where its tiles alone do not fill the CUs); "tiled", "mfma": one pass each
            for path in ("auto", "tiled", "mfma"):
                us, err = time_shape(fmt, n, k, b, path, 0, dev, mats=mats, reps=3)
                if us is None:
                    row[path] = {"error": err}
                    continue
                tf = 2.0 * n * k * b / us / 1e6
                row[path] = {"us": round(us, 2), "tflops": round(tf, 1),
                             "frac_fp16_mfma_peak": round(tf / MFMA_FP16_PEAK_TFLOPS, 4)}
            del mats
            if fmt == "nf4_f16":
                w = torch.randn(n, k, device=dev, dtype=torch.float16)
                x = torch.randn(b, k, device=dev, dtype=torch.float16)
                for _ in range(3):
                    y = x @ w.t()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(20):
                    y = x @ w.t()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / 20
                row["fp16_dense_torch"] = {"us": round(us, 2), "tflops": round(2.0 * n * k * b / us / 1e6, 1)}
                del w, x, y
                torch.cuda.empty_cache()
            out["shapes"].append(row)
            log(f"[prefill] {fmt} {name} {n}x{k} B={b} (auto {ap}, S={sk}): " +
                ", ".join(f"{p} {row[p]['us']} us" for p in ("auto", "tiled", "mfma", "fp16_dense_torch")
                          if p in row and "us" in row[p]))
    return out


GPTQ_BLOCK = 128
GPTQ_GROUP = 128
# fp32 multiply and add as separate VALU instructions (no FMA, no packed fp32): one flop per lane
# per cycle, 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.
VALU_FP32_UNFUSED_PEAK_TFLOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def gptq_suite(args, dev):
    """GPTQ's column loop over the seven matrices of one Qwen2.5-1.5B decoder layer (LLM Compressor
    0.14, "The fused kernel"): INT4 codes -8..7 on a symmetric grid fixed beforehand (absmax / 7 per
    group of 128), lazy blocks of 128 columns, U a seeded random upper factor per input width
    (q, k, v, gate and up share one: they read the same activations).  The layer's launches (one
    fused block kernel and one lazy update per block) are captured as one HIP graph; also graphs
    of only the block kernels and only the lazy updates, for their per-launch times.  Returns a
    dict of the figures."""
    import ctypes

    import numpy as np
    import torch

    import bit_weight_only_w4_amd as w4
    import synth_inputs

    L = w4.lib()
    vp = ctypes.c_void_p
    gen = torch.Generator(device=dev).manual_seed(5)
    ufac = {}
    mats = []
    for name, n, k in synth_inputs.QWEN15_LAYER:
        key = name if name in ("o", "down") else "x"
        if key not in ufac:
            ufac[key] = torch.from_numpy(synth_inputs.upper_factor(k, seed=k + len(ufac))).to(dev)
        w = torch.randn(n, k, generator=gen, device=dev) * 0.02
        s = (w.abs().view(n, k // GPTQ_GROUP, GPTQ_GROUP).amax(dim=2) / 7.0).contiguous()
        z = torch.zeros_like(s)
        mats.append((name, n, k, w, ufac[key], s, z, *w4.gptq_outputs(w)))

    def launches(kind):
        out = []
        for name, n, k, w, u, s, z, q, c, e in mats:
            for c0 in range(0, k, GPTQ_BLOCK):
                bc = min(GPTQ_BLOCK, k - c0)
                if kind in ("all", "block"):
                    out.append(("block", name, n, k, c0, bc, (w, u, s, z, q, c, e)))
                if kind in ("all", "lazy") and c0 + bc < k:
                    out.append(("lazy", name, n, k, c0, bc, (w, u, s, z, q, c, e)))
        return out

    def launch(item, stream):
        kind, name, n, k, c0, bc, (w, u, s, z, q, c, e) = item
        if kind == "layer":
            st = L.w4_gptq_quantize(vp(w.data_ptr()), vp(u.data_ptr()), vp(s.data_ptr()),
                                    vp(z.data_ptr()), n, k, GPTQ_GROUP, -8, 7, GPTQ_BLOCK,
                                    vp(q.data_ptr()), vp(c.data_ptr()), vp(e.data_ptr()), vp(stream))
        elif kind == "block":
            st = L.w4_gptq_block_update(vp(w.data_ptr()), vp(u.data_ptr()), vp(s.data_ptr()),
                                        vp(z.data_ptr()), n, k, GPTQ_GROUP, -8, 7, c0, bc,
                                        vp(q.data_ptr()), vp(c.data_ptr()), vp(e.data_ptr()), vp(stream))
        else:
            st = L.w4_gptq_lazy_update(vp(w.data_ptr()), vp(u.data_ptr()), vp(e.data_ptr()), n, k, c0,
                                       bc, vp(stream))
        w4.check(st, kind)

    def graph_of(items):
        s0 = torch.cuda.Stream(device=dev)
        s0.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s0):
            for it in items:
                launch(it, s0.cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s0):
            for it in items:
                launch(it, s0.cuda_stream)
        torch.cuda.synchronize()
        return g

    reps, warm = max(3, args.steps // 20), 2
    res = {"block": GPTQ_BLOCK, "group": GPTQ_GROUP, "matrices": []}
    layer_cols = sum(k for _, _, k in synth_inputs.QWEN15_LAYER)
    # the whole loop per matrix through w4_gptq_quantize (block kernels beside the lazy updates on
    # a helper stream); the kernel-only graphs below launch the blocks and updates one by one
    items = [("layer", name, n, k, 0, 0, (w, u, s, z, q, c, e))
             for name, n, k, w, u, s, z, q, c, e in mats]
    g = graph_of(items)
    ms = time_replays(g, reps, warm)
    del g
    res["layer"] = {"ms": round(ms, 4), "launches": len(launches("all")), "columns": layer_cols,
                    "us_per_column": round(ms * 1e3 / layer_cols, 3)}
    log(f"[gptq] layer: {ms:.3f} ms, {ms * 1e3 / layer_cols:.2f} us per column")
    for kind in ("block", "lazy"):
        its = launches(kind)
        g = graph_of(its)
        ms_k = time_replays(g, reps, warm)
        del g
        flops = 0.0
        for _, _, n, k, c0, bc, _ in its:
            if kind == "lazy":
                flops += 2.0 * n * (k - c0 - bc) * bc
            else:
                flops += 2.0 * n * bc * (bc - 1) / 2
        tf = flops / (ms_k / 1e3) / 1e12
        res[kind] = {"ms": round(ms_k, 4), "launches": len(its),
                     "us_per_launch": round(ms_k * 1e3 / len(its), 3),
                     "flop": flops, "tflops": round(tf, 2),
                     "frac_unfused_fp32_peak": round(tf / VALU_FP32_UNFUSED_PEAK_TFLOPS, 4)}
        log(f"[gptq] {kind} kernels: {ms_k:.3f} ms over {len(its)} launches, {tf:.1f} TFLOP/s")
    for name, n, k, *_ in mats:
        its = [it for it in items if it[1] == name]
        g = graph_of(its)
        ms_m = time_replays(g, reps, warm)
        del g
        res["matrices"].append({"name": name, "rows": n, "cols": k, "ms": round(ms_m, 4),
                                "us_per_column": round(ms_m * 1e3 / k, 3)})
        log(f"[gptq] {name} {n}x{k}: {ms_m:.3f} ms")
    # the oracle's fp32 loop on the q matrix (the same arithmetic, numpy on the host), for scale
    name, n, k = synth_inputs.QWEN15_LAYER[0]
    from oracle import gptq as G

    w = synth_inputs.weights(n, k, seed=1)
    u = synth_inputs.upper_factor(k, seed=2)
    sg = (np.abs(w.reshape(n, k // GPTQ_GROUP, GPTQ_GROUP)).max(axis=2) / np.float32(7)).astype(np.float32)
    t0 = time.perf_counter()
    G.gptq(w, u, sg, np.zeros_like(sg), -8, 7, group=GPTQ_GROUP, block=GPTQ_BLOCK, dtype=np.float32)
    cpu_s = time.perf_counter() - t0
    res["cpu_oracle_q"] = {"seconds": round(cpu_s, 3), "us_per_column": round(cpu_s * 1e6 / k, 1),
                           "threads": 1}
    log(f"[gptq] oracle fp32 loop on q {n}x{k} (host): {cpu_s:.2f} s")
    return res


def sparse24_suite(args, dev):
    """The 197-GEMV decode step at batch 1 with 2:4 sparse fp16 weights (Do Quantization and
    Sparsity make LLM Inference Faster?, "Custom CUDA 2:4 GEMV"): every matrix compressed on the
    GPU from N(0, 0.02) draws, the step captured as one HIP graph of 197 w4_sparse24_gemv
    launches; per shape, the sparse GEMV against the fused NF4 GEMV and a dense fp16 GEMV of the
    same shape (torch.matmul, for context), each timed as a graph over weight copies that exceed
    the last-level cache.  Algorithmic bytes per sparse GEMV: 1.125 B per weight + x + y."""
    import ctypes

    import torch

    import bit_weight_only_w4_amd as w4
    import synth_inputs

    L = w4.lib()
    vp = ctypes.c_void_p
    shapes = synth_inputs.decode_step_shapes()
    gen = torch.Generator(device=dev).manual_seed(7)
    mats = []
    for i, (name, n, k) in enumerate(shapes):
        w = torch.randn(n, k, generator=gen, device=dev) * 0.02
        mats.append((n, k, *w4.sparse24_compress(w, "f16")))
        del w
    xs = {k: torch.randn(1, k, generator=gen, device=dev).to(torch.float16) for k in {k for _, _, k in shapes}}
    ys = [torch.empty((1, n), device=dev) for _, n, _ in shapes]

    def launch(i, stream):
        n, k, v, m = mats[i]
        w4.check(L.w4_sparse24_gemv(vp(xs[k].data_ptr()), vp(v.data_ptr()), vp(m.data_ptr()), 0, n,
                                    k, 1, vp(ys[i].data_ptr()), vp(stream)), "w4_sparse24_gemv")

    def graph_of(fn, count):
        s0 = torch.cuda.Stream(device=dev)
        s0.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s0):
            for i in range(count):
                fn(i, s0.cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s0):
            for i in range(count):
                fn(i, s0.cuda_stream)
        torch.cuda.synchronize()
        return g

    total = sum(n * k * 9 // 8 + 2 * k + 4 * n for _, n, k in shapes)
    res = {"shapes": []}
    units = step_units(shapes, "grouped")
    arr = ctypes.c_void_p

    def launch_unit(j, stream):
        u = units[j]
        if len(u) == 1:
            return launch(u[0], stream)
        g_ = len(u)
        k = mats[u[0]][1]
        w4.check(L.w4_sparse24_gemv_grouped(
            vp(xs[k].data_ptr()), g_, (arr * g_)(*[mats[i][2].data_ptr() for i in u]),
            (arr * g_)(*[mats[i][3].data_ptr() for i in u]),
            (ctypes.c_int64 * g_)(*[mats[i][0] for i in u]), 0, k, 1,
            (arr * g_)(*[ys[i].data_ptr() for i in u]), vp(stream)), "w4_sparse24_gemv_grouped")

    for sched, fn, count in (("grouped", launch_unit, len(units)), ("serial", launch, len(shapes))):
        g = graph_of(fn, count)
        ms = time_replays(g, args.steps, args.warmup)
        del g
        res[sched] = {"ms": round(ms, 5), "tok_s": round(1e3 / ms, 2), "launches": count,
                      "algorithmic_bytes": total, "gbs": round(total / (ms / 1e3) / 1e9, 1)}
        log(f"[s24] decode step, {sched} ({count} launches, B = 1): {ms * 1e3:.1f} us, "
            f"{1e3 / ms:.1f} tok/s, {total / (ms / 1e3) / 1e9:.0f} GB/s")
    res["step"] = res["grouped"]
    del mats, ys
    torch.cuda.empty_cache()
    for name, n, k in [("q/o", 1536, 1536), ("k/v", 256, 1536), ("gate/up", 8960, 1536),
                       ("down", 1536, 8960), ("lm_head", 151936, 1536)]:
        per = n * k * 9 // 8
        copies = max(2, min(64, (600 << 20) // per))
        row = {"shape": name, "n": n, "k": k, "copies": copies}
        sm = [w4.sparse24_compress(torch.randn(n, k, generator=gen, device=dev) * 0.02, "f16")
              for _ in range(copies)]
        x = xs[k]
        yb = torch.empty((1, n), device=dev)

        def ls(i, stream, sm=sm, n=n, k=k, x=x, yb=yb):
            v, m = sm[i]
            w4.check(L.w4_sparse24_gemv(vp(x.data_ptr()), vp(v.data_ptr()), vp(m.data_ptr()), 0, n, k,
                                        1, vp(yb.data_ptr()), vp(stream)), "w4_sparse24_gemv")
        g = graph_of(ls, copies)
        us = time_replays(g, 20, 3) * 1e3 / copies
        del g, sm
        byt = per + 2 * k + 4 * n
        row["sparse24_us"] = round(us, 3)
        row["sparse24_gbs"] = round(byt / us / 1e3, 1)
        t_nf4, _ = time_shape("nf4_f16", n, k, 1, "gemv", 0, dev,
                              mats=rotated_mats("nf4_f16", n, k, dev, min_bytes=256 << 20), reps=3)
        row["nf4_gemv_us"] = round(t_nf4, 3) if t_nf4 else None
        dcopies = max(2, min(32, (600 << 20) // (n * k * 2)))
        dw = [torch.randn(n, k, generator=gen, device=dev).to(torch.float16) for _ in range(dcopies)]
        for _ in range(3):
            for d in dw:
                torch.matmul(x, d.t())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            for d in dw:
                torch.matmul(x, d.t())
        e1.record()
        torch.cuda.synchronize()
        row["fp16_dense_torch_us"] = round(e0.elapsed_time(e1) * 1e3 / (5 * dcopies), 3)
        del dw
        torch.cuda.empty_cache()
        res["shapes"].append(row)
        log(f"[s24] {name} {n}x{k}: sparse {row['sparse24_us']} us ({row['sparse24_gbs']} GB/s), "
            f"NF4 GEMV {row['nf4_gemv_us']} us, fp16 dense {row['fp16_dense_torch_us']} us")
    return res


def shapes_suite(args, dev):
    """Per-shape table for the other workloads: INT4 decode steps (B = 1, 8) and split-K vs one
    pass on down; small-batch GEMM on gate / down / lm_head at B = 1, 8, 32, 128 for the GEMV,
    MFMA and two-pass paths, and GEMV against MFMA at B = 2..6; the larger single-GPU model's
    shapes at B = 1, 4, 16."""
    import synth_inputs

    rows = []
    probe_us = {}

    def add(group, fmt, name, n, k, b, path, split_k=0):
        us, err = time_shape(fmt, n, k, b, path, split_k, dev)
        ab = algorithmic_bytes(fmt, n, k, b)
        if ab not in probe_us:
            probe_us[ab] = time_read_probe(ab, dev)
        r = {"group": group, "fmt": fmt, "shape": name, "n": n, "k": k, "b": b, "path": path,
             "split_k": split_k, "algorithmic_bytes": ab}
        if us is None:
            r["error"] = err
        else:
            r["us"] = round(us, 3)
            r["gbs"] = round(ab / us / 1e3, 1)
            r["frac_hbm"] = round(ab / us / 1e3 / HBM_PEAK_GBS, 4)
            r["tflops"] = round(2.0 * n * k * b / us / 1e6, 2)
            # the same bytes through the streaming-read probe, launched the same way
            r["read_probe_us"] = round(probe_us[ab], 3)
            r["frac_size_matched_read"] = round(probe_us[ab] / us, 4)
        rows.append(r)
        log(f"[shapes] {group:10s} {fmt:9s} {name:8s} {n:6d}x{k:5d} B={b:3d} {path:7s} S={split_k:2d} "
            + (f"{r['us']:9.2f} us {r['gbs']:8.0f} GB/s {r['tflops']:7.2f} TFLOP/s "
               f"(read probe {r['read_probe_us']:.2f} us)" if us else f"ERR {err}"))

    # INT4 g128, bf16 x: the five decode shapes at B = 1 and 8; split-K vs one pass on down
    for b in (1, 8):
        for name, n, k in (("q/o", 1536, 1536), ("k/v", 256, 1536), ("gate/up", 8960, 1536),
                           ("down", 1536, 8960), ("lm_head", 151936, 1536)):
            add("int4-step", "int4_bf16", name, n, k, b, "auto")
        for sk in (2, 4, 8, 16):
            add("int4-splitk", "int4_bf16", "down", 1536, 8960, b, "splitk", sk)
    for sk in (2, 4, 8, 16):
        add("nf4-splitk", "nf4_f16", "down", 1536, 8960, 1, "splitk", sk)
    # NF4 fp16 small-batch GEMM: GEMV path (B <= 8), MFMA, two-pass
    for name, n, k in (("gate", 8960, 1536), ("down", 1536, 8960), ("lm_head", 151936, 1536)):
        for b in (1, 8, 32, 128):
            if b <= 8:
                add("nf4-gemm", "nf4_f16", name, n, k, b, "gemv")
            add("nf4-gemm", "nf4_f16", name, n, k, b, "mfma")
            add("nf4-gemm", "nf4_f16", name, n, k, b, "twopass")
    # GEMV against MFMA at small batches (where the automatic path switches)
    for name, n, k in (("gate", 8960, 1536), ("down", 1536, 8960), ("lm_head", 151936, 1536)):
        for b in (2, 3, 4, 6):
            add("crossover", "nf4_f16", name, n, k, b, "gemv")
            add("crossover", "nf4_f16", name, n, k, b, "mfma")
    # larger single-GPU model
    for fmt in ("nf4_f16", "int4_f16"):
        for name, n, k in synth_inputs.LARGE_SHAPES:
            if name == "up":
                continue
            for b in (1, 4, 16):
                add("large", fmt, name, n, k, b, "auto")
    return rows


# Launches whose instruction mix the counter runs record: (name, format, N, K, B, path).
COUNTER_CASES = [
    ("gemv nf4 gate B=1", "nf4_f16", 8960, 1536, 1, "gemv"),
    ("gemv nf4 down B=1", "nf4_f16", 1536, 8960, 1, "gemv"),
    ("gemv nf4 lm_head B=1", "nf4_f16", 151936, 1536, 1, "gemv"),
    ("gemv int4 gate B=1", "int4_bf16", 8960, 1536, 1, "gemv"),
    ("gemv nf4 gate B=4", "nf4_f16", 8960, 1536, 4, "gemv"),
    ("mfma nf4 gate B=8", "nf4_f16", 8960, 1536, 8, "mfma"),
    ("mfma nf4 gate B=32", "nf4_f16", 8960, 1536, 32, "mfma"),
    ("mfma nf4 gate B=128", "nf4_f16", 8960, 1536, 128, "mfma"),
    ("mfma nf4 lm_head B=8", "nf4_f16", 151936, 1536, 8, "mfma"),
    ("mfma nf4 lm_head B=32", "nf4_f16", 151936, 1536, 32, "mfma"),
    ("mfma nf4 lm_head B=128", "nf4_f16", 151936, 1536, 128, "mfma"),
    ("twopass nf4 gate B=1", "nf4_f16", 8960, 1536, 1, "twopass"),
    ("tiled nf4 gate B=512", "nf4_f16", 8960, 1536, 512, "tiled"),
    ("tiled nf4 lm_head B=512", "nf4_f16", 151936, 1536, 512, "tiled"),
    ("tiled nf4 L.gate B=512", "nf4_f16", 28672, 8192, 512, "tiled"),
    ("tiled fp4 lm_head B=512", "fp4_f16", 151936, 1536, 512, "tiled"),
    ("tiled nf4 bf16 lm_head B=512", "nf4_bf16", 151936, 1536, 512, "tiled"),
    ("tiled int4 bf16 L.gate B=512", "int4_bf16", 28672, 8192, 512, "tiled"),
]
COUNTER_LAUNCHES = 3
COUNTER_KERNELS = ("gemv_kernel", "mfma_kernel", "gemm_kernel", "fold_kernel", "dequant", "dense")


def counters_suite(dev):
    """COUNTER_LAUNCHES launches of every COUNTER_CASES entry, in order, after all inputs are
    made (so that the only library launches in the run are these)."""
    import torch

    import bit_weight_only_w4_amd as w4

    made = []
    for name, fmt, n, k, b, path in COUNTER_CASES:
        gen = torch.Generator(device=dev).manual_seed(n + k)
        w = torch.randn(n, k, generator=gen, device=dev) * 0.02
        p, sc = w4.quantize(fmt, w)
        del w
        xdt = torch.float16 if fmt.endswith("_f16") else torch.bfloat16
        x = torch.randn(b, k, generator=gen, device=dev).to(xdt)
        ws = None
        if path == "twopass":
            ws = torch.empty(w4.workspace_bytes(fmt, n, k, b, path, 0), dtype=torch.uint8, device=dev)
        made.append((p, sc, x, ws))
    torch.cuda.synchronize()
    for (name, fmt, n, k, b, path), (p, sc, x, ws) in zip(COUNTER_CASES, made):
        for _ in range(COUNTER_LAUNCHES):
            w4.matmul_ex(x, p, sc, fmt, path=path, workspace=ws)
        torch.cuda.synchronize()
        log(f"[counters] {name}: {COUNTER_LAUNCHES} launches")


def counters_from(dirs):
    """Per-launch SQ/GRBM counter averages of every COUNTER_CASES entry from rocprofv3 --pmc runs
    of --suite counters (one counter set per directory), with VALU instructions per MAC
    (64 lanes * SQ_INSTS_VALU / (B N K)) and MFMA busy cycles per MFMA instruction.  CPU-only."""
    import collections
    import csv

    per_case = [collections.defaultdict(list) for _ in COUNTER_CASES]
    meta = [dict() for _ in COUNTER_CASES]
    for d in dirs:
        disp = collections.OrderedDict()
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if not any(kw in r["Kernel_Name"] for kw in COUNTER_KERNELS):
                    continue
                e = disp.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"],
                                                            "grid": int(r["Grid_Size"]),
                                                            "vgpr": int(r["VGPR_Count"]),
                                                            "lds": int(r["LDS_Block_Size"]),
                                                            "c": {}})
                e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        ids = sorted(disp)
        pos = 0
        for ci, (name, fmt, n, k, b, path) in enumerate(COUNTER_CASES):
            per_launch = 2 if path == "twopass" else 1
            for _ in range(COUNTER_LAUNCHES):
                group = [disp[i] for i in ids[pos:pos + per_launch]]
                pos += per_launch
                if len(group) != per_launch:
                    raise SystemExit(f"counters: {d} ends before case {name!r}")
                tot = collections.Counter()
                for e in group:
                    tot.update(e["c"])
                for cname, v in tot.items():
                    per_case[ci][cname].append(v)
                meta[ci] = {"kernels": [e["kernel"].replace("void ", "").replace(
                    "w4::(anonymous namespace)::", "").split("(")[0] for e in group],
                    "grid": [e["grid"] for e in group], "vgpr": [e["vgpr"] for e in group],
                    "lds": [e["lds"] for e in group]}
        if pos != len(ids):
            raise SystemExit(f"counters: {d} has {len(ids) - pos} library dispatches past the cases")
    out = []
    for ci, (name, fmt, n, k, b, path) in enumerate(COUNTER_CASES):
        c = {cn: sum(v) / len(v) for cn, v in per_case[ci].items()}
        rec = {"case": name, "fmt": fmt, "n": n, "k": k, "b": b, "path": path, **meta[ci],
               "counters_per_launch": {cn: round(v, 1) for cn, v in sorted(c.items())}}
        macs = float(b) * n * k
        if "SQ_INSTS_VALU" in c:
            rec["valu_insts_per_mac"] = round(64.0 * c["SQ_INSTS_VALU"] / macs, 4)
        if "SQ_INSTS_LDS" in c:
            rec["lds_insts_per_mac"] = round(64.0 * c["SQ_INSTS_LDS"] / macs, 4)
        if c.get("SQ_INSTS_MFMA"):
            rec["mfma_insts"] = round(c["SQ_INSTS_MFMA"], 1)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                rec["mfma_busy_cycles_per_mfma_inst"] = round(
                    c["SQ_VALU_MFMA_BUSY_CYCLES"] / c["SQ_INSTS_MFMA"], 2)
        out.append(rec)
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "counters_paths.json")
    with open(path, "w") as f:
        json.dump({"launches_per_case": COUNTER_LAUNCHES, "sources": sorted(dirs), "cases": out},
                  f, indent=1)
        f.write("\n")
    return path, out


def main():
    args = parse_args()
    if args.counters_from:
        path, out = counters_from(args.counters_from)
        print(json.dumps({"counters": path, "cases": len(out)}))
        return
    if args.trace_from:
        out = trace_path(args.fmt, args.batch, args.path, args.schedule)
        rec = trace_from(args.trace_from, args.fmt, args.batch, args.path, args.schedule, out)
        print(json.dumps({"trace": out, "kernels": {k: v["step_weighted_median_ns"]
                                                    for k, v in rec["kernels"].items()}}))
        return
    if args.traffic_from:
        out = traffic_path(args.fmt, args.batch, args.path, args.schedule)
        rec = traffic_from_counters(*args.traffic_from, args.fmt, args.batch, args.path,
                                    args.schedule, out)
        print(json.dumps({"traffic": out, "kernels": {k: v["traffic_bytes"]
                                                      for k, v in rec["kernels"].items()}}))
        return
    if args.suite == "counters":
        import torch

        import bit_weight_only_w4_amd as w4

        w4.lib()
        counters_suite(torch.device("cuda:0"))
        print(json.dumps({"suite": "counters", "cases": len(COUNTER_CASES),
                          "launches_per_case": COUNTER_LAUNCHES}), flush=True)
        return
    if args.suite == "steps":
        import torch

        import bit_weight_only_w4_amd as w4

        w4.lib()
        rows = steps_suite(args, torch.device("cuda:0"))
        if args.report:
            os.makedirs(os.path.dirname(os.path.abspath(args.report)), exist_ok=True)
            with open(args.report, "w") as f:
                json.dump(rows, f, indent=1)
        print(json.dumps({"metric": "decode step in other formats and batches", "rows": rows}),
              flush=True)
        return
    if args.suite == "prefill":
        import torch

        import bit_weight_only_w4_amd as w4

        w4.lib()
        res = prefill_suite(args, torch.device("cuda:0"))
        if args.report:
            os.makedirs(os.path.dirname(os.path.abspath(args.report)), exist_ok=True)
            with open(args.report, "w") as f:
                json.dump(res, f, indent=1)
        print(json.dumps({"metric": "prefill step (512 tokens) and per-shape GEMM table",
                          "steps": res["steps"]}), flush=True)
        return
    if args.suite == "sparse24":
        import torch

        res = sparse24_suite(args, torch.device("cuda:0"))
        if args.report:
            os.makedirs(os.path.dirname(os.path.abspath(args.report)), exist_ok=True)
            with open(args.report, "w") as f:
                json.dump(res, f, indent=1)
        print(json.dumps({"metric": "2:4 sparse decode step (197 GEMVs, B=1)", **res["step"]}),
              flush=True)
        return
    if args.suite == "gptq":
        import torch

        res = gptq_suite(args, torch.device("cuda:0"))
        if args.report:
            os.makedirs(os.path.dirname(os.path.abspath(args.report)), exist_ok=True)
            with open(args.report, "w") as f:
                json.dump(res, f, indent=1)
        print(json.dumps({"metric": "GPTQ column loop, one Qwen2.5-1.5B layer", **res["layer"]}),
              flush=True)
        return
    if args.suite == "shapes":
        import torch

        import bit_weight_only_w4_amd as w4

        w4.lib()
        dev = torch.device("cuda:0")
        rows = shapes_suite(args, dev)
        if args.report:
            os.makedirs(os.path.dirname(os.path.abspath(args.report)), exist_ok=True)
            with open(args.report, "w") as f:
                json.dump(rows, f, indent=1)
        ok = [r for r in rows if "us" in r]
        print(json.dumps({"metric": "per-shape fused W4 GEMV/GEMM table", "rows": len(rows),
                          "measured": len(ok), "report": args.report}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (--gpus {args.gpus} requested); "
              "multi-GPU sharding is described, not measured", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_weight_only_w4_amd as w4

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    w4.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    step = Step(args.fmt, args.batch, args.path, dev)
    total_bytes = sum(step.bytes)

    # every schedule of the same 197 GEMVs, the selected one first
    timed = {}
    for sched in [args.schedule] + [x for x in ("serial", "grouped", "dag") if x != args.schedule]:
        g = capture(step, dev, step_units(step.shapes, sched), sched)
        timed[sched] = time_replays(g, args.steps, args.warmup)
        del g
        log(f"[bench] step ({sched}) {timed[sched] * 1e3:.1f} us -> "
            f"{args.batch * 1e3 / timed[sched]:.1f} tok/s")
    ms = timed[args.schedule]
    tok_s = args.batch * 1e3 / ms
    step_gbs = total_bytes / (ms / 1e3) / 1e9
    log(f"[bench] selected {args.schedule}: algorithmic {total_bytes / 1e6:.1f} MB -> "
        f"{step_gbs:.0f} GB/s ({100 * step_gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s)")

    units = step_units(step.shapes, args.schedule)
    shapes = time_kinds_rotated(step, dev, units, args.kernel_reps)
    kernels = kernel_classes(step, units, shapes)
    for kind, r in shapes.items():
        log(f"[bench] {kind:10s} {r['n']:6d}x{r['k']:5d} {r['path']:7s} {r['us']:8.2f} us/launch "
            f"{r['gbs']:8.0f} GB/s  ({r['graph_launches']} rotated launches) [{r['kernel']}]")
    kinds_sum_us = sum(shapes[step.unit_kind(u)]["us"] for u in units)
    log(f"[bench] sum over the step's launches of their kinds' rotated times: {kinds_sum_us:.1f} us "
        f"(step {ms * 1e3:.1f} us)")
    for key, d in sorted(kernels.items(), key=lambda kv: -kv[1]["us"] * kv[1]["launches"]):
        log(f"[bench] kernel {key}: {d['launches']} launches/step, {d['us']:.2f} us/launch, "
            f"{d['bytes'] / (d['us'] / 1e6) / 1e9:.0f} GB/s")
    dom_key = max(kernels, key=lambda kk: kernels[kk]["us"] * kernels[kk]["launches"])
    dom = kernels[dom_key]
    achieved = dom["bytes"] / (dom["us"] / 1e6) / 1e9

    read_gbs, copy_gbs = measure_ceilings(dev)
    log(f"[bench] ceilings: streaming read {read_gbs:.0f} GB/s, copy {copy_gbs:.0f} GB/s")
    del step  # its 197 matrices: the other steps below allocate their own
    torch.cuda.empty_cache()
    extras = None
    if not args.no_table and args.batch == 1:
        extras = line_extras(args, dev)
    table = None
    if not args.no_table:
        table = shape_table(args.fmt, dev, read_gbs, large=not args.no_large)
    traced = stored_trace(args.fmt, args.batch, args.path, args.schedule)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.fmt, args.batch, args.cpu_seconds)
        log(f"[bench] cpu baseline: {cpu}")

    wfmt = args.fmt.split("_")[0].upper()
    line = {
        "metric": "W4 GEMV achieved HBM GB/s & % roofline; decode-step tok/s (197 GEMVs, B=1)",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if args.fmt.endswith("_f16") else "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"Qwen2.5-1.5B decode step: 197 distinct GEMVs (28x q,k,v,o,gate,"
                         f"up,down + lm_head) in {len(units)} launches, {wfmt} "
                         f"{ {'NF4': 'bs64 fp32 absmax', 'INT4': 'g128 bf16 scale', 'FP4': 'E2M1 bs64 fp32 absmax/6', 'INT4A': 'asymmetric g128 bf16 scale + zero point'}[wfmt]}, "
                         f"{args.fmt.split('_')[1]} x, batch {args.batch}, fp32 accumulate/output"),
            "format": args.fmt,
            "batch": args.batch,
            "path": args.path,
            "schedule": args.schedule,
            "launches_per_step": len(units),
            "other_schedule": {sc: {"ms_per_step": round(t, 5),
                                    "tok_s": round(args.batch * 1e3 / t, 2)}
                               for sc, t in timed.items() if sc != args.schedule},
            "algorithmic_bytes_per_step": total_bytes,
            "step_gbs": round(step_gbs, 1),
            "step_frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4),
            "measured_read_ceiling_gbs": round(read_gbs, 1),
            "measured_copy_ceiling_gbs": round(copy_gbs, 1),
            "step_frac_of_measured_read": round(step_gbs / read_gbs, 4),
            "per_shape_us": {kk: round(r["us"], 3) for kk, r in shapes.items()},
            "per_shape_timing": (f"HIP events over graph replays of each launch kind, rotated over "
                                 f"more than {ROTATE_BYTES >> 20} MiB of distinct weights (the "
                                 f"step's own matrices, then clones), launch to launch"),
            "sum_of_kind_times_us": round(kinds_sum_us, 1),
            "single_gemv_256x1536_us": (next((r["us"] for r in table or [] if r["group"] == "single"
                                              and "us" in r), None)),
            "shape_table": table,
            "other_steps": extras["steps"] if extras else None,
            "down_splitk_us": extras["down_splitk"] if extras else None,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom_key,
            "launches_per_step": dom["launches"],
            "avg_launch_us": round(dom["us"], 3),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(args.fmt, args.batch, args.path, args.schedule, dom_key),
            "timing": "HIP events, rotated graph replays of the kernel's launch kinds, launch to launch",
            "per_kind": {kd: {"launches_per_step": shapes[kd]["count"],
                              "avg_launch_us": round(shapes[kd]["us"], 3),
                              "bytes": shapes[kd]["bytes"],
                              "achieved": round(shapes[kd]["gbs"], 1),
                              "frac": round(shapes[kd]["gbs"] / HBM_PEAK_GBS, 4)}
                         for kd in dom["kinds"]},
            "traced": traced_entry(traced, dom_key, dom) if traced else None,
        },
        "cpu_baseline": cpu,
    }
    if args.report:
        with open(args.report, "w") as f:
            json.dump({"line": line, "shapes": shapes, "kernels": kernels}, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
