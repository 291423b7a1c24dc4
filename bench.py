#!/usr/bin/env python3
"""Benchmark of the FP8-blk GEMV on one MI355X.

Metric: effective weight GB/s (codes + f32 block-scale grid read per second)
and its fraction of the MI355X HBM3E peak (8.0 TB/s).

Default workload (one "step"): the whole-step dense sweep -- 43 layers x
[q 4096x4096, kv 1024x4096, o 4096x4096, gate 2048x4096, up 2048x4096,
down 4096x2048] plus the 129280x4096 head: 259 distinct FP8-blk linears
(~3.2 GB of codes, far above the 256 MB Infinity Cache, so every step reads
cold from HBM), M=1, back to back on one stream. Inputs are drawn on the
device with seeded generators and are resident in HBM before timing.

Launch modes (--mode): "sequence" (default) runs the 259 linears as one
sequence launch -- one persistent kernel that streams them in list order;
"graph" replays one launch per linear from a captured HIP graph; "stream"
enqueues those launches one by one. Every mode computes the same outputs bit
for bit; the JSON line reports the other modes beside the headline.

Output: one JSON line. Besides the headline it carries
  roofline      the dominant kernel's algorithmic bytes per launch / its
                average launch duration (HIP events on the launching stream
                around the timed launches), against the 8 TB/s HBM peak;
  cpu_baseline  the CPU oracle's double-precision GEMV over the same sweep;
  per_config    per-launch times of the single-linear workloads (decode
                shape, projection pair, verify panel at M=1..16), cold from HBM
                (graphs over distinct copies), for the vector and matrix-core
                kernels and their bf16 twins;
  expert_sweep  the native expert arm: one decode step's routed-expert
                projections (43 layers x 8 activated experts x gate 2048x4096,
                up 2048x4096, down 4096x2048 = 1032 FP4 linears, ~4.5 GB) as one
                sequence launch per step, NVFP4 and MXFP4, M = 1 and 8.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "FP8-blk GEMV effective weight GB/s (% of HBM peak), M=1 and M=16"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--mode", choices=("sequence", "graph", "stream"), default="sequence",
                   help="one sequence launch per step (default), or one launch per linear replayed from a captured "
                        "HIP graph, or enqueued one by one")
    p.add_argument("--arm", choices=("fp8", "bf16"), default="fp8", help="time the FP8 arm or the bf16 twin")
    p.add_argument("--layers", type=int, default=43, help="layers in the sweep (default: the full 43)")
    p.add_argument("--no-extra", action="store_true", help="skip the per-config cold-cache table")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-expert", action="store_true", help="skip the native expert arm's sweep")
    p.add_argument("--expert-only", action="store_true",
                   help="run only the native expert arm's sweep (for profiling) and print its JSON")
    p.add_argument("--expert-m", default="1,8", help="panel rows of the expert sweep (comma-separated)")
    p.add_argument("--summarize-expert-trace", nargs=2, metavar=("KERNEL_STATS_CSV", "KERNEL_TRACE_CSV"),
                   help="write the expert kernel's rocprofv3 --stats summary (markdown) and exit")
    p.add_argument("--summarize-expert-counters", nargs=2, metavar=("FETCH_SIZE_CSV", "WRITE_SIZE_CSV"),
                   help="calibrate the expert kernel's FETCH_SIZE / WRITE_SIZE, write its counters JSON, print markdown")
    p.add_argument("--panel-only", action="store_true",
                   help="run only the M-row verify panel sweep (matrix-core sequence launch; for profiling) and "
                        "print its JSON")
    p.add_argument("--chain-only", action="store_true",
                   help="run only the dependent decode chain (graph of launches and the chained launch) and print "
                        "its JSON")
    p.add_argument("--panel-m", default="1,2,4,8,16", help="panel rows of the verify panel sweep (comma-separated)")
    p.add_argument("--summarize-panel-trace", nargs=2, metavar=("KERNEL_STATS_CSV", "KERNEL_TRACE_CSV"),
                   help="write the panel sweep kernel's rocprofv3 --stats summary (markdown) and exit")
    p.add_argument("--summarize-panel-counters", nargs=2, metavar=("FETCH_SIZE_CSV", "WRITE_SIZE_CSV"),
                   help="calibrate the panel sweep kernel's FETCH_SIZE / WRITE_SIZE (one --panel-m value), write "
                        "its counters JSON, print markdown")
    p.add_argument("--reps", type=int, default=10, help="graph replays per config measurement")
    p.add_argument("--config-only", action="store_true",
                   help="run only the per-config cold-launch table (for rocprofv3 runs of those launches)")
    p.add_argument("--manifest", default="",
                   help="with --config-only: write the order and count of the timed GEMV dispatches here")
    p.add_argument("--summarize-config-trace", metavar="KERNEL_TRACE_CSV",
                   help="markdown summary of a --config-only kernel trace (needs --manifest)")
    p.add_argument("--summarize-config-counters", nargs=2, metavar=("FETCH_SIZE_CSV", "WRITE_SIZE_CSV"),
                   help="counter summary of --config-only runs (needs --manifest); writes profiles/")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (a known-size reference for counter runs)")
    p.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_STATS_CSV", "KERNEL_TRACE_CSV"),
                   help="CPU only: print a markdown summary of a rocprofv3 --kernel-trace --stats run and exit")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_SIZE_CSV", "WRITE_SIZE_CSV"),
                   help="CPU only: calibrate two rocprofv3 --pmc runs of --copy-calibration against the 1 GiB "
                        "copy, print a markdown summary, write profiles/gemv_<arm>_m1_sweep_counters.json, exit")
    p.add_argument("--command", default="", help="the command line that produced the CSVs (recorded in summaries)")
    return p.parse_args()


class Sweep:
    """The sweep's linears on the device, load-checked, with prepared calls."""

    def __init__(self, torch, fb, inputs, dev, layers, arm):
        self.plan = inputs.sweep_plan(layers)
        self.dev = dev
        self.xs = {c: inputs.device_x(c, 1, 7 + c, dev) for c in sorted({l.cols for l in self.plan.linears})}
        ws = torch.empty(fb.fp8blk_workspace_bytes(fb.OP_LOAD_CHECK, 1, 16), dtype=torch.uint8, device=dev)
        self.lins = []
        for spec in self.plan.linears:
            codes, scales = inputs.device_linear(spec.rows, spec.cols, spec.seed, dev)
            grid = torch.empty(scales.shape, dtype=torch.float32, device=dev)
            fb.fp8blk_load_check(codes, scales, grid, ws)  # raises on any refusal
            y = torch.empty((1, spec.rows), dtype=torch.float32, device=dev)
            w = codes
            if arm == "bf16":
                w = torch.empty((spec.rows, spec.cols), dtype=torch.int16, device=dev)
                fb.fp8blk_dequant_bf16(codes, grid, w)
                del codes
            self.lins.append(dict(spec=spec, w=w, grid=grid, x=self.xs[spec.cols], y=y, scales=scales))
        torch.cuda.synchronize()
        self.arm = arm
        self.weight_bytes = self.plan.weight_bytes()  # FP8 codes + f32 grid, the metric's bytes
        self.read_bytes = sum(self.algo_bytes(l["spec"]) for l in self.lins)

    def algo_bytes(self, spec):
        """Algorithmic bytes of one launch: weights (codes or bf16 slab), f32
        grid (FP8 arm), x (bf16) and y (f32)."""
        gr, gc = -(-spec.rows // 128), -(-spec.cols // 128)
        wb = spec.rows * spec.cols * (1 if self.arm == "fp8" else 2)
        return wb + (4 * gr * gc if self.arm == "fp8" else 0) + 2 * spec.cols + 4 * spec.rows

    def sequence(self, fb):
        """The sweep's linears as one planned sequence launch (same bits)."""
        if self.arm == "fp8":
            seq = fb.fp8blk_sequence_init(fb.ARM_FP8, [(l["w"], l["grid"], l["x"], l["y"]) for l in self.lins])
            return seq, fb.prepared("fp8blk_gemv_sequence", seq)
        seq = fb.fp8blk_sequence_init(fb.ARM_BF16, [(l["w"], l["x"], l["y"]) for l in self.lins])
        return seq, fb.prepared("bf16_gemv_twin_sequence", seq)

    def calls(self, fb, stream=None):
        out = []
        for l in self.lins:
            if self.arm == "fp8":
                out.append(fb.prepared("fp8blk_gemv", l["w"], l["grid"], l["x"], l["y"], stream=stream))
            else:
                out.append(fb.prepared("bf16_gemv_twin", l["w"], l["x"], l["y"], stream=stream))
        return out

    def calls_grouped(self, fb, stream=None):
        """The same linears with the projections of one input in one launch:
        per layer [q, kv], o, [gate, up], down; then the head."""
        out, k = [], 0
        while k < len(self.lins):
            l = self.lins[k]
            kind = l["spec"].name.split(".")[-1]
            n = 2 if kind in ("q", "gate") else 1
            ls = self.lins[k:k + n]
            if n == 1:
                out += Sweep.calls(_Sub(ls, self.arm), fb, stream)
            elif self.arm == "fp8":
                out.append(fb.prepared("fp8blk_gemv_grouped", [(m["w"], m["grid"], m["y"]) for m in ls], l["x"],
                                       stream=stream))
            else:
                out.append(fb.prepared("bf16_gemv_twin_grouped", [(m["w"], m["y"]) for m in ls], l["x"],
                                       stream=stream))
            k += n
        return out


class _Sub:
    """A subset of a sweep's linears (for per-shape graphs and grouping)."""

    def __init__(self, lins, arm):
        self.lins, self.arm = lins, arm


def run_calls(calls):
    for c in calls:
        st = c()
        if st != 0:
            raise RuntimeError(f"GEMV launch returned status {st}")


def time_sweep(torch, fb, sw, steps, warmup, mode, grouped=False):
    """Wall time of `steps` whole sweeps on one stream, events around all of them."""
    stream = torch.cuda.current_stream()
    make = sw.calls_grouped if grouped else sw.calls
    graph = None
    if mode == "graph":
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            run_calls(make(fb))  # warm the code objects before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            run_calls(make(fb, stream=cap))
        torch.cuda.synchronize()
        step = graph.replay
    else:
        calls = make(fb)
        step = lambda: run_calls(calls)  # noqa: E731
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall


class Chain:
    """The sweep's linears as a dependent decode chain: per layer [q, kv] read
    the layer input, o reads q's output, [gate, up] read o's output, down reads
    gate's output and the next layer reads down's output; the head reads the
    last layer's output. A group is one launch (q + kv and gate + up as one
    grouped launch, "Module dsv4_gpu" page, DecodePath: one launch per
    projection). Between groups a glue step, standing in for the engine's
    norms, attention and activations (not part of this library), writes the
    next input: x = bf16(c * y), one torch kernel, with c fixed per group from
    an eager pass so the values stay near unit scale."""

    def __init__(self, torch, fb, sw, dev):
        self.torch, self.fb, self.sw = torch, fb, sw
        assert sw.arm == "fp8"
        lins = sw.lins
        self.layers = (len(lins) - 1) // 6
        bf = torch.bfloat16
        self.x_in = [torch.empty((1, 4096), dtype=bf, device=dev) for _ in range(self.layers + 1)]
        self.x_in[0].copy_(sw.xs[4096].view(bf))
        self.x_o = [torch.empty((1, 4096), dtype=bf, device=dev) for _ in range(self.layers)]
        self.x_g = [torch.empty((1, 4096), dtype=bf, device=dev) for _ in range(self.layers)]
        self.x_d = [torch.empty((1, 2048), dtype=bf, device=dev) for _ in range(self.layers)]
        self.c = None
        # (kind, members, x): members are sweep linears (dicts with w, grid, y)
        self.groups = []
        for l in range(self.layers):
            q, kv, o, gate, up, down = lins[6 * l:6 * l + 6]
            self.groups += [("launch", [q, kv], self.x_in[l]), ("glue", q["y"], self.x_o[l]),
                            ("launch", [o], self.x_o[l]), ("glue", o["y"], self.x_g[l]),
                            ("launch", [gate, up], self.x_g[l]), ("glue", gate["y"], self.x_d[l]),
                            ("launch", [down], self.x_d[l]), ("glue", down["y"], self.x_in[l + 1])]
        self.groups.append(("launch", [lins[-1]], self.x_in[self.layers]))
        self.n_launches = sum(1 for g in self.groups if g[0] == "launch")
        self.n_glue = len(self.groups) - self.n_launches

    def calls(self, stream=None):
        """The chain's launches and glue steps, in order, as callables."""
        torch, fb = self.torch, self.fb
        out, gi = [], 0
        for kind, a, b in self.groups:
            if kind == "launch":
                if len(a) == 1:
                    out.append(fb.prepared("fp8blk_gemv", a[0]["w"], a[0]["grid"], b, a[0]["y"], stream=stream))
                else:
                    out.append(fb.prepared("fp8blk_gemv_grouped", [(m["w"], m["grid"], m["y"]) for m in a], b,
                                           stream=stream))
            else:
                c = self.c[gi]
                out.append(lambda y=a, x=b, c=c: (torch.mul(y, c, out=x), 0)[1])
                gi += 1
        return out

    def scaled_calls(self, stream=None):
        """The chain's launches with the glue inside them: group gi >= 1 reads
        x = bf16(c * y) of the first member of group gi - 1, formed in the
        kernel's x loads (fp8blk_gemv_scaled_input and its grouped form); the
        first group reads the chain input. No glue kernels."""
        fb = self.fb
        launches = [g for g in self.groups if g[0] == "launch"]
        out = []
        for gi, (_kind, a, x) in enumerate(launches):
            if gi == 0:
                out += self._one("launch", a, x, stream)
                continue
            src, c = launches[gi - 1][1][0]["y"], self.c[gi - 1]
            if len(a) == 1:
                out.append(fb.prepared("fp8blk_gemv_scaled_input", a[0]["w"], a[0]["grid"], src, c, a[0]["y"],
                                       stream=stream))
            else:
                out.append(fb.prepared("fp8blk_gemv_grouped_scaled_input", [(m["w"], m["grid"], m["y"]) for m in a],
                                       src, c, stream=stream))
        return out

    def next_calls(self, stream=None):
        """The chain's launches with the glue in the producer: group gi (but
        the last) also writes the next group's input x = bf16(c * y) of its
        first member beside its outputs (fp8blk_gemv_next_input and its
        grouped form); group gi + 1 reads it as a plain bf16 input."""
        fb = self.fb
        launches = [g for g in self.groups if g[0] == "launch"]
        out = []
        for gi, (_kind, a, x) in enumerate(launches):
            if gi + 1 == len(launches):
                out += self._one("launch", a, x, stream)
                continue
            xn, c = launches[gi + 1][2], self.c[gi]
            if len(a) == 1:
                out.append(fb.prepared("fp8blk_gemv_next_input", a[0]["w"], a[0]["grid"], x, a[0]["y"], c, xn,
                                       stream=stream))
            else:
                out.append(fb.prepared("fp8blk_gemv_grouped_next_input", [(m["w"], m["grid"], m["y"]) for m in a],
                                       x, 0, c, xn, stream=stream))
        return out

    def calibrate(self):
        """Run the chain eagerly once, fixing each glue step's scale so that
        its output has unit root mean square."""
        torch = self.torch
        self.c = [1.0] * self.n_glue
        gi = 0
        for kind, a, b in self.groups:
            if kind == "launch":
                run_calls(Chain._one(self, kind, a, b))
            else:
                rms = float(a.float().pow(2).mean().sqrt())
                self.c[gi] = 1.0 / rms if rms > 0 and rms == rms and rms != float("inf") else 1.0
                torch.mul(a, self.c[gi], out=b)
                gi += 1
        torch.cuda.synchronize()

    def _one(self, kind, a, b, stream=None):
        fb = self.fb
        if len(a) == 1:
            return [fb.prepared("fp8blk_gemv", a[0]["w"], a[0]["grid"], b, a[0]["y"], stream=stream)]
        return [fb.prepared("fp8blk_gemv_grouped", [(m["w"], m["grid"], m["y"]) for m in a], b, stream=stream)]


def persistent_chain(torch, fb, ch):
    """The Chain's launch groups as a fp8blk_gemv_chain plan: group gi >= 1
    reads bf16(c * y) of the first member of group gi - 1, with the glue scale
    the calibration fixed; the first group reads the chain input."""
    launches = [g for g in ch.groups if g[0] == "launch"]
    groups = []
    for gi, (_kind, members, _x) in enumerate(launches):
        mem = [(m["w"], m["grid"], m["y"]) for m in members]
        groups.append((mem, None if gi == 0 else (gi - 1, 0), 1.0 if gi == 0 else ch.c[gi - 1]))
    return fb.fp8blk_chain_init(groups)


def chain_sweep(torch, fb, sw, steps, warmup, dev):
    """Time the dependent chain (Chain) per step, events around `steps`
    steps on the replaying stream: as one HIP graph of launches that also
    write the next group's input (the headline), of launches with glue
    kernels between them, of launches that form their input from the
    previous output, of the launches alone on stale inputs (the floor), and
    as one chained launch (fp8blk_gemv_chain)."""
    ch = Chain(torch, fb, sw, dev)
    ch.calibrate()
    stream = torch.cuda.current_stream()

    def graph_of(calls_of):
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            run_calls(calls_of(None))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            run_calls(calls_of(cap))
        torch.cuda.synchronize()
        for _ in range(max(warmup, 20)):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3

    t = graph_of(lambda st: ch.calls(stream=st))
    v = sw.weight_bytes * steps / t / 1e9
    finite = all(bool(torch.isfinite(l["y"]).all()) for l in sw.lins)
    launches_only = lambda st: [c for (kind, _a, _b), c in zip(ch.groups, ch.calls(stream=st)) if kind == "launch"]  # noqa: E731
    t0 = graph_of(launches_only)
    v0 = sw.weight_bytes * steps / t0 / 1e9
    # the glue inside the launches: each group's kernel forms its x = bf16(c * y) itself
    t1 = graph_of(lambda st: ch.scaled_calls(stream=st))
    v1 = sw.weight_bytes * steps / t1 / 1e9
    f1 = all(bool(torch.isfinite(l["y"]).all()) for l in sw.lins)
    # the glue in the producer: each group's kernel also writes the next group's bf16 input
    t2 = graph_of(lambda st: ch.next_calls(stream=st))
    v2 = sw.weight_bytes * steps / t2 / 1e9
    f2 = all(bool(torch.isfinite(l["y"]).all()) for l in sw.lins)
    # the same chain as one cooperative launch per step (fp8blk_gemv_chain)
    pc = persistent_chain(torch, fb, ch)
    pc_ms = None
    if pc is not None:
        run = lambda: fb.fp8blk_gemv_chain(pc, ch.x_in[0])  # noqa: E731
        for _ in range(max(warmup, 20)):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        pc_ms = e0.elapsed_time(e1) / steps
        pc_status = fb.fp8blk_chain_status(pc)
        pc_finite = all(bool(torch.isfinite(l["y"]).all()) for l in sw.lins)
    log(f"dependent chain ({ch.n_launches} GEMV launches + {ch.n_glue} glue kernels per step, graph): "
        f"{t / steps * 1e3:.4f} ms/step, {v:.1f} GB/s ({100 * v / HBM_PEAK_GBS:.1f}% of peak); outputs finite: {finite}; "
        f"the GEMV launches alone {t0 / steps * 1e3:.4f} ms/step, {v0:.1f} GB/s ({100 * v0 / HBM_PEAK_GBS:.1f}%); "
        f"glue inside the launches (graph) {t1 / steps * 1e3:.4f} ms/step, {v1:.1f} GB/s "
        f"({100 * v1 / HBM_PEAK_GBS:.1f}%); glue in the producer (graph) {t2 / steps * 1e3:.4f} ms/step, "
        f"{v2:.1f} GB/s ({100 * v2 / HBM_PEAK_GBS:.1f}%)"
        + ("" if pc_ms is None else f"; one chained launch {pc_ms:.4f} ms/step, "
           f"{sw.weight_bytes / (pc_ms / 1e3) / 1e9:.1f} GB/s "
           f"({100 * sw.weight_bytes / (pc_ms / 1e3) / 1e9 / HBM_PEAK_GBS:.1f}%), status {pc_status}"))
    # the headline: the glue in the producer (the fastest dependent path with the glue done); the other ways
    # of running the same chain beside it
    return {"value": round(v2, 1), "unit": "GB/s", "pct_hbm_peak": round(100 * v2 / HBM_PEAK_GBS, 2),
            "ms_per_step": round(t2 / steps * 1e3, 4), "gemv_launches_per_step": ch.n_launches,
            "glue_kernels_per_step": 0, "outputs_finite": f2,
            "mode": "each launch but the last also writes the next group's input x = bf16(c*y) beside its outputs "
                    "(fp8blk_gemv_next_input, fp8blk_gemv_grouped_next_input); one HIP graph per step",
            "glue_kernels": {"value": round(v, 1), "unit": "GB/s", "pct_hbm_peak": round(100 * v / HBM_PEAK_GBS, 2),
                             "ms_per_step": round(t / steps * 1e3, 4), "glue_kernels_per_step": ch.n_glue,
                             "outputs_finite": finite,
                             "note": "x = bf16(c*y) written by one torch kernel between the launches"},
            "gemv_launches_alone": {"value": round(v0, 1), "unit": "GB/s",
                                    "pct_hbm_peak": round(100 * v0 / HBM_PEAK_GBS, 2),
                                    "ms_per_step": round(t0 / steps * 1e3, 4),
                                    "note": "the same launches on stale inputs, no glue: the floor of this launch "
                                            "sequence"},
            "glue_in_launches": {"value": round(v1, 1), "unit": "GB/s", "pct_hbm_peak": round(100 * v1 / HBM_PEAK_GBS, 2),
                                 "ms_per_step": round(t1 / steps * 1e3, 4), "launches_per_step": ch.n_launches,
                                 "outputs_finite": f1,
                                 "note": "the same groups, each launch after the first reading x = bf16(c*y) of the "
                                         "previous group's output inside its x loads (fp8blk_gemv_scaled_input, "
                                         "fp8blk_gemv_grouped_scaled_input), no glue kernels, one HIP graph per step"},
            "one_launch": None if pc_ms is None else {
                "value": round(sw.weight_bytes / (pc_ms / 1e3) / 1e9, 1), "unit": "GB/s",
                "pct_hbm_peak": round(100 * sw.weight_bytes / (pc_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
                "ms_per_step": round(pc_ms, 4), "launches_per_step": 1, "status": fb.fp8blk_strerror(pc_status),
                "outputs_finite": pc_finite,
                "note": "fp8blk_gemv_chain: the same groups, inputs x = bf16(c*y) formed inside the launch, one "
                        "cooperative launch per step, events around the timed launches"},
            "workload": "the sweep's 259 linears as a dependent decode chain: per layer [q+kv] -> o -> [gate+up] "
                        "-> down -> next layer, then the head; one launch per group, x = bf16(c*y) between "
                        "groups (standing in for the engine's glue)"}


def time_panel_sequence(torch, fb, inputs, sw, M, steps, warmup, dev):
    """The sweep's linears with an M-row verify panel (one bf16 panel per
    distinct cols, N(0,1)) as one matrix-core sequence launch per step; returns
    seconds for `steps` launches, HIP events on the launching stream."""
    xs = {c: inputs.device_x(c, M, 7 + c, dev) for c in sorted({l["spec"].cols for l in sw.lins})}
    ys = [torch.empty((M, l["spec"].rows), dtype=torch.float32, device=dev) for l in sw.lins]
    if sw.arm == "fp8":
        seq = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(l["w"], l["grid"], xs[l["spec"].cols], y)
                                                        for l, y in zip(sw.lins, ys)])
        call = fb.prepared("fp8blk_gemv_mfma_sequence", seq)
    else:
        seq = fb.fp8blk_sequence_init(fb.ARM_BF16_MFMA, [(l["w"], xs[l["spec"].cols], y) for l, y in zip(sw.lins, ys)])
        call = fb.prepared("bf16_gemv_twin_mfma_sequence", seq)
    stream = torch.cuda.current_stream()
    for _ in range(max(warmup, 50)):  # the set-up above leaves the GPU idle: bring its clocks up first
        run_calls([call])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run_calls([call])
    e1.record(stream)
    torch.cuda.synchronize()
    del seq
    return e0.elapsed_time(e1) / 1e3


def panel_sweep(torch, fb, inputs, sw, dev, steps, warmup, Ms):
    """The verify step's dense traffic: the sweep's linears with an M-row
    panel, one matrix-core sequence launch per step, for each M. Per M: the
    effective weight GB/s (the metric's bytes: codes + f32 grid) and the
    roofline of the launch (algorithmic bytes: weights, each linear's bf16
    panel read once and its f32 outputs written once)."""
    out = {}
    for M in Ms:
        t = time_panel_sequence(torch, fb, inputs, sw, M, steps, warmup, dev)
        v = sw.weight_bytes * steps / t / 1e9
        algo = sum(sw.algo_bytes(l["spec"]) + 2 * (M - 1) * l["spec"].cols + 4 * (M - 1) * l["spec"].rows
                   for l in sw.lins)
        ach = algo * steps / t / 1e9
        out[str(M)] = {"value": round(v, 1), "unit": "GB/s", "pct_hbm_peak": round(100 * v / HBM_PEAK_GBS, 2),
                       "ms_per_step": round(t / steps * 1e3, 4),
                       "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": panel_traffic(sw.arm, M),
                                    "kernel": f"k_mfseq ({sw.arm}), one launch per step",
                                    "avg_launch_us": round(t / steps * 1e6, 2), "avg_algo_bytes_per_launch": algo,
                                    "source_hash": source_hash(PANEL_SOURCES)}}
        log(f"sweep with an M={M} verify panel, matrix-core sequence launch: {t / steps * 1e3:.4f} ms/step, "
            f"{v:.1f} GB/s ({100 * v / HBM_PEAK_GBS:.1f}% of peak); {ach:.1f} GB/s algorithmic")
    return out


def expert_sweep(torch, fb, inputs, dev, steps, warmup, fmt, Ms=(1, 8)):
    """The native expert arm over one decode step's routed-expert projections
    (inputs.expert_sweep_plan: 1032 FP4 linears, each load-checked), one
    sequence launch per step, HIP events on the launching stream. The
    activation of each distinct width is quantized once by fp8blk_act_quant
    (outside the timing; its own per-launch time is reported). Returns a dict
    per M: effective weight GB/s (codes + block scales)."""
    plan = inputs.expert_sweep_plan()
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    lins = []
    for spec in plan:
        codes, scales = inputs.device_fp4_linear(fmt, spec.rows, spec.cols, spec.seed, dev)
        fb.fp4_load_check(fmt, codes, scales, ws)  # raises on any refusal
        lins.append((spec, codes, scales))
    weight_bytes = sum(inputs.fp4_weight_bytes(fmt, sp.rows, sp.cols) for sp, _, _ in lins)
    g = 1.0 if fmt == inputs.MXFP4 else 2.0 ** -6
    stream = torch.cuda.current_stream()
    out = {"format": inputs.FP4_NAMES[fmt], "linears": len(lins), "weight_bytes_per_step": weight_bytes}
    for M in Ms:
        acts = {}
        for c in sorted({sp.cols for sp, _, _ in lins}):
            x = inputs.device_x(c, M, 70 + c, dev)
            xq = torch.empty((M, c), dtype=torch.uint8, device=dev)
            xs = torch.empty((M, c // 128), dtype=torch.uint8, device=dev)
            fb.fp8blk_act_quant(x, xq, xs)
            acts[c] = (x, xq, xs)
        ys = [torch.empty((M, sp.rows), dtype=torch.float32, device=dev) for sp, _, _ in lins]
        seq = fb.fp4_expert_sequence_init(fmt, [(c_, s_, g, acts[sp.cols][1], acts[sp.cols][2], y)
                                                for (sp, c_, s_), y in zip(lins, ys)])
        call = fb.prepared("fp4_expert_sequence", seq)
        for _ in range(max(warmup, 50)):  # the set-up above leaves the GPU idle: bring its clocks up first
            run_calls([call])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            run_calls([call])
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3
        v = weight_bytes * steps / t / 1e9
        # algorithmic bytes of the launch: weights (codes + block scales), each
        # linear's activation codes and scales, and its f32 outputs
        algo = weight_bytes + sum(M * sp.cols + M * (sp.cols // 128) + 4 * M * sp.rows for sp, _, _ in lins)
        ach = algo * steps / t / 1e9
        traffic = expert_traffic(fmt, M)
        r = {"value": round(v, 1), "unit": "GB/s", "pct_hbm_peak": round(100 * v / HBM_PEAK_GBS, 2),
             "ms_per_step": round(t / steps * 1e3, 4),
             "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                          "kernel": f"k_expert ({inputs.FP4_NAMES[fmt]}), one launch per step",
                          "avg_launch_us": round(t / steps * 1e6, 2), "avg_algo_bytes_per_launch": algo,
                          "source_hash": source_hash(EXPERT_SOURCES)}}
        if M == Ms[0]:
            x, xq, xs = acts[4096]
            e0.record(stream)
            for _ in range(100):
                fb.fp8blk_act_quant(x, xq, xs)
            e1.record(stream)
            torch.cuda.synchronize()
            r["act_quant_us_per_call_4096"] = round(e0.elapsed_time(e1) * 10, 2)
        out[f"M{M}"] = r
        log(f"expert sweep {out['format']} M={M}: {r['ms_per_step']} ms/step, {r['value']} GB/s "
            f"({r['pct_hbm_peak']}% of peak)")
        del seq, ys, acts
    del lins
    torch.cuda.synchronize()
    return out


def time_sequence(torch, fb, sw, steps, warmup):
    """Time `steps` sequence launches back to back on the current stream,
    HIP events around all of them (on that stream)."""
    seq, call = sw.sequence(fb)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        run_calls([call])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        run_calls([call])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del seq
    return e0.elapsed_time(e1) / 1e3, wall


def per_shape_launches(torch, fb, sw, reps=10):
    """Average launch duration per distinct shape: a HIP graph of all the
    sweep's linears of that shape (distinct buffers, so still cold), replayed
    `reps` times between events on the replaying stream."""
    stream = torch.cuda.current_stream()
    shapes = {}
    for l in sw.lins:
        key = (l["spec"].name.split(".")[-1], l["spec"].rows, l["spec"].cols)
        shapes.setdefault(key, []).append(l)
    out = []
    for (name, rows, cols), ls in shapes.items():
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            run_calls(Sweep.calls(_Sub(ls, sw.arm), fb, stream=cap))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * len(ls))
        wb = ls[0]["spec"].weight_bytes()
        out.append({"shape": f"{name} {rows}x{cols}", "launches_per_step": len(ls), "us": round(us, 3),
                    "weight_GBps": round(wb / us / 1e3, 1)})
    return out


# The sources each dominant kernel is built from: a counter summary is used
# only while they are unchanged.
SEQ_SOURCES = ("block_scaled_fp8_fp8blk_amd/csrc/fp8blk_seq.hip", "block_scaled_fp8_fp8blk_amd/csrc/fp8blk_device.hpp")
PER_LINEAR_SOURCES = ("block_scaled_fp8_fp8blk_amd/csrc/fp8blk_gemv.hip",
                      "block_scaled_fp8_fp8blk_amd/csrc/fp8blk_device.hpp")


def mode_sources(mode):
    return SEQ_SOURCES if mode == "sequence" else PER_LINEAR_SOURCES


EXPERT_SOURCES = ("block_scaled_fp8_fp8blk_amd/csrc/fp8blk_expert.hip", "block_scaled_fp8_fp8blk_amd/csrc/fp8blk_device.hpp")
PANEL_SOURCES = ("block_scaled_fp8_fp8blk_amd/csrc/fp8blk_mfma.hip", "block_scaled_fp8_fp8blk_amd/csrc/fp8blk_device.hpp")


def source_hash(sources):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def expert_counters_path(M=1):
    return os.path.join(ROOT, "profiles", f"expert_fp4_sweep_m{M}_counters.json")


def expert_traffic(fmt, M=1):
    """HBM bytes per launch of the expert kernel at panel size M from the
    committed counter summary (None when absent or taken on other kernel
    sources)."""
    try:
        with open(expert_counters_path(M)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(EXPERT_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch", {}).get(str(fmt))


def panel_counters_path(arm, M):
    return os.path.join(ROOT, "profiles", f"gemv_{arm}_panel_sweep_m{M}_counters.json")


def panel_traffic(arm, M):
    """HBM bytes per launch of the panel sweep kernel from the committed
    counter summary for this M (None when absent or taken on other sources)."""
    try:
        with open(panel_counters_path(arm, M)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(PANEL_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


def counters_path(arm, mode):
    kind = "sequence" if mode == "sequence" else "per_linear"
    return os.path.join(ROOT, "profiles", f"gemv_{arm}_m1_sweep_{kind}_counters.json")


def counted_traffic(arm, mode):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None when absent or taken on other kernel sources (the
    summary records the source hash it was taken on)."""
    path = counters_path(arm, mode)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(mode_sources(mode)):
        return None
    return rec.get("hbm_bytes_per_launch")


# Kernels of the single-linear GEMV entry points (one dispatch per call).
CONFIG_KERNELS = ("k_gemv_m1<", "k_panel<", "k_mfma<", "k_mfma_shot<")
CONFIG_SOURCES = ("block_scaled_fp8_fp8blk_amd/csrc/fp8blk_gemv.hip", "block_scaled_fp8_fp8blk_amd/csrc/fp8blk_mfma.hip",
                  "block_scaled_fp8_fp8blk_amd/csrc/fp8blk_device.hpp")
CONFIG_ARMS = (("vec", "fp8blk_gemv"), ("vec_twin", "bf16_gemv_twin"), ("mfma", "fp8blk_gemv_mfma"),
               ("mfma_twin", "bf16_gemv_twin_mfma"))


def config_counters_path():
    return os.path.join(ROOT, "profiles", "gemv_per_config_counters.json")


def config_traffic():
    """{(linear, M, arm): HBM bytes per launch} from the committed counter
    summary of the per-config launches ({} when absent or taken on other
    kernel sources)."""
    try:
        with open(config_counters_path()) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    if rec.get("source_hash") != source_hash(CONFIG_SOURCES):
        return {}
    return {(r["linear"], r["M"], r["arm"]): r["hbm_bytes_per_launch"] for r in rec.get("blocks", [])}


def per_config(torch, fb, inputs, dev, reps, manifest=None):
    """Per-launch times of the single-linear workloads (decode shape,
    projection pair, verify panel at M = 1..16), both arms of both kernels.
    Like the sweep: a HIP graph launches the GEMV on enough distinct copies of
    the linear to exceed 512 MB (twice the Infinity Cache), so every launch
    reads cold from HBM, and `reps` replays are timed between events.
    manifest: a list that receives, in launch order, one entry per timed block
    with its number of GEMV dispatches (an eager warm-up pass, one untimed
    replay, `reps` timed replays), so that a profiler's per-dispatch records
    can be assigned to the blocks."""
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    rows_out = []
    counted = config_traffic()

    def timed(make_calls):
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            run_calls(make_calls(None))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            calls = make_calls(cap)
            run_calls(calls)
        torch.cuda.synchronize()
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / (reps * len(calls))

    def add(name, L, Ms):
        codes = torch.from_numpy(L.codes).to(dev)
        scales = torch.from_numpy(L.scales).to(dev)
        grid = torch.empty(scales.shape, dtype=torch.float32, device=dev)
        fb.fp8blk_load_check(codes, scales, grid, ws)
        slab = torch.empty((L.rows, L.cols), dtype=torch.int16, device=dev)
        fb.fp8blk_dequant_bf16(codes, grid, slab)
        copies = max(4, -(-(512 << 20) // (L.rows * L.cols)))
        cs = [codes] + [codes.clone() for _ in range(copies - 1)]
        ss = [slab] + [slab.clone() for _ in range(copies - 1)]
        xall = torch.from_numpy(L.x.view("int16")).to(dev)
        wbytes = L.weight_bytes()
        for M in Ms:
            x = xall[:M].contiguous()
            y = torch.empty((M, L.rows), dtype=torch.float32, device=dev)
            t = {}
            for arm, fn in CONFIG_ARMS:
                ws_ = cs if fn.startswith("fp8blk") else ss
                if fn.startswith("fp8blk"):
                    mk = lambda st, fn=fn, ws_=ws_: [fb.prepared(fn, w, grid, x, y, stream=st) for w in ws_]  # noqa: E731
                else:
                    mk = lambda st, fn=fn, ws_=ws_: [fb.prepared(fn, w, x, y, stream=st) for w in ws_]  # noqa: E731
                t[arm] = timed(mk)
                if manifest is not None:
                    manifest.append({"linear": name, "rows": L.rows, "cols": L.cols, "M": M, "arm": arm,
                                     "dispatches": copies * (reps + 2), "timed_dispatches": copies * reps})
            pct = lambda sec: round(100 * wbytes / sec / 1e9 / HBM_PEAK_GBS, 1)  # noqa: E731
            # algorithmic bytes of one launch: weights (+ grid on the FP8 arms), x, y
            algo = {a: (wbytes if a in ("vec", "mfma") else 2 * L.rows * L.cols) + 2 * M * L.cols + 4 * M * L.rows
                    for a, _ in CONFIG_ARMS}
            rows_out.append(dict(linear=name, rows=L.rows, cols=L.cols, M=M, copies=copies,
                                 us=round(t["vec"] * 1e6, 2), weight_GBps=round(wbytes / t["vec"] / 1e9, 1),
                                 pct_hbm_peak=pct(t["vec"]),
                                 twin_us=round(t["vec_twin"] * 1e6, 2),
                                 twin_GBps=round(2 * L.rows * L.cols / t["vec_twin"] / 1e9, 1),
                                 mfma_us=round(t["mfma"] * 1e6, 2), mfma_GBps=round(wbytes / t["mfma"] / 1e9, 1),
                                 mfma_pct_hbm_peak=pct(t["mfma"]),
                                 mfma_twin_us=round(t["mfma_twin"] * 1e6, 2),
                                 mfma_twin_GBps=round(2 * L.rows * L.cols / t["mfma_twin"] / 1e9, 1),
                                 algo_bytes={a: algo[a] for a, _ in CONFIG_ARMS},
                                 traffic={a: counted.get((name, M, a)) for a, _ in CONFIG_ARMS}))
            r = rows_out[-1]
            log(f"  {name} M={M}: vector arm {r['us']} us, {r['weight_GBps']} GB/s ({r['pct_hbm_peak']}%), twin "
                f"{r['twin_GBps']} GB/s | matrix-core arm {r['mfma_us']} us, {r['mfma_GBps']} GB/s "
                f"({r['mfma_pct_hbm_peak']}%), twin {r['mfma_twin_GBps']} GB/s")
        del cs, ss

    add("decode_4096x4096", inputs.decode_shape(), [1])
    for L in inputs.projection_pair():
        add(L.name, L, [1])
    for L in inputs.verify_panel():
        add(L.name, L, [1] + list(inputs.VERIFY_M))
    return rows_out


BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def prefill(torch, fb, inputs, dev, reps):
    """The staged prefill path (bf16 dequant slab + one hipBLASLt GEMM) on the
    decode-shape and projection linears with a 2048-token bf16 panel: time per
    call of the whole staged path and of the GEMM alone (events around `reps`
    back-to-back calls), as TFLOP/s of 2 N rows cols against the bf16
    matrix-core peak."""
    import numpy as np
    out = []
    rng = np.random.default_rng(11)
    N = 2048
    stream = torch.cuda.current_stream()
    pp = inputs.projection_pair()
    for L in (inputs.decode_shape(), pp[0], pp[2]):
        codes = torch.from_numpy(L.codes).to(dev)
        scales = torch.from_numpy(L.scales).to(dev)
        grid = torch.empty(scales.shape, dtype=torch.float32, device=dev)
        fb.fp8blk_load_check(codes, scales, grid, torch.empty(256, dtype=torch.uint8, device=dev))
        x = torch.from_numpy(inputs.round_to_bf16_bits(rng.standard_normal((N, L.cols), dtype=np.float32))
                             .view(np.int16)).to(dev)
        y = torch.empty((N, L.rows), dtype=torch.float32, device=dev)
        ws = torch.empty(fb.fp8blk_workspace_bytes(fb.OP_GEMM_STAGED, L.rows, L.cols, N), dtype=torch.uint8,
                         device=dev)
        wst = torch.empty(fb.fp8blk_workspace_bytes(fb.OP_BF16_GEMM, L.rows, L.cols, N), dtype=torch.uint8,
                          device=dev)
        slab = torch.empty((L.rows, L.cols), dtype=torch.int16, device=dev)
        fb.fp8blk_dequant_bf16(codes, grid, slab)
        staged = fb.prepared("fp8blk_gemm_staged", codes, grid, x, y, ws)
        gemm = fb.prepared("bf16_gemm_twin", slab, x, y, wst)
        res = {}
        for name, call in (("staged", staged), ("gemm", gemm)):
            run_calls([call] * 3)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_calls([call] * reps)
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / 1e3 / reps
        flops = 2.0 * N * L.rows * L.cols
        r = {"linear": L.name, "rows": L.rows, "cols": L.cols, "tokens": N,
             "staged_us": round(res["staged"] * 1e6, 1), "gemm_us": round(res["gemm"] * 1e6, 1),
             "staged_TFLOPs": round(flops / res["staged"] / 1e12, 1),
             "gemm_TFLOPs": round(flops / res["gemm"] / 1e12, 1),
             "gemm_frac_of_bf16_peak": round(flops / res["gemm"] / 1e12 / BF16_MFMA_PEAK_TFLOPS, 3),
             "dequant_share": round(1 - res["gemm"] / res["staged"], 3)}
        out.append(r)
        log(f"  prefill {L.name} {L.rows}x{L.cols} N={N}: staged {r['staged_us']} us ({r['staged_TFLOPs']} TFLOP/s), "
            f"GEMM alone {r['gemm_us']} us ({r['gemm_TFLOPs']} TFLOP/s, {100 * r['gemm_frac_of_bf16_peak']:.1f}% of "
            f"the bf16 matrix-core peak), dequant share {100 * r['dequant_share']:.1f}%")
        del codes, scales, grid, x, y, ws, wst, slab
    return out


def cpu_baseline(torch, sw, oracle):
    """The oracle's double GEMV (O6) over the sweep's linears, timed on the host
    cores (inputs copied to host memory first, outside the timing)."""
    nthreads = min(16, os.cpu_count() or 1)
    host = []
    for l in sw.lins:
        if sw.arm != "fp8":
            return None
        host.append((l["w"].cpu().numpy(), l["scales"].cpu().numpy(), l["x"].cpu().numpy().view("uint16")))
    times = []
    for _ in range(2):
        t0 = time.perf_counter()
        for codes, scales, x in host:
            oracle.gemv_f64(codes, scales, x, nthreads=nthreads)
        times.append(time.perf_counter() - t0)
    t = min(times)
    return {"value": round(sw.weight_bytes / t / 1e9, 3), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": f"the full sweep ({len(host)} linears, {sw.weight_bytes / 1e9:.2f} GB of weights), double "
                      f"GEMV over {nthreads} host threads, best of 2 passes of {t:.2f} s each or more"}


def _short(name):
    import re
    m = re.search(r"\b(k_\w+(?:<[^>]*>)?)", name)
    return m.group(1) if m else name[:60]


def summarize_trace(stats_csv, trace_csv, command, mode="sequence"):
    """Markdown: per-kernel stats of the FP8-blk kernels and per-shape medians."""
    import csv
    import collections
    title = "one sequence launch per step" if mode == "sequence" else "one launch per linear"
    lines = [f"# rocprofv3 kernel trace: FP8-blk GEMV, whole-step sweep (M=1), {title}", "",
             f"Command: `{command}`" if command else "", "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        if "fp8blk" in r["Name"]:
            lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.1f} | {r['MinNs']} | {r['MaxNs']} |")
    by = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        if "k_gemv_m1" in r["Kernel_Name"] or "k_panel" in r["Kernel_Name"] or "k_seq" in r["Kernel_Name"]:
            by[(_short(r["Kernel_Name"]), int(r["Grid_Size_X"]))].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines += ["", "Per launch shape (kernel<arm, rows per wave, segments per wave, activation rows>, grid = threads; one launch per "
              "linear: q/o 4096x4096, kv 1024x4096, gate/up 2048x4096, down 4096x2048, head 129280x4096; the "
              "sequence kernel: its persistent grid):", "",
              "| kernel | grid | launches | median us | min us |", "|---|---|---|---|---|"]
    for (k, g), v in sorted(by.items(), key=lambda kv: kv[0][1]):
        v.sort()
        lines.append(f"| {k} | {g} | {len(v)} | {v[len(v) // 2] / 1e3:.2f} | {v[0] / 1e3:.2f} |")
    print("\n".join(lines))


def summarize_expert_trace(stats_csv, command, trace_csv=None, M=1):
    """Markdown: rocprofv3 --stats rows of the expert arm's kernels, and the
    median and minimum launch of the expert kernel per format from the
    per-dispatch trace (the stats average includes the warm-up launches)."""
    import csv
    import collections
    names = {"0": "MXFP4", "1": "NVFP4"}
    lines = [f"# rocprofv3 kernel trace: native expert arm, routed-expert sweep (1032 FP4 linears), M={M}", "",
             f"Command: `{command}`" if command else "", "",
             "k_expert<format, tiles, token groups, steps per window, list, single token>; format 0 = MXFP4, 1 = NVFP4. "
             "Each k_expert launch is one whole step (every linear of the sweep).", "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        n = r["Name"]
        if "k_expert" in n or "k_act_quant" in n or "k_fp4" in n:
            short = _short(n)
            if "k_expert<" in short:
                short += f" ({names.get(short.split('<')[1][0], '?')})"
            lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']):.1f} | {r['MinNs']} | {r['MaxNs']} |")
    if trace_csv:
        by = collections.defaultdict(list)
        for r in csv.DictReader(open(trace_csv)):
            if "k_expert<" in r["Kernel_Name"]:
                by[r["Kernel_Name"].split("k_expert<")[1][0]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        lines += ["", "Per dispatch, from the kernel trace:", "", "| kernel | launches | median us | min us |",
                  "|---|---|---|---|"]
        for f, v in sorted(by.items()):
            v.sort()
            lines.append(f"| k_expert ({names.get(f, f)}) | {len(v)} | {v[len(v) // 2] / 1e3:.1f} | {v[0] / 1e3:.1f} |")
    print("\n".join(lines))


def summarize_expert_counters(fetch_csv, write_csv, command, M=1):
    """Calibrate FETCH_SIZE / WRITE_SIZE (KiB per dispatch) against the three
    1 GiB copies of --copy-calibration and give the HBM bytes per launch of
    the expert kernel at panel size M (one --expert-m value per run), per
    format (median over its dispatches)."""
    import csv
    import collections

    def load(path):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][-3:]
        per = collections.defaultdict(list)
        for r in rows:
            n = r["Kernel_Name"]
            if "k_expert<" in n:
                per[n.split("k_expert<")[1][0]].append(float(r["Counter_Value"]))
        return copies, {f: sorted(v)[len(v) // 2] for f, v in per.items()}

    fc, ff = load(fetch_csv)
    wc, wf = load(write_csv)
    gib_kib = 1 << 20
    f_factor = gib_kib / sorted(fc)[len(fc) // 2]
    w_factor = gib_kib / sorted(wc)[len(wc) // 2]
    per = {f: int((ff[f] * f_factor + wf[f] * w_factor) * 1024) for f in ff}
    rec = {"source_hash": source_hash(EXPERT_SOURCES), "M": M, "fetch_factor": round(f_factor, 4),
           "write_factor": round(w_factor, 4), "hbm_bytes_per_launch": per,
           "kib": {f: {"fetch": ff[f], "write": wf[f]} for f in ff}, "command": command}
    with open(expert_counters_path(M), "w") as fh:
        json.dump(rec, fh, indent=1)
    names = {"0": "MXFP4", "1": "NVFP4"}
    lines = [f"# rocprofv3 counters: native expert arm, routed-expert sweep (1032 FP4 linears), M={M}", "",
             f"Command (run once with `--pmc FETCH_SIZE`, once with `--pmc WRITE_SIZE`): `{command}`", "",
             f"Calibration (1 GiB device copy in the same process): FETCH_SIZE x {f_factor:.3f}, "
             f"WRITE_SIZE x {w_factor:.3f} give bytes.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB per launch |", "|---|---|---|---|"]
    for f in sorted(per):
        lines.append(f"| k_expert ({names.get(f, f)}) | {ff[f]:.1f} | {wf[f]:.1f} | {per[f] / 1e6:.3f} |")
    lines += ["", f"Source hash {rec['source_hash']}."]
    print("\n".join(lines))


def summarize_panel_trace(stats_csv, trace_csv, command, M):
    """Markdown: rocprofv3 --stats rows of the matrix-core sequence kernel and
    its per-dispatch median and minimum from the trace (the stats average
    includes the warm-up launches)."""
    import csv
    import collections
    lines = [f"# rocprofv3 kernel trace: verify panel sweep (259 FP8-blk linears, M={M} bf16 panel), one "
             "matrix-core sequence launch per step", "",
             f"Command: `{command}`" if command else "", "",
             "k_mfseq<kind, tiles, panel registers>: kind 0 = FP8 arm. Each launch is one whole step.", "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        if "k_mfseq" in r["Name"]:
            lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.1f} | {r['MinNs']} | "
                         f"{r['MaxNs']} |")
    by = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        if "k_mfseq" in r["Kernel_Name"]:
            by[_short(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines += ["", "Per dispatch, from the kernel trace:", "", "| kernel | launches | median us | min us |",
              "|---|---|---|---|"]
    for k, v in sorted(by.items()):
        v.sort()
        lines.append(f"| {k} | {len(v)} | {v[len(v) // 2] / 1e3:.1f} | {v[0] / 1e3:.1f} |")
    print("\n".join(lines))


def summarize_panel_counters(fetch_csv, write_csv, command, M, arm="fp8"):
    """Calibrate FETCH_SIZE / WRITE_SIZE (KiB per dispatch) against the three
    1 GiB copies of --copy-calibration and give the HBM bytes per launch of
    the matrix-core sequence kernel (median over its dispatches; one panel
    size per run)."""
    import csv

    def load(path):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][-3:]
        v = sorted(float(r["Counter_Value"]) for r in rows if "k_mfseq" in r["Kernel_Name"])
        return copies, v[len(v) // 2]

    fc, fk = load(fetch_csv)
    wc, wk = load(write_csv)
    gib_kib = 1 << 20
    f_factor = gib_kib / sorted(fc)[len(fc) // 2]
    w_factor = gib_kib / sorted(wc)[len(wc) // 2]
    per = int((fk * f_factor + wk * w_factor) * 1024)
    rec = {"source_hash": source_hash(PANEL_SOURCES), "arm": arm, "M": M, "fetch_factor": round(f_factor, 4),
           "write_factor": round(w_factor, 4), "hbm_bytes_per_launch": per,
           "kib": {"fetch": fk, "write": wk}, "command": command}
    with open(panel_counters_path(arm, M), "w") as fh:
        json.dump(rec, fh, indent=1)
    lines = [f"# rocprofv3 counters: verify panel sweep (259 FP8-blk linears, M={M} bf16 panel), one matrix-core "
             "sequence launch per step", "",
             f"Command (run once with `--pmc FETCH_SIZE`, once with `--pmc WRITE_SIZE`): `{command}`", "",
             f"Calibration (1 GiB device copy in the same process): FETCH_SIZE x {f_factor:.3f}, "
             f"WRITE_SIZE x {w_factor:.3f} give bytes.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | written MB | HBM MB per launch |",
             "|---|---|---|---|---|---|",
             f"| k_mfseq ({arm}) | {fk:.1f} | {wk:.1f} | {fk * f_factor * 1024 / 1e6:.3f} | "
             f"{wk * w_factor * 1024 / 1e6:.3f} | {per / 1e6:.3f} |", "",
             f"Source hash {rec['source_hash']}."]
    print("\n".join(lines))


def _config_blocks(rows_by_dispatch, manifest):
    """Assign the GEMV dispatches of a --config-only run, in launch order, to
    the manifest's blocks. rows_by_dispatch: per-dispatch records (dicts with
    Kernel_Name) in dispatch order, every kernel of the run."""
    gemv = [r for r in rows_by_dispatch if any(k in r["Kernel_Name"] for k in CONFIG_KERNELS)]
    need = sum(b["dispatches"] for b in manifest)
    if len(gemv) != need:
        raise SystemExit(f"config summary: {len(gemv)} GEMV dispatches in the profile, {need} in the manifest")
    out, i = [], 0
    for b in manifest:
        out.append(gemv[i:i + b["dispatches"]])
        i += b["dispatches"]
    return out


def summarize_config_trace(trace_csv, manifest_path, command):
    """Markdown: per config block (linear, M, arm), the kernel, its grid and
    the median, p10, p90 and mean duration of the timed launches from a rocprofv3 kernel
    trace of a --config-only run, with the weight GB/s the median gives."""
    import csv
    manifest = json.load(open(manifest_path))
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"]))
    blocks = _config_blocks(rows, manifest)
    lines = ["# rocprofv3 kernel trace: single-linear workloads, cold single launches", "",
             f"Command: `{command}`" if command else "", "",
             "Each launch reads its own copy of the linear (copies > 512 MB in all), so every launch is cold. "
             "Timed launches: the graph replays (the eager warm-up pass and the first replay excluded). Weight "
             "bytes: codes + f32 grid (FP8 arms) or the bf16 slab (twins). vec = fp8blk_gemv, vec_twin = "
             "bf16_gemv_twin, mfma = fp8blk_gemv_mfma, mfma_twin = bf16_gemv_twin_mfma.", "",
             "| linear | M | arm | kernel | grid (threads) | timed launches | median us | p10 us | p90 us | mean us | "
             "weight GB/s (median) | % of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for b, recs in zip(manifest, blocks):
        timed = recs[-b["timed_dispatches"]:]
        d = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed)
        med, mean = d[len(d) // 2] / 1e3, sum(d) / len(d) / 1e3
        p10, p90 = d[len(d) // 10] / 1e3, d[(9 * len(d)) // 10] / 1e3
        gr, gc = -(-b["rows"] // 128), -(-b["cols"] // 128)
        wb = b["rows"] * b["cols"] + 4 * gr * gc if b["arm"] in ("vec", "mfma") else 2 * b["rows"] * b["cols"]
        names = {(_short(r["Kernel_Name"]), r.get("Grid_Size", r.get("Grid_Size_X", "?"))) for r in timed}
        k, g = sorted(names)[0]
        lines.append(f"| {b['linear']} | {b['M']} | {b['arm']} | {k} | {g} | {len(d)} | {med:.2f} | {p10:.2f} | "
                     f"{p90:.2f} | {mean:.2f} | {wb / med / 1e3:.1f} | {100 * wb / med / 1e3 / HBM_PEAK_GBS:.1f} |")
    print("\n".join(lines))


def summarize_config_counters(fetch_csv, write_csv, manifest_path, command):
    """Calibrate FETCH_SIZE / WRITE_SIZE (KiB per dispatch) against the three
    1 GiB copies of --copy-calibration, then give the HBM bytes per launch of
    each config block (median over its dispatches, all cold); writes the JSON
    that bench.py's per_config rows take their traffic from."""
    import csv

    def load(path):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][-3:]
        return copies, _config_blocks(rows, manifest)

    manifest = json.load(open(manifest_path))
    fc, fb_ = load(fetch_csv)
    wc, wb_ = load(write_csv)
    gib_kib = 1 << 20
    f_factor = gib_kib / sorted(fc)[len(fc) // 2]
    w_factor = gib_kib / sorted(wc)[len(wc) // 2]
    recs = []
    lines = ["# rocprofv3 counters: single-linear workloads, cold single launches", "",
             f"Command (run once with `--pmc FETCH_SIZE`, once with `--pmc WRITE_SIZE`): `{command}`", "",
             f"Calibration (1 GiB device copy in the same process): FETCH_SIZE x {f_factor:.3f}, "
             f"WRITE_SIZE x {w_factor:.3f} give bytes. Per block: the median over its dispatches (each reads its "
             "own cold copy). Algorithmic bytes: weights (codes + f32 grid, or the bf16 slab), x and y.", "",
             "| linear | M | arm | read MB | written MB | HBM MB per launch | algorithmic MB | HBM / algorithmic |",
             "|---|---|---|---|---|---|---|---|"]
    for b, fr, wr in zip(manifest, fb_, wb_):
        fk = sorted(float(r["Counter_Value"]) for r in fr)[len(fr) // 2]
        wk = sorted(float(r["Counter_Value"]) for r in wr)[len(wr) // 2]
        rd, wt = fk * f_factor * 1024, wk * w_factor * 1024
        gr, gc = -(-b["rows"] // 128), -(-b["cols"] // 128)
        wbytes = b["rows"] * b["cols"] + 4 * gr * gc if b["arm"] in ("vec", "mfma") else 2 * b["rows"] * b["cols"]
        algo = wbytes + 2 * b["M"] * b["cols"] + 4 * b["M"] * b["rows"]
        recs.append({"linear": b["linear"], "M": b["M"], "arm": b["arm"], "hbm_bytes_per_launch": int(rd + wt),
                     "read_bytes": int(rd), "write_bytes": int(wt), "algo_bytes": algo,
                     "kib": {"fetch": fk, "write": wk}})
        lines.append(f"| {b['linear']} | {b['M']} | {b['arm']} | {rd / 1e6:.3f} | {wt / 1e6:.3f} | "
                     f"{(rd + wt) / 1e6:.3f} | {algo / 1e6:.3f} | {(rd + wt) / algo:.3f} |")
    rec = {"source_hash": source_hash(CONFIG_SOURCES), "fetch_factor": round(f_factor, 4),
           "write_factor": round(w_factor, 4), "blocks": recs, "command": command}
    with open(config_counters_path(), "w") as fh:
        json.dump(rec, fh, indent=1)
    lines += ["", f"Source hash {rec['source_hash']}."]
    print("\n".join(lines))


def m1_launch_key(rows, cols):
    """(kernel instance, grid threads) of fp8blk_gemv's launch for an M = 1
    linear, as the library's plan picks it (rows per wave R, segments per wave
    TPW, waves per row sw; 4-wave workgroups): used to tell the sweep's
    launches apart in counter and trace summaries."""
    T = -(-cols // 1024)
    if T <= 2:
        tpw, R = T, 4 // T
    elif rows < 4096:
        tpw, R = 4, 1
    else:
        tpw, R = (2 if rows >= 16384 and T <= 8 else 4), 2
    sw = 1 if T <= tpw else 2 if T <= 2 * tpw else 4
    blocks = -(-(-(-rows // R)) // (4 // sw))
    return (f"k_gemv_m1<0, {R}, {tpw}, 1>", blocks * 256)


def summarize_counters(fetch_csv, write_csv, command, arm="fp8", mode="sequence"):
    """Calibrate FETCH_SIZE / WRITE_SIZE (KiB per dispatch) against the 1 GiB
    copies of --copy-calibration, then give the HBM bytes per launch of the
    dominant kernel: the sequence kernel (one dispatch per step), or the mean
    over every dispatch of the per-linear kernel. (In the one-launch-per-linear
    run every such dispatch belongs to whole sweep steps: the timed steps, and
    per shape a graph of that shape's launches of one step, replayed, so the
    mix of shapes is that of a step.)"""
    import csv
    import collections

    def load(path):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        # the three 1 GiB calibration copies are the last copy dispatches of the run
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][-3:]
        gem = collections.defaultdict(list)
        for r in rows:
            name = r["Kernel_Name"]
            if mode == "sequence" and "k_seq" in name:
                gem["k_seq"].append(float(r["Counter_Value"]))
            elif mode != "sequence" and "k_gemv_m1<" in name:
                gem[(_short(name), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        return copies, gem

    fc, fg = load(fetch_csv)
    wc, wg = load(write_csv)
    gib_kib = 1 << 20
    f_factor = gib_kib / (sorted(fc)[len(fc) // 2])
    w_factor = gib_kib / (sorted(wc)[len(wc) // 2])
    mean_bytes = {k: (sum(fg[k]) / len(fg[k]) * f_factor + sum(wg[k]) / len(wg[k]) * w_factor) * 1024 for k in fg}
    if mode == "sequence":
        per_step = {"k_seq": 1}
    else:
        # launches of each kernel instance and grid in one sweep step
        per_step = collections.Counter(m1_launch_key(l.rows, l.cols) for l in __import__(
            "block_scaled_fp8_fp8blk_amd.inputs", fromlist=["sweep_plan"]).sweep_plan().linears)
    n = sum(per_step.values())
    tot = sum(per_step[k] * mean_bytes[k] for k in per_step)
    rec = {"source_hash": source_hash(mode_sources(mode)), "arm": arm, "mode": mode, "fetch_factor": round(f_factor, 4),
           "write_factor": round(w_factor, 4), "hbm_bytes_per_launch": int(tot / n),
           "per_dispatch_kib": {str(k): {"launches_per_step": per_step[k], "dispatches_counted": len(fg[k]),
                                         "fetch_mean": sum(fg[k]) / len(fg[k]),
                                         "write_mean": sum(wg[k]) / len(wg[k])} for k in per_step},
           "command": command}
    with open(counters_path(arm, mode), "w") as f:
        json.dump(rec, f, indent=1)
    title = "one sequence launch per step" if mode == "sequence" else "one launch per linear"
    lines = [f"# rocprofv3 counters: FP8-blk GEMV ({arm} arm), whole-step sweep (M=1), {title}", "",
             f"Command (run once with `--pmc FETCH_SIZE`, once with `--pmc WRITE_SIZE`): `{command}`", "",
             f"Calibration (1 GiB device copy in the same process): FETCH_SIZE x {f_factor:.3f}, "
             f"WRITE_SIZE x {w_factor:.3f} give bytes.", "",
             "| kernel | grid (threads) | launches per step | dispatches counted | FETCH_SIZE KiB (mean) | "
             "WRITE_SIZE KiB (mean) | HBM MB per launch |",
             "|---|---|---|---|---|---|---|"]
    for k in sorted(per_step, key=str):
        fm, wm = sum(fg[k]) / len(fg[k]), sum(wg[k]) / len(wg[k])
        kn, grid = (k, "persistent") if k == "k_seq" else k
        lines.append(f"| {kn} | {grid} | {per_step[k]} | {len(fg[k])} | {fm:.1f} | {wm:.1f} | {mean_bytes[k] / 1e6:.3f} |")
    lines += ["", f"Average HBM bytes per launch over one step: {tot / n / 1e6:.3f} MB "
              f"(source hash {rec['source_hash']})."]
    print("\n".join(lines))


def warm_clocks(torch, dev, seconds=0.5):
    """Keep the GPU busy for a moment so that its clocks are up before timing
    (a run that starts with the table would otherwise time its first rows at
    idle clocks)."""
    a = torch.randn(4096, 4096, device=dev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        a = a @ a
        a.div_(a.abs().max())
        torch.cuda.synchronize()
    del a


def copy_calibration(torch, dev):
    """Three 1 GiB device copies: the counter summaries scale FETCH_SIZE and
    WRITE_SIZE by what these read for known bytes."""
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 3 x 1 GiB device copies done")
    del src, dst


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.command, args.mode)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.command, args.arm, args.mode)
        return
    if args.summarize_expert_trace or args.summarize_expert_counters:
        if "," in args.expert_m:
            raise SystemExit("--summarize-expert-*: give the one --expert-m value the profiled runs used")
    if args.summarize_expert_trace:
        summarize_expert_trace(args.summarize_expert_trace[0], args.command, args.summarize_expert_trace[1],
                               int(args.expert_m))
        return
    if args.summarize_expert_counters:
        summarize_expert_counters(*args.summarize_expert_counters, args.command, int(args.expert_m))
        return
    if args.summarize_panel_trace:
        summarize_panel_trace(*args.summarize_panel_trace, args.command, int(args.panel_m))
        return
    if args.summarize_panel_counters:
        summarize_panel_counters(*args.summarize_panel_counters, args.command, int(args.panel_m), args.arm)
        return
    if args.summarize_config_trace:
        summarize_config_trace(args.summarize_config_trace, args.manifest, args.command)
        return
    if args.summarize_config_counters:
        summarize_config_counters(*args.summarize_config_counters, args.manifest, args.command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world > 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus}, WORLD_SIZE {world} requested): the FP8-blk "
              f"GEMV is a single-GPU kernel here, and sharding it over GPUs is a design note, not a run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_fp8_fp8blk_amd as fb
    from block_scaled_fp8_fp8blk_amd import inputs

    fb.load()
    dev = torch.device("cuda:0")
    expert_ms = tuple(int(v) for v in args.expert_m.split(","))
    if args.expert_only:
        res = {f: expert_sweep(torch, fb, inputs, dev, args.steps, args.warmup, f, expert_ms)
               for f in (inputs.NVFP4, inputs.MXFP4)}
        if args.copy_calibration:
            copy_calibration(torch, dev)
        print(json.dumps({"expert_sweep": {inputs.FP4_NAMES[f]: r for f, r in res.items()}}), flush=True)
        return
    if args.config_only:
        warm_clocks(torch, dev)
        manifest = []
        extra = per_config(torch, fb, inputs, dev, args.reps, manifest)
        if args.copy_calibration:
            copy_calibration(torch, dev)
        if args.manifest:
            with open(args.manifest, "w") as f:
                json.dump(manifest, f)
        print(json.dumps({"per_config": extra}), flush=True)
        return
    panel_ms = tuple(int(v) for v in args.panel_m.split(","))
    if args.panel_only:
        sw = Sweep(torch, fb, inputs, dev, args.layers, args.arm)
        panel = panel_sweep(torch, fb, inputs, sw, dev, args.steps, args.warmup, panel_ms)
        if args.copy_calibration:
            copy_calibration(torch, dev)
        print(json.dumps({"panel_sweep_matrix_core_sequence": panel}), flush=True)
        return
    if args.chain_only:
        sw = Sweep(torch, fb, inputs, dev, args.layers, "fp8")
        chain = chain_sweep(torch, fb, sw, args.steps, args.warmup, dev)
        print(json.dumps({"dependent_chain": chain}), flush=True)
        return
    log(f"setting up the sweep ({args.layers} layers + head, arm {args.arm})")
    t0 = time.perf_counter()
    sw = Sweep(torch, fb, inputs, dev, args.layers, args.arm)
    log(f"  {len(sw.lins)} linears, {sw.weight_bytes / 1e9:.3f} GB weights, set up in {time.perf_counter() - t0:.1f} s")

    # The three launch modes over the same linears (same output bits).
    modes = {}
    ssecs, swall = time_sequence(torch, fb, sw, args.steps, args.warmup)
    modes["sequence"] = (ssecs, swall, 1)
    log(f"sweep, one sequence launch: {ssecs / args.steps * 1e3:.4f} ms/step, "
        f"{sw.weight_bytes * args.steps / ssecs / 1e9:.1f} GB/s "
        f"({100 * sw.weight_bytes * args.steps / ssecs / 1e9 / HBM_PEAK_GBS:.1f}% of peak)")
    for m in ("graph", "stream"):
        if m != args.mode and m != "graph":
            continue
        psecs, pwall = time_sweep(torch, fb, sw, args.steps, args.warmup, m)
        modes[m] = (psecs, pwall, len(sw.lins))
        log(f"sweep, one launch per linear ({m}): {psecs / args.steps * 1e3:.4f} ms/step, "
            f"{sw.weight_bytes * args.steps / psecs / 1e9:.1f} GB/s "
            f"({100 * sw.weight_bytes * args.steps / psecs / 1e9 / HBM_PEAK_GBS:.1f}% of peak)")
    gsecs, _ = time_sweep(torch, fb, sw, args.steps, args.warmup, "graph", grouped=True)
    gvalue = sw.weight_bytes * args.steps / gsecs / 1e9
    n_grouped = len(sw.calls_grouped(fb))
    log(f"sweep, shared-input projections grouped ({n_grouped} launches, graph): {gsecs / args.steps * 1e3:.4f} "
        f"ms/step, {gvalue:.1f} GB/s ({100 * gvalue / HBM_PEAK_GBS:.1f}% of peak)")

    secs, wall, launches = modes[args.mode]
    ms_per_step = secs / args.steps * 1e3
    value = sw.weight_bytes * args.steps / secs / 1e9
    log(f"headline ({args.mode}): {ms_per_step:.4f} ms/step, {value:.1f} GB/s "
        f"({100 * value / HBM_PEAK_GBS:.1f}% of peak), host wall {wall:.3f} s")

    # Roofline of the dominant kernel. Sequence mode: one launch per step, the
    # persistent kernel, so the timed region / steps is its average duration.
    # Per-linear modes: the launches run back to back (the kernel trace shows
    # no idle gaps), so the timed region / launches is their average duration.
    avg_launch = secs / (args.steps * launches)
    algo_per_launch = sw.read_bytes / launches
    achieved = algo_per_launch / avg_launch / 1e9
    traffic = counted_traffic(args.arm, args.mode)
    kname = ("k_seq (fp8, 16-slot steps)" if args.arm == "fp8" else "k_seq (bf16 twin, 8-slot steps)") \
        if args.mode == "sequence" else ("k_gemv_m1 (fp8)" if args.arm == "fp8" else "k_gemv_m1 (bf16 twin)")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kname,
            "launches_per_step": launches, "avg_launch_us": round(avg_launch * 1e6, 3),
            "avg_algo_bytes_per_launch": int(algo_per_launch), "source_hash": source_hash(mode_sources(args.mode))}
    log(f"roofline: {kname}, avg launch {roof['avg_launch_us']} us, {achieved:.1f} GB/s algorithmic "
        f"({100 * roof['frac']:.1f}%)")
    shapes = per_shape_launches(torch, fb, sw)
    for r in shapes:
        log(f"  one launch per linear, {r['shape']}: {r['us']} us per launch, {r['weight_GBps']} GB/s")
    launch_modes = {}
    for m, (t, _, nl) in modes.items():
        v = sw.weight_bytes * args.steps / t / 1e9
        launch_modes[m] = {"value": round(v, 1), "unit": "GB/s", "pct_hbm_peak": round(100 * v / HBM_PEAK_GBS, 2),
                           "launches_per_step": nl, "ms_per_step": round(t / args.steps * 1e3, 4)}
    launch_modes["graph_grouped"] = {"value": round(gvalue, 1), "unit": "GB/s", "launches_per_step": n_grouped,
                                     "ms_per_step": round(gsecs / args.steps * 1e3, 4),
                                     "pct_hbm_peak": round(100 * gvalue / HBM_PEAK_GBS, 2),
                                     "note": "q+kv and gate+up each in one launch, graph-replayed"}
    launch_modes["per_linear_shapes"] = shapes

    # The same linears as a dependent decode chain (each group's input is the
    # previous group's output).
    chain = chain_sweep(torch, fb, sw, args.steps, args.warmup, dev) if args.arm == "fp8" else None

    # The verify step's dense traffic: the same linears with an M-row panel, as
    # one matrix-core sequence launch.
    panel = panel_sweep(torch, fb, inputs, sw, dev, args.steps, args.warmup, panel_ms) if not args.no_extra else {}

    if args.copy_calibration:
        copy_calibration(torch, dev)

    extra = None
    pre = None
    if not args.no_extra:
        log("per-config cold-cache table")
        extra = per_config(torch, fb, inputs, dev, args.reps)
        log("staged prefill GEMM")
        pre = prefill(torch, fb, inputs, dev, args.reps)

    cpu = None
    if not args.no_cpu and args.arm == "fp8":
        import oracle
        log("CPU oracle baseline over the sweep")
        cpu = cpu_baseline(torch, sw, oracle)
        if cpu:
            log(f"  oracle: {cpu['value']} GB/s on {cpu['cores']} threads")

    experts = None
    if not args.no_expert:
        experts = {inputs.FP4_NAMES[f]: expert_sweep(torch, fb, inputs, dev, args.steps, args.warmup, f, expert_ms)
                   for f in (inputs.NVFP4, inputs.MXFP4)}

    m16 = [r for r in (extra or []) if r["M"] == 16 and r["rows"] == 12288]
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, drawn on the device; e4m3 codes of N(0,1)*0.05, e8m0 scales in [124,130], "
                "x = bf16 of N(0,1))",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "config": {"workload": f"whole-step dense sweep: {args.layers} x [q 4096x4096, kv 1024x4096, o 4096x4096, "
                               f"gate 2048x4096, up 2048x4096, down 4096x2048] + head 129280x4096; "
                               f"{len(sw.lins)} distinct FP8-blk linears, M=1, back to back on one stream",
                   "launch": args.mode,
                   "arm": args.arm, "M": 1, "linears": len(sw.lins),
                   "weight_bytes_per_step": sw.weight_bytes, "cold_cache": "working set 12x the 256 MB MALL"},
        "roofline": roof,
        "launch_modes": launch_modes,
        "dependent_chain": chain,
        "cpu_baseline": cpu,
        "panel_sweep_matrix_core_sequence": ({"workload": "the same 259 linears, each with an M-row bf16 verify "
                                                          "panel, one matrix-core sequence launch per step",
                                              "by_M": panel} if panel else None),
        "m16_verify_12288x4096": ({"vector_arm": {"weight_GBps": m16[0]["weight_GBps"],
                                                  "pct_hbm_peak": m16[0]["pct_hbm_peak"], "us": m16[0]["us"]},
                                   "matrix_core_arm": {"weight_GBps": m16[0]["mfma_GBps"],
                                                       "pct_hbm_peak": m16[0]["mfma_pct_hbm_peak"],
                                                       "us": m16[0]["mfma_us"]}} if m16 else None),
        "per_config": extra,
        "prefill_staged": pre,
        "expert_sweep": ({"workload": "native expert arm: 43 layers x 8 activated experts x [gate 2048x4096, "
                                      "up 2048x4096, down 4096x2048] = 1032 FP4 linears (codes + block scales), "
                                      "one sequence launch per step; activations quantized per 128 by "
                                      "fp8blk_act_quant", **experts} if experts else None),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
