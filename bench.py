#!/usr/bin/env python3
"""Benchmark of the k-quant matmul hot path on one MI355X.

Metric: Q4_K x q8_1 GEMV weight GB/s (fraction of HBM peak); prefill MMQ int8
TOPS (fraction of int8 MFMA peak).

A step is one Llama-3-8B-shaped decode pass at batch 1 (workload
"llama3_8b_decode_gemv_q4k_b1"): quantise the attention-output input and run
attn-out 4096x4096; quantise the FFN input and run gate and up 14336x4096 as
one launch over their contiguous 28672 rows (one shared q8_1 activation);
quantise the down input and run down 4096x14336.  ``value`` is the weight bytes of that pass (108,527,616) per
second of step time.  The weights rotate over enough device copies that the
footprint exceeds twice the 256 MB Infinity Cache, so every step streams its
weights from HBM.  Inputs are resident in HBM before the timed region.

The other workloads are measured the same way and reported under
``secondary``: batch-4 and batch-8 decode (fused QKV 6144x4096 and down
4096x14336 with residual), the Q6_K output head 128256x4096 (batch 1 and 4), the
Qwen2-7B prefill MMQ at 2048 tokens (Q4_K gate/up 18944x3584, down
3584x18944, QKV 4608x3584; Q6_K v 512x3584 and down 3584x18944), the fused
producers RMSNorm -> q8_1 and SwiGLU -> q8_1
at decode and prefill sizes next to a standalone quantisation, separately
stored q, k, v projections as three launches against one segmented launch,
and the Q6_K launches on the raw layout against the split layout.

The steps are launched as HIP graph replays, each graph holding at least
16 consecutive steps (the weight copies in turn); a replay of a graph costs a
fixed ~6.5 us on the device before its first kernel (measured with the
decode step: 38.8 us per step with one graph per step, 32.3 us with eight
steps per graph, 31.3 us from stream launches in C++), which a graph of one
step would add to every step.  Steps left over from a whole graph run as
one-step graphs.

``roofline`` describes the dominant kernel of the step, kq_gemv_q4k: its
algorithmic bytes per launch (weights + q8_1 activation + f32 output) over
its average launch duration.  Each launch of the step is timed on its own
right after the timed steps: a HIP graph runs it back to back at least 16
times (the weight copies in turn), and HIP events recorded on that stream
around repeated replays, each after an untimed warm-up of the same length,
give the average duration per launch.

``cpu_baseline`` times the CPU oracle on the host cores on the same step and
also reports how far the GPU step outputs are from it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA (5.0 POPS)
MALL_BYTES = 256 * 2 ** 20      # Infinity Cache
GRAPH_MIN = 16                  # steps (or launches) per HIP graph, at least
METRIC = "Q4_K×q8_1 GEMV weight GB/s (% HBM peak); prefill MMQ int8 TOPS (% peak)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copies_for(nbytes: int) -> int:
    """Copies whose footprint exceeds twice the Infinity Cache."""
    return max(2, math.ceil(2.2 * MALL_BYTES / max(nbytes, 1)))


class Workload:
    """Device buffers of one workload plus the launches of one step."""

    def __init__(self, cfg: int, rotate: bool = True):
        import numpy as np
        import torch

        import q6_q8_matmul_amd as kq
        from kq_inputs import WORKLOADS, tensor

        self.kq = kq
        self.cfg = cfg
        self.wl = WORKLOADS[cfg]
        self.ops = [dict(op) for op in self.wl.get("bench_ops", self.wl["ops"])]
        host = {}
        for name, kind, a, b in self.wl["tensors"]:
            host[name] = tensor(cfg, name)
        for op in self.ops:              # row-concatenated weights share one launch
            if isinstance(op["w"], list):
                key = "|".join(op["w"])
                host[key] = np.concatenate([host[n] for n in op["w"]], axis=0)
                op["w"] = key
        self.host = host
        wnames = sorted({op["w"] for op in self.ops})
        self.weight_bytes_step = sum(host[op["w"]].nbytes for op in self.ops)
        unique_w = sum(host[n].nbytes for n in wnames)
        self.ncopies = copies_for(unique_w) if rotate else 1
        self.w = [{n: torch.from_numpy(host[n]).cuda() for n in wnames}]
        for _ in range(self.ncopies - 1):
            self.w.append({n: t.clone() for n, t in self.w[0].items()})
        self.x = {}
        self.xq = {}
        for op in self.ops:
            xn = op["x"]
            if xn not in self.x:
                self.x[xn] = torch.from_numpy(host[xn]).cuda()
                rows, k = host[xn].shape
                self.xq[xn] = torch.empty((rows, k // 32 * 36), dtype=torch.uint8, device="cuda")
        self.res = {}
        self.y = []
        self.ws = {}
        for i, op in enumerate(self.ops):
            if op["op"] in ("mmq_q4k", "mmq_q6k"):
                fn = kq.kq_mmq_q4k_workspace_bytes if op["op"] == "mmq_q4k" else kq.kq_mmq_q6k_workspace_bytes
                nb = fn(op["m"], op["n"], op["k"])
                self.ws[i] = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        for op in self.ops:
            rows = op.get("batch", op.get("n"))
            self.y.append(torch.empty((rows, op["m"]), dtype=torch.float32, device="cuda"))
            if "residual" in op:
                self.res[op["residual"]] = torch.from_numpy(host[op["residual"]]).cuda()
        torch.cuda.synchronize()

    def launch_fn(self, i: int, w):
        """The launch of op i on weight tensor w."""
        kq = self.kq
        op = self.ops[i]
        xq = self.xq[op["x"]]
        y = self.y[i]
        if op["op"] == "gemv_q4k" or op["op"] == "gemv_q6k":
            res = self.res.get(op.get("residual"))
            fn = kq.kq_gemv_q4k if op["op"] == "gemv_q4k" else kq.kq_gemv_q6k
            return lambda: fn(w, xq, y, res, op["m"], op["k"], op["batch"])
        ws = self.ws[i]
        if op["op"] == "mmq_q6k":          # the K split when the product is small
            return lambda: kq.kq_mmq_q6k_ws(w, xq, y, op["m"], op["n"], op["k"], ws, ws.numel())
        # Q4_K: the K split where tiles leave CUs idle
        return lambda: kq.kq_mmq_q4k_ws(w, xq, y, op["m"], op["n"], op["k"], ws, ws.numel())

    def launches(self, c: int):
        """(label, kind, callable) for every launch of one step on copy c."""
        kq = self.kq
        out = []
        done = set()
        for i, op in enumerate(self.ops):
            xn = op["x"]
            if xn not in done:
                x, xq = self.x[xn], self.xq[xn]
                rows, k = x.shape
                out.append((f"quantize {xn}", "quantize",
                            lambda x=x, xq=xq, rows=rows, k=k: kq.kq_quantize_q8_1(x, xq, rows, k)))
                done.add(xn)
            out.append((op["label"], op["op"], self.launch_fn(i, self.w[c][op["w"]])))
        return out

    def launch_rotation(self, label: str):
        """The callables that time launch `label` on its own: one per copy
        of its weight tensor, enough copies that their footprint exceeds
        twice the Infinity Cache (the step's copies, plus clones), so every
        launch streams its weights from HBM; a quantisation has one."""
        for i, op in enumerate(self.ops):
            if op["label"] == label:
                name = op["w"]
                n = max(self.ncopies, copies_for(self.host[name].nbytes))
                ws = [self.w[c][name] for c in range(self.ncopies)]
                ws += [ws[0].clone() for _ in range(n - len(ws))]
                return [self.launch_fn(i, w) for w in ws]
        return [fn for lab, _, fn in self.launches(0) if lab == label]

    def step(self, c: int):
        for _, _, fn in self.launches(c):
            fn()

    def op_bytes(self, i: int) -> int:
        """Algorithmic bytes of op i: weights + q8_1 activation + f32 output
        (+ f32 residual read)."""
        op = self.ops[i]
        rows = op.get("batch", op.get("n"))
        b = self.host[op["w"]].nbytes + rows * (op["k"] // 32) * 36 + rows * op["m"] * 4
        if "residual" in op:
            b += rows * op["m"] * 4
        return b

    def op_ops(self, i: int) -> float:
        op = self.ops[i]
        rows = op.get("batch", op.get("n"))
        return 2.0 * op["m"] * rows * op["k"]


def cycle_len(ncopies: int) -> int:
    """Steps (or launches) per graph: whole rounds of the weight copies, at
    least GRAPH_MIN."""
    return ncopies * math.ceil(GRAPH_MIN / ncopies)


def build_graphs(wl: Workload):
    """A graph of cycle_len(ncopies) consecutive steps (copy i % ncopies for
    step i) and one graph per copy of a single step, for a remainder."""
    import torch

    side = torch.cuda.Stream()
    spg = cycle_len(wl.ncopies)
    many = torch.cuda.CUDAGraph()
    with torch.cuda.graph(many, stream=side):
        for i in range(spg):
            wl.step(i % wl.ncopies)
    single = []
    for c in range(wl.ncopies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            wl.step(c)
        single.append(g)
    torch.cuda.synchronize()
    return {"steps_per_graph": spg, "many": many, "single": single}


def run_steps(wl: Workload, n: int, graphs=None):
    """Steps 0..n-1 (copy i % ncopies for step i): whole multi-step graphs,
    then one-step graphs for the rest; without graphs, eager launches."""
    i = 0
    while i < n:
        if graphs is None:
            wl.step(i % wl.ncopies)
            i += 1
        elif n - i >= graphs["steps_per_graph"]:
            graphs["many"].replay()
            i += graphs["steps_per_graph"]
        else:
            graphs["single"][i % wl.ncopies].replay()
            i += 1


def timed_steps(wl: Workload, steps: int, warmup: int, graphs=None):
    """Wall time per step (ms) over `steps` steps bracketed by events and
    synchronisation; weights rotate over the copies."""
    import torch

    run_steps(wl, warmup, graphs)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    run_steps(wl, steps, graphs)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def kernel_durations(wl: Workload, target_ms: float = 10.0, rounds: int = 5,
                     warm_ms: float = 50.0):
    """Duration (ms) of every launch of the step.  For each launch a HIP graph
    holds it cycle_len(n) times over n copies of its own weight tensor
    (Workload.launch_rotation: enough copies that every launch streams from
    HBM), back to back on one stream.  In each of
    `rounds` interleaved rounds every launch's graph is replayed between two
    HIP events recorded on the stream the kernels run on, and the elapsed
    time is divided by the launch count (after an untimed warm-up of at least
    warm_ms of the same graph); in the same round the same launches
    are also issued straight to that stream, back to back between two events
    (a graph's kernel nodes start a few microseconds apart, which a long
    kernel's per-launch figure otherwise carries; short kernels are limited
    by the host's launch rate there instead).  Returns (label, kind, mean,
    median, min) of the graph figures and the median of the stream figures
    over the rounds."""
    import torch

    side = torch.cuda.Stream()
    launches = wl.launches(0)
    fns = [wl.launch_rotation(label) for label, _, _ in launches]
    nper = [cycle_len(len(f)) for f in fns]       # launches per graph
    graphs = []
    for j in range(len(launches)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(nper[j]):
                fns[j][i % len(fns[j])]()
        graphs.append(g)
    stream = torch.cuda.current_stream()
    reps, warm = [], []
    for g in graphs:
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        t_graph = max(a.elapsed_time(b), 1e-3)
        reps.append(max(3, min(200, int(target_ms / t_graph))))
        warm.append(max(reps[-1], math.ceil(warm_ms / t_graph)))
    per = [[] for _ in graphs]
    per_s = [[] for _ in graphs]
    for _ in range(rounds):
        for j, g in enumerate(graphs):
            # untimed warm-up of at least warm_ms: the measured launch of a
            # round follows other (often light) launches, and a heavy kernel
            # right after them ran slower for a while (the head 128256x4096:
            # 84-87 against 79.5 us, converging after ~0.1 s of it)
            for _ in range(warm[j]):
                g.replay()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps[j]):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            per[j].append(a.elapsed_time(b) / (reps[j] * nper[j]))
            a.record(stream)
            for _ in range(reps[j]):
                for i in range(nper[j]):
                    fns[j][i % len(fns[j])]()
            b.record(stream)
            torch.cuda.synchronize()
            per_s[j].append(a.elapsed_time(b) / (reps[j] * nper[j]))
    out = []
    for j, (label, kind, _) in enumerate(launches):
        v = sorted(per[j])
        vs = sorted(per_s[j])
        out.append((label, kind, sum(v) / len(v), v[len(v) // 2], v[0], vs[len(vs) // 2]))
    del graphs, fns
    torch.cuda.empty_cache()
    return out


def _graph_time_ms(fn, target_ms: float = 20.0, per_graph: int = GRAPH_MIN):
    """Average duration (ms) of fn(): a HIP graph holds per_graph launches back
    to back; it is replayed between two events on the launching stream."""
    import torch

    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(per_graph):
            fn()
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    reps = max(3, min(500, int(target_ms / max(a.elapsed_time(b), 1e-3))))
    for _ in range(reps):           # untimed warm-up of the same length
        g.replay()
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * per_graph)


def _stream_time_ms(fn, target_ms: float = 20.0, per_round: int = GRAPH_MIN):
    """Average duration (ms) of fn() issued straight to the current stream,
    per_round calls back to back per repetition, between two events."""
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(per_round):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(per_round):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    reps = max(3, min(500, int(target_ms / max(a.elapsed_time(b), 1e-3))))
    for _ in range(reps * per_round):   # untimed warm-up of the same length
        fn()
    a.record(stream)
    for _ in range(reps * per_round):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * per_round)


def measure_producers(cfg: int):
    """Fused producers (RMSNorm -> q8_1, SwiGLU -> q8_1) of workload cfg, each
    timed alone, with the f32 output written and with q8_1 only, next to the
    standalone quantisation of an activation of the same size.  Inputs stay
    in the caches between back-to-back launches (they are small next to the
    weight streams)."""
    import torch

    import q6_q8_matmul_amd as kq
    from kq_inputs import WORKLOADS, tensor

    wl = WORKLOADS[cfg]
    t = {name: torch.from_numpy(tensor(cfg, name)).cuda() for name, *_r in wl["tensors"]}
    out = []
    for op in wl["ops"]:
        rows, n = op["rows"], op["n"]
        xq = torch.empty((rows, n // 32 * 36), dtype=torch.uint8, device="cuda")
        xq2 = torch.empty_like(xq)
        y = torch.empty((rows, n), dtype=torch.float32, device="cuda")
        if op["op"] == "rmsnorm_q8_1":
            x, res, g = t[op["x"]], t[op["res"]], t[op["g"]]
            fused = lambda yy: kq.kq_rmsnorm_q8_1(x, res, g, op["eps"], yy, xq, rows, n)
            read = 2 * rows * n * 4 + n * 4
        else:
            gate, up = t[op["gate"]], t[op["up"]]
            fused = lambda yy: kq.kq_swiglu_q8_1(gate, up, yy, xq, rows, n)
            read = 2 * rows * n * 4
        fused(y)
        torch.cuda.synchronize()
        ms_y = _graph_time_ms(lambda: fused(y))
        ms_q = _graph_time_ms(lambda: fused(None))
        ms_quant = _graph_time_ms(lambda: kq.kq_quantize_q8_1(y, xq2, rows, n))
        qbytes = rows * n // 32 * 36
        out.append({"op": op["label"], "kernel": "kq_" + op["op"], "shape": [rows, n],
                    "avg_us": round(ms_y * 1e3, 2),
                    "GBps": round((read + rows * n * 4 + qbytes) / (ms_y * 1e-3) / 1e9, 1),
                    "avg_us_q8_1_only": round(ms_q * 1e3, 2),
                    "standalone_quantize_avg_us": round(ms_quant * 1e3, 2)})
    return {"workload": wl["name"], "kernels": out,
            "note": "inputs cache-resident between back-to-back launches"}


def measure_segmented(cfg: int):
    """Workload cfg's GEMVs share one activation: time them as separate
    launches and as one segmented launch (kq_gemv_q4k_seg), each replayed as a
    HIP graph over rotating weight copies."""
    import torch

    import q6_q8_matmul_amd as kq
    from kq_inputs import WORKLOADS, tensor

    wl = WORKLOADS[cfg]
    ops = wl["ops"]
    host = {op["w"]: tensor(cfg, op["w"]) for op in ops}
    nbytes = sum(h.nbytes for h in host.values())
    ncopy = copies_for(nbytes)
    copies = [{n: torch.from_numpy(h).cuda() for n, h in host.items()}]
    for _ in range(ncopy - 1):
        copies.append({n: t.clone() for n, t in copies[0].items()})
    x = torch.from_numpy(tensor(cfg, ops[0]["x"])).cuda()
    xq = kq.quantize_q8_1(x)
    k, batch = ops[0]["k"], ops[0]["batch"]
    ys = [torch.empty((batch, op["m"]), dtype=torch.float32, device="cuda") for op in ops]
    ms = [op["m"] for op in ops]

    def run(c, seg):
        ws = [copies[c][op["w"]] for op in ops]
        if seg:
            kq.kq_gemv_q4k_seg(ws, ms, ys, None, xq, k, batch)
        else:
            for w, y, m in zip(ws, ys, ms):
                kq.kq_gemv_q4k(w, xq, y, None, m, k, batch)

    out = {}
    for seg in (False, True):
        run(0, seg)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for c in range(ncopy):
                run(c, seg)
        stream = torch.cuda.current_stream()
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(20):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / (20 * ncopy) * 1e3
        out["one_segmented_launch" if seg else "separate_launches"] = {
            "us": round(us, 2), "weight_GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    return {"workload": wl["name"], "weight_bytes": nbytes, "weight_copies": ncopy, **out}


def measure_split(cfg: int):
    """The Q6_K launches of workload cfg on the raw layout and on the split
    layout (kq_repack_q6k once at load), each replayed as a HIP graph over
    rotating weight copies."""
    import torch

    import q6_q8_matmul_amd as kq
    from kq_inputs import WORKLOADS, tensor

    wl = WORKLOADS[cfg]
    out = []
    for op in wl["ops"]:
        m, k = op["m"], op["k"]
        rows = op.get("batch", op.get("n"))
        h = tensor(cfg, op["w"])
        ncopy = copies_for(h.nbytes)
        raw = [torch.from_numpy(h).cuda()]
        raw += [raw[0].clone() for _ in range(ncopy - 1)]
        split = [kq.repack_q6k(r, m, k) for r in raw]
        xq = kq.quantize_q8_1(torch.from_numpy(tensor(cfg, op["x"])).cuda())
        y = torch.empty((rows, m), dtype=torch.float32, device="cuda")
        e = {"op": op["label"], "shape": [m, k, rows]}
        for name, ws in (("raw", raw), ("split", split)):
            if op["op"] == "gemv_q6k":
                fn = kq.kq_gemv_q6k if name == "raw" else kq.kq_gemv_q6k_split
                launch = lambda w, fn=fn: fn(w, xq, y, None, m, k, rows)
            else:
                fn = kq.kq_mmq_q6k if name == "raw" else kq.kq_mmq_q6k_split
                launch = lambda w, fn=fn: fn(w, xq, y, m, rows, k)
            it = iter(range(1 << 30))
            us = _graph_time_ms(lambda: launch(ws[next(it) % ncopy]), per_graph=cycle_len(ncopy)) * 1e3
            us_s = _stream_time_ms(lambda: launch(ws[next(it) % ncopy]), per_round=cycle_len(ncopy)) * 1e3
            e[f"{name}_us"] = round(us, 2)
            e[f"{name}_stream_us"] = round(us_s, 2)
            if op["op"] == "gemv_q6k":
                e[f"{name}_weight_GBps"] = round(h.nbytes / (us * 1e-6) / 1e9, 1)
                e[f"{name}_stream_weight_GBps"] = round(h.nbytes / (us_s * 1e-6) / 1e9, 1)
            else:
                e[f"{name}_tops"] = round(2.0 * m * rows * k / (us * 1e-6) / 1e12, 1)
                e[f"{name}_stream_tops"] = round(2.0 * m * rows * k / (us_s * 1e-6) / 1e12, 1)
        out.append(e)
        del raw, split
        torch.cuda.empty_cache()
    return {"workload": wl["name"], "layouts": out}


class ClockPower:
    """Engine clock and board power sampled from the driver's sysfs files
    while a workload runs: the current level of pp_dpm_sclk (the line marked
    '*') and hwmon power1_input (microwatts), every `period` seconds on a
    helper thread.  The summary keeps the samples taken while the engine
    clock was above its idle level."""

    def __init__(self, period: float = 0.02):
        import glob
        import threading

        self.period = period
        self.samples = []
        self.sclk = self.power = None
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            if os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
                self.sclk = os.path.join(dev, "pp_dpm_sclk")
                pw = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_input")))
                self.power = pw[0] if pw else None
                break
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        mhz = watts = None
        try:
            for line in open(self.sclk):
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", line, flags=re.I)
                    mhz = int(m.group(1)) if m else None
            if self.power:
                watts = int(open(self.power).read().strip()) / 1e6
        except (OSError, ValueError):
            pass
        return mhz, watts

    def _run(self):
        while not self._stop.is_set():
            self.samples.append(self._read())
            self._stop.wait(self.period)

    def __enter__(self):
        if self.sclk:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.sclk:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.sclk:
            return {"source": None, "note": "no pp_dpm_sclk under /sys/class/drm"}
        busy = [(c, w) for c, w in self.samples if c is not None and c > 500]
        out = {"source": f"{self.sclk} ('*' level), {self.power} (uW)",
               "samples": len(self.samples), "busy_samples": len(busy)}
        if busy:
            cs = sorted(c for c, _ in busy)
            ws = sorted(w for _, w in busy if w is not None)
            out.update({"sclk_MHz_median": cs[len(cs) // 2], "sclk_MHz_min": cs[0],
                        "sclk_MHz_max": cs[-1]})
            if ws:
                out.update({"power_W_median": round(ws[len(ws) // 2], 1),
                            "power_W_max": round(ws[-1], 1)})
        return out


def measure_ksplit(cfg: int):
    """The prefill products of workload cfg that the K split applies to,
    without a workspace (kq_mmq_q4k / kq_mmq_q6k) and with the workspace the
    split asks for (kq_mmq_q4k_ws / kq_mmq_q6k_ws), each replayed as a HIP
    graph over rotating weight copies."""
    import torch

    import q6_q8_matmul_amd as kq
    from kq_inputs import WORKLOADS, tensor

    wl = WORKLOADS[cfg]
    out = []
    for op in wl["ops"]:
        if not op["op"].startswith("mmq"):
            continue
        q4 = op["op"] == "mmq_q4k"
        plain = kq.kq_mmq_q4k if q4 else kq.kq_mmq_q6k
        split = kq.kq_mmq_q4k_ws if q4 else kq.kq_mmq_q6k_ws
        wsb = kq.kq_mmq_q4k_workspace_bytes if q4 else kq.kq_mmq_q6k_workspace_bytes
        m, n, k = op["m"], op["n"], op["k"]
        nb = wsb(m, n, k)
        if nb == 0:                       # not split: nothing to compare
            continue
        h = tensor(cfg, op["w"])
        ncopy = copies_for(h.nbytes)
        ws_ = [torch.from_numpy(h).cuda()]
        ws_ += [ws_[0].clone() for _ in range(ncopy - 1)]
        xq = kq.quantize_q8_1(torch.from_numpy(tensor(cfg, op["x"])).cuda())
        y = torch.empty((n, m), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        e = {"op": op["label"], "kernel": "kq_" + op["op"], "shape": [m, k, n], "workspace_bytes": nb}
        for name, launch in (("no_workspace", lambda w: plain(w, xq, y, m, n, k)),
                             ("k_split", lambda w: split(w, xq, y, m, n, k, ws, nb))):
            it = iter(range(1 << 30))
            us = _graph_time_ms(lambda: launch(ws_[next(it) % ncopy]), per_graph=cycle_len(ncopy)) * 1e3
            e[f"{name}_us"] = round(us, 2)
            e[f"{name}_tops"] = round(2.0 * m * n * k / (us * 1e-6) / 1e12, 1)
        out.append(e)
        del ws_, ws
        torch.cuda.empty_cache()
    return {"workload": wl["name"], "products": out}


def measure(cfg: int, steps: int, warmup: int, use_graph: bool):
    import torch

    wl = Workload(cfg)
    wl.step(0)                      # first calls outside any capture
    torch.cuda.synchronize()
    graphs = build_graphs(wl) if use_graph else None
    with ClockPower() as cp:
        ms = timed_steps(wl, steps, warmup, graphs)
        durs = kernel_durations(wl)
    del graphs
    return wl, ms, durs, cp.summary()


# Forms of kq_read_probe swept for the read ceiling: (workgroups per CU, 0
# for one workgroup per chunk; 16-byte loads in flight per thread).
PROBE_FORMS = [(0, u) for u in (4, 8, 16, 32)] + [(w, u) for w in (1, 2, 3, 4, 8) for u in (8, 16, 32)]


def _probe_label(form):
    w, u = form
    return f"one-shot, {u} loads/thread" if w == 0 else f"persistent {w} WG/CU, {u} loads/thread"


def _cus() -> int:
    import torch

    return torch.cuda.get_device_properties(0).multi_processor_count


def stream_read_ceiling(nbytes: int = 2 << 30, reps: int = 10):
    """Measured streaming-read ceiling of the device: every form of
    kq_read_probe in PROBE_FORMS (one-shot and persistent grids, 4 to 32
    16-byte loads in flight per thread) over a 2 GiB buffer, larger than the
    Infinity Cache, event-timed, median of `reps` launches each; the best
    form is the ceiling.  The 8 TB/s spec peak stays the roofline; this is
    the practical read rate beside it."""
    import torch

    import q6_q8_matmul_amd as kq

    cus = _cus()
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sweep = {}
    for form in PROBE_FORMS:
        grid = form[0] * cus
        out = torch.empty(kq.kq_read_probe_words(nbytes, grid, form[1]), dtype=torch.int32, device="cuda")
        for _ in range(2):
            kq.kq_read_probe(buf, nbytes, out, grid, form[1], stream.cuda_stream)
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            kq.kq_read_probe(buf, nbytes, out, grid, form[1], stream.cuda_stream)
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        t = sorted(ts)[len(ts) // 2]
        sweep[_probe_label(form)] = round(nbytes / t / 1e9, 1)
        del out
    del buf
    torch.cuda.empty_cache()
    best = max(sweep, key=sweep.get)
    return {"GBps": sweep[best], "form": best, "bytes": nbytes, "sweep_GBps": sweep,
            "how": "kq_read_probe over 2 GiB in every form of the sweep (one-shot and persistent "
                   "grids, 4-32 16-byte loads in flight per thread), median of 10 event-timed "
                   "launches each; the best form is the ceiling"}


def read_floors_us(wl: Workload):
    """Per GEMV launch of the step, the least time any kq_read_probe form of
    PROBE_FORMS takes to read the same weight tensor, rotated over the same
    number of copies as the launch's own timing and timed the same way
    (graph replays of whole rounds of the copies).  Returns {label: (us, form)}."""
    import torch

    import q6_q8_matmul_amd as kq

    cus = _cus()
    out = {}
    for op in wl.ops:
        if not op["op"].startswith("gemv"):
            continue
        n = max(wl.ncopies, copies_for(wl.host[op["w"]].nbytes))
        bufs = [wl.w[c][op["w"]] for c in range(wl.ncopies)]
        bufs += [bufs[0].clone() for _ in range(n - len(bufs))]
        nbytes = bufs[0].numel() // 16 * 16
        best = None
        for form in PROBE_FORMS:
            grid = form[0] * cus
            res = torch.empty(kq.kq_read_probe_words(nbytes, grid, form[1]), dtype=torch.int32, device="cuda")
            launches = [lambda b=b: kq.kq_read_probe(b, nbytes, res, grid, form[1]) for b in bufs]
            ms = _graph_time_ms(lambda: [f() for f in launches], target_ms=5.0,
                                per_graph=cycle_len(len(launches)) // len(launches)) / len(launches)
            if best is None or ms < best[0]:
                best = (ms, form)
            del res
        out[op["label"]] = (round(best[0] * 1e3, 2), _probe_label(best[1]))
        del bufs
        torch.cuda.empty_cache()
    return out


def _cpu_model() -> dict:
    """lscpu's model fields of the host (under a hypervisor the model name
    may be generic; family/model/stepping still identify the part)."""
    import subprocess

    out = {}
    try:
        text = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in text.splitlines():
            key, _, val = line.partition(":")
            key = key.strip()
            if key in ("Model name", "Vendor ID", "CPU family", "Model", "Stepping",
                       "Hypervisor vendor", "CPU(s)"):
                out[key] = val.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    if "Model name" not in out:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    out["Model name"] = line.split(":", 1)[1].strip()
                    break
        except OSError:
            out["Model name"] = "unknown"
    return out


def cpu_baseline(wl: Workload, seconds: float):
    """The oracle on the host: the same step (quantise + every matmul of the
    workload) repeated until `seconds` have passed; also the GPU step
    outputs compared with the oracle's."""
    import numpy as np
    import torch

    import oracle

    oracle.build(force=False)
    threads = oracle.max_threads()

    def one_step():
        xq = {xn: oracle.quantize_q8_1(wl.host[xn]) for xn in wl.x}
        outs = []
        for op in wl.ops:
            kind = "q4k" if op["op"].endswith("q4k") else "q6k"
            rows = op.get("batch", op.get("n"))
            res = wl.host.get(op.get("residual")) if "residual" in op else None
            outs.append(oracle.matmul(kind, wl.host[op["w"]], xq[op["x"]], op["m"], rows, op["k"],
                                      residual=res))
        return xq, outs

    def timed(budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            got = one_step()
            reps += 1
            if time.perf_counter() - t0 >= budget:
                return got, reps, time.perf_counter() - t0

    (xq, outs), reps, dt = timed(seconds)
    # the same step on one thread, over a quarter of the time
    oracle.set_threads(1)
    try:
        _, reps1, dt1 = timed(seconds / 4)
    finally:
        oracle.set_threads(threads)
    # parity of the GPU step outputs (copy 0) with the oracle
    wl.step(0)
    torch.cuda.synchronize()
    worst = 0.0
    q_ok = all(np.array_equal(wl.xq[xn].cpu().numpy(), xq[xn]) for xn in wl.x)
    for i, (y_ref, den) in enumerate(outs):
        ok, r = oracle.tolerance_ok(wl.y[i].cpu().numpy(), y_ref, den)
        worst = max(worst, r)
    gbps = wl.weight_bytes_step * reps / dt / 1e9
    return {
        "value": round(gbps, 3),
        "unit": "GB/s",
        "cores": threads,
        "value_1_thread": round(wl.weight_bytes_step * reps1 / dt1 / 1e9, 3),
        "cpu_model": _cpu_model().get("Model name", "unknown"),
        "cpu_lscpu": _cpu_model(),
        "kind": "oracle",
        "sample": f"the whole step ({wl.wl['name']}: q8_1 quantisation of every input plus every "
                  f"matmul, f64 dequantise-then-dot) repeated {reps}x in {dt:.1f} s on {threads} "
                  f"threads; value_1_thread: {reps1}x in {dt1:.1f} s on one",
    }, {"q8_1_bitexact": bool(q_ok), "max_err_over_den": worst, "tolerance": 1e-5}


# --------------------------------------------------------------------------
# Summaries of rocprofv3 output (kernel traces and counter collections) for
# the launches of one step, and the HBM traffic they record.
# --------------------------------------------------------------------------

KERNEL_SOURCES = {
    "gemv_q4k": "q6_q8_matmul_amd/csrc/gemv_q4k.hip",
    "gemv_q6k": "q6_q8_matmul_amd/csrc/gemv_q6k.hip",
    "mmq_q4k": "q6_q8_matmul_amd/csrc/mmq_q4k.hip",
    "mmq_q6k": "q6_q8_matmul_amd/csrc/mmq_q6k.hip",
    "quantize": "q6_q8_matmul_amd/csrc/quantize_q8_1.hip",
}
FETCH_SCALE_NOTE = ("FETCH_SIZE and WRITE_SIZE are scaled by bytes / counter reading of the "
                    "plain copy kernels (__amd_rocclr_copyBuffer, the weight copies of known size) "
                    "in the same run")


def source_hash(kernel: str) -> str:
    """Hash of what a counter measurement depends on: the code of the
    kernel's source and of the shared device header (comments and
    whitespace removed, so editing a comment retires nothing) and the
    compiler flags of the build."""
    import hashlib

    from q6_q8_matmul_amd.build import HIPCC_FLAGS

    parts = []
    for rel in (KERNEL_SOURCES[kernel], "q6_q8_matmul_amd/csrc/kq_device.h"):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        parts.append(" ".join(text.split()))
    flags = " ".join(f for f in HIPCC_FLAGS if not f.startswith("/") and f != "-I")
    parts.append(flags)
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()[:16]


def _step_labels(cfg: int):
    from kq_inputs import WORKLOADS

    wl = WORKLOADS[cfg]
    ops = wl.get("bench_ops", wl["ops"])
    labels, kinds, seen = [], [], set()
    for op in ops:
        if op["x"] not in seen:
            labels.append(f"quantize {op['x']}")
            kinds.append("quantize")
            seen.add(op["x"])
        labels.append(op["label"])
        kinds.append(op["op"])
    return labels, kinds


KERNEL_NAMES = {"quantize": "quantize_q8_1_kernel", "gemv_q4k": "gemv_q4k_",   # _kernel or _persistent
                "gemv_q6k": "gemv_q6k_kernel", "mmq_q4k": "mmq_q4k_kernel",
                "mmq_q6k": "mmq_q6k_kernel"}


def _steps_in(rows, cfg):
    """Per step, the dispatches of its launches in order (matched by kernel name)."""
    labels, kinds = _step_labels(cfg)
    by_disp = {}
    for r in rows:
        # the K-split sum that follows a split Q6_K product is reported by
        # --stats, not matched as a launch of the step
        if "kq::" in r["Kernel_Name"] and "splitk_sum" not in r["Kernel_Name"]:
            by_disp.setdefault(r.get("Dispatch_Id") or r.get("Correlation_Id"), []).append(r)
    disp = sorted(by_disp.values(), key=lambda v: int(v[0]["Start_Timestamp"]))
    steps, j, n = [], 0, len(kinds)
    while j + n <= len(disp):
        if all(KERNEL_NAMES[kinds[t]] in disp[j + t][0]["Kernel_Name"] for t in range(n)):
            steps.append(disp[j:j + n])
            j += n
        else:
            j += 1
    return labels, kinds, steps


def _op_weight_bytes(cfg: int):
    """Weight bytes per matmul launch label of workload cfg."""
    from kq_inputs import WORKLOADS

    wl = WORKLOADS[cfg]
    shapes = {name: (kind, a, b) for name, kind, a, b in wl["tensors"]}
    out = {}
    for op in wl.get("bench_ops", wl["ops"]):
        if "w" not in op:
            continue
        names = op["w"] if isinstance(op["w"], list) else [op["w"]]
        out[op["label"]] = sum(shapes[nm][1] * shapes[nm][2] // 256 * (144 if shapes[nm][0] == "q4k" else 210)
                               for nm in names)
    return out


def _op_bytes(cfg: int):
    """Algorithmic bytes per launch label: weights + q8_1 input + f32 output
    (+ f32 residual), and the weight sizes the run copies."""
    from kq_inputs import WORKLOADS

    wl = WORKLOADS[cfg]
    ops = wl.get("bench_ops", wl["ops"])
    wbytes = _op_weight_bytes(cfg)
    out, weights = {}, set()
    for op in ops:
        wb = wbytes[op["label"]]
        weights.add(wb)
        rows = op.get("batch", op.get("n"))
        b = wb + rows * (op["k"] // 32) * 36 + rows * op["m"] * 4
        if "residual" in op:
            b += rows * op["m"] * 4
        out[op["label"]] = b
    return out, sorted(weights)


def _copy_scale(readings, sizes, tol: float = 0.05):
    """Bytes per counter unit from the plain copy kernels of a run: each copy
    moves one weight tensor, of one of the known `sizes`, but how often each
    tensor is copied varies.  The scale is the one under which the most
    readings land within `tol` (relative) of some size -- at least 90 % of
    them, else None -- refined over those matches."""
    if not readings or not sizes:
        return None
    best = []
    for r in readings:
        for size in sizes:
            s = size / r
            matched = []
            for r2 in readings:
                near = min(sizes, key=lambda z: abs(math.log(z / (r2 * s))))
                if abs(math.log(near / (r2 * s))) < tol:
                    matched.append((near, r2))
            if len(matched) > len(best):
                best = matched
    if len(best) < 0.9 * len(readings):
        return None
    return sum(z for z, _ in best) / sum(r for _, r in best)


def summarize(cfg: int, trace_csv=None, fetch_csv=None, write_csv=None):
    """Text summary of rocprofv3 CSV output of this script for workload cfg.
    Counter readings are scaled by (bytes / reading) of the plain copy
    kernels in the same run -- the weight copies, whose sizes are known."""
    import csv

    out = []
    labels, kinds = _step_labels(cfg)
    if trace_csv:
        rows = list(csv.DictReader(open(trace_csv)))
        _, _, steps = _steps_in(rows, cfg)
        out.append(f"kernel trace: {len(steps)} steps matched in {trace_csv}")
        out.append(f"{'launch':22s} {'kernel':16s} {'median_us':>10s} {'min_us':>8s}")
        med = {}
        for t, lab in enumerate(labels):
            d = sorted(int(s[t][0]["End_Timestamp"]) - int(s[t][0]["Start_Timestamp"]) for s in steps)
            if d:
                med[lab] = d[len(d) // 2] / 1e3
                out.append(f"{lab:22s} {kinds[t]:16s} {d[len(d)//2]/1e3:10.2f} {d[0]/1e3:8.2f}")
        # rates of the matmul launches at those medians
        from kq_inputs import WORKLOADS

        ops = {op["label"]: op for op in WORKLOADS[cfg].get("bench_ops", WORKLOADS[cfg]["ops"])}
        wbytes = _op_weight_bytes(cfg)
        for t, lab in enumerate(labels):
            if lab not in med or lab not in wbytes:
                continue
            if kinds[t].startswith("mmq"):
                op = ops[lab]
                tops = 2.0 * op["m"] * op["n"] * op["k"] / (med[lab] * 1e-6) / 1e12
                out.append(f"  {lab}: 2*M*N*K = {2 * op['m'] * op['n'] * op['k']:.4e} ops at the median: "
                           f"{tops:.0f} TOPS = {100 * tops / INT8_PEAK_TOPS:.1f} % of "
                           f"{INT8_PEAK_TOPS / 1e3:.1f} POPS")
            else:
                out.append(f"  {lab}: weight bytes {wbytes[lab]:,} at the median: "
                           f"{wbytes[lab] / (med[lab] * 1e-6) / 1e9:,.0f} GB/s")
        stats = os.path.join(os.path.dirname(trace_csv), "run_kernel_stats.csv")
        if os.path.exists(stats):
            out.append("rocprofv3 --stats (run_kernel_stats.csv), kq kernels (every call of the run):")
            for r in csv.DictReader(open(stats)):
                if "kq::" in r["Name"]:
                    m = re.search(r"(\w+_(?:kernel|persistent|ksplit)(<[^>]*>)?)", r["Name"])
                    nm = m.group(1) if m else r["Name"][:40]
                    out.append(f"  {nm:48s} calls {int(r['Calls']):5d}  avg {float(r['AverageNs'])/1e3:9.2f} us"
                               f"  min {float(r['MinNs'])/1e3:8.2f}  max {float(r['MaxNs'])/1e3:8.2f}")
    op_bytes, weight_sizes = _op_bytes(cfg)
    per, scale = {}, {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        if not path:
            continue
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == name]
        copies = [float(r["Counter_Value"]) * 1024 for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) * 1024 >= min(weight_sizes) / 4]
        sc = _copy_scale(copies, weight_sizes)
        if sc is not None:
            scale[name] = sc
        _, _, steps = _steps_in(rows, cfg)
        out.append(f"{name}: {len(steps)} steps matched in {path}; copy-kernel scale "
                   f"{scale.get(name, float('nan')):.4f} from {len(copies)} weight copies")
        per[name] = {}
        for t, lab in enumerate(labels):
            v = sorted(float(s[t][0]["Counter_Value"]) for s in steps)
            if v:
                per[name][lab] = v[len(v) // 2] * 1024
                out.append(f"  {lab:22s} median {v[len(v)//2]:12.2f} KiB")
    traffic = None
    if "FETCH_SIZE" in scale and "WRITE_SIZE" in scale:
        hbm = {lab: per["FETCH_SIZE"][lab] * scale["FETCH_SIZE"] + per["WRITE_SIZE"][lab] * scale["WRITE_SIZE"]
               for lab in op_bytes if lab in per["FETCH_SIZE"]}
        raw = {lab: per["FETCH_SIZE"][lab] + per["WRITE_SIZE"][lab] for lab in hbm}
        out.append("HBM bytes per launch: raw FETCH + WRITE (KiB x 1024), scaled, algorithmic:")
        out.append(f"  {'launch':22s} {'raw':>16s} {'scaled':>16s} {'algorithmic':>16s}  scaled/alg")
        for lab, v in hbm.items():
            out.append(f"  {lab:22s} {raw[lab]:16,.0f} {v:16,.0f} {op_bytes[lab]:16,}  {v / op_bytes[lab]:.4f}")
        kern = kinds[labels.index(next(iter(hbm)))]
        traffic = {"kernel": "kq_" + kern, "workload": _workload_name(cfg),
                   "source_sha256_16": source_hash(kern),
                   "fetch_scale": round(scale["FETCH_SIZE"], 5), "write_scale": round(scale["WRITE_SIZE"], 5),
                   "fetch_bytes_raw": {k: round(per["FETCH_SIZE"][k]) for k in hbm},
                   "write_bytes_raw": {k: round(per["WRITE_SIZE"][k]) for k in hbm},
                   "hbm_bytes": {k: round(v) for k, v in hbm.items()},
                   "algorithmic_bytes": op_bytes,
                   "hbm_bytes_per_launch": round(sum(hbm.values()) / len(hbm)),
                   "algorithmic_bytes_per_launch": round(sum(op_bytes.values()) / len(op_bytes))}
    return "\n".join(out), traffic


# MI355X layout used to normalise the SQ counters of one kernel: the busy
# cycles are summed over every SIMD (4 per CU) and GRBM_GUI_ACTIVE over the
# XCDs, so a kernel's cycles are GRBM_GUI_ACTIVE / XCDS.
MI355X_CUS, MI355X_XCDS, SIMDS_PER_CU = 256, 8, 4
MMQ_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
                "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE")
LDS_COUNTERS = ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS")


def summarize_counters(cfg: int, counters_csv: str):
    """Per launch of workload cfg, the median of each counter over the
    run's steps, and for the MMQ launches the matrix-core busy fraction, the
    VALU instruction count charged at 4 cycles each (VALU x4) and the int8
    MFMA work the counters saw against 2*M*N*K; with the LDS counters, the
    fraction of CU-cycles the LDS is busy and stalled on bank conflicts."""
    import csv
    from kq_inputs import WORKLOADS

    rows = list(csv.DictReader(open(counters_csv)))
    labels, kinds, steps = _steps_in(rows, cfg)
    ops = {op["label"]: op for op in WORKLOADS[cfg].get("bench_ops", WORKLOADS[cfg]["ops"])}
    record = {}
    out = [f"counters: {len(steps)} steps matched in {counters_csv}",
           f"normalisation: kernel cycles = GRBM_GUI_ACTIVE / {MI355X_XCDS} XCDs; "
           f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS_PER_CU} SIMDs x {MI355X_CUS} CUs x kernel cycles); "
           f"VALU x4 = 4 x SQ_ACTIVE_INST_VALU / the same, i.e. every VALU instruction charged "
           f"4 cycles; a plain v_fmac_f32 stream at 2-8 wavefronts per SIMD issues one "
           f"instruction per ~2.2-2.8 cycles and reads 1.44-1.78 on this measure, so a "
           f"saturated VALU reads about 1.6, not 1.0"]
    present = {r["Counter_Name"] for r in rows}
    names = [n for n in MMQ_COUNTERS + LDS_COUNTERS if n in present]
    if present & set(LDS_COUNTERS):
        out.append(f"LDS busy = SQ_LDS_IDX_ACTIVE / ({MI355X_CUS} CUs x kernel cycles); LDS bank-conflict "
                   f"= SQ_LDS_BANK_CONFLICT / the same")
    for t, lab in enumerate(labels):
        if kinds[t] == "quantize":
            continue
        med = {}
        for name in names:
            v = sorted(sum(float(r["Counter_Value"]) for r in s[t] if r["Counter_Name"] == name)
                       for s in steps)
            if v:
                med[name] = v[len(v) // 2]
        op = ops[lab]
        rows = op.get("n", op.get("batch"))
        work = 2.0 * op["m"] * rows * op["k"]
        out.append(f"{lab} ({kinds[t]}, {op['m']}x{op['k']} x {rows} columns, 2MNK = {work:.4e}):")
        for name in names:
            if name in med:
                out.append(f"  {name:28s} median {med[name]:16,.0f}")
        cyc = med.get("GRBM_GUI_ACTIVE", 0) / MI355X_XCDS
        if cyc > 0:
            simd_cycles = SIMDS_PER_CU * MI355X_CUS * cyc
            rec = record.setdefault(kinds[t], {"kernel": "kq_" + kinds[t], "workload": _workload_name(cfg),
                                               "source_sha256_16": source_hash(kinds[t]), "launches": {}})
            lrec = rec["launches"].setdefault(lab, {})
            if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
                busy = med['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles
                lrec["mfma_busy"] = round(busy, 4)
                out.append(f"  MFMA busy {100 * busy:6.1f} %")
            if "SQ_ACTIVE_INST_VALU" in med:
                vx4 = 4 * med['SQ_ACTIVE_INST_VALU'] / simd_cycles
                lrec["valu_x4"] = round(vx4, 4)
                out.append(f"  VALU x4   {100 * vx4:6.1f} %")
            if "SQ_LDS_IDX_ACTIVE" in med:
                lds = med["SQ_LDS_IDX_ACTIVE"] / (MI355X_CUS * cyc)
                conf = med.get("SQ_LDS_BANK_CONFLICT", 0.0) / (MI355X_CUS * cyc)
                lrec["lds_busy"], lrec["lds_bank_conflict"] = round(lds, 4), round(conf, 4)
                out.append(f"  LDS busy  {100 * lds:6.1f} %   bank-conflict {100 * conf:5.1f} %")
        if kinds[t].startswith("gemv") and med.get("SQ_INSTS_VALU"):
            # one Q4_K wavefront pass covers 16 superblock-rows, a Q6_K one 16
            sbrows = op["m"] * (op["k"] // 256)
            per = med["SQ_INSTS_VALU"] / (sbrows / 16)
            out.append(f"  VALU instructions per wavefront pass (16 superblock-rows) {per:8.1f}")
            rec = record.setdefault(kinds[t], {"kernel": "kq_" + kinds[t], "workload": _workload_name(cfg),
                                               "source_sha256_16": source_hash(kinds[t]), "launches": {}})
            rec["launches"].setdefault(lab, {})["valu_per_pass"] = round(per, 1)
        if med.get("SQ_INSTS_VALU_MFMA_MOPS_I8"):   # one count = 512 int8 ops
            mops = 512 * med["SQ_INSTS_VALU_MFMA_MOPS_I8"]
            out.append(f"  int8 MFMA ops 512 x SQ_INSTS_VALU_MFMA_MOPS_I8 = {mops:.4e} = {mops / work:.3f} x 2MNK")
        # engine clock: GRBM_GUI_ACTIVE per XCD over the dispatch's own
        # timestamps (the counter also counts a few microseconds of activity
        # around a dispatch, so short launches read high)
        clk, durs = [], []
        for st in steps:
            for r in st[t]:
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and r.get("End_Timestamp"):
                    ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                    if ns > 0:
                        clk.append(float(r["Counter_Value"]) / MI355X_XCDS / ns)
                        durs.append(ns / 1e3)
                    break
        if clk:
            clk.sort()
            durs.sort()
            out.append(f"  clock {clk[len(clk) // 2]:9.3f} GHz  (GRBM_GUI_ACTIVE / {MI355X_XCDS} over the median "
                       f"dispatch time {durs[len(durs) // 2]:.1f} us of this counter run)")
            if kinds[t] in record:
                record[kinds[t]]["launches"].setdefault(lab, {})["clock_GHz"] = round(clk[len(clk) // 2], 3)
    for rec in record.values():
        out.append("counters_json: " + json.dumps(rec))
    return "\n".join(out)


def _workload_name(cfg: int) -> str:
    from kq_inputs import WORKLOADS

    return WORKLOADS[cfg]["name"]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if
    the kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic_json: "):
            d = json.loads(line[len("traffic_json: "):])
            if d.get("source_sha256_16") == source_hash(kernel):
                return d
    return None


def mmq_roofline(entry):
    """Roofline object of the prefill half of the metric: the Q4_K MMQ
    launches of the prefill workload, 2*M*N*K int8 ops per launch over the
    launch's mean duration, against the dense int8 MFMA peak; matrix-core
    busy fraction and VALU x4 figure from the committed counter summary when it was
    taken on the current source."""
    if not entry:
        return None
    ks = [e for e in entry["kernels"] if e["kernel"] == "kq_mmq_q4k"]
    if not ks:
        return None
    ops = [2.0 * e["shape"][0] * e["shape"][1] * e["shape"][2] for e in ks]
    secs = [e["avg_us"] * 1e-6 for e in ks]
    achieved = sum(ops) / sum(secs) / 1e12
    out = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
           "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": None, "kernel": "kq_mmq_q4k",
           "workload": entry["workload"], "ops_per_launch": round(sum(ops) / len(ops)),
           "avg_launch_us": round(sum(secs) * 1e6 / len(secs), 2),
           "per_launch": {e["op"]: {"tops": e["tops"], "frac": e["frac_int8_peak"],
                                    "median_us": e.get("median_us"), "min_us": e.get("min_us")} for e in ks}}
    rec = read_counters("mmq_q4k", entry["workload"])
    if rec:
        for lab, v in rec["launches"].items():
            if lab in out["per_launch"]:
                out["per_launch"][lab].update({k: v[k] for k in ("mfma_busy", "valu_x4", "clock_GHz") if k in v})
        out["counters"] = f"profiles/mmq_q4k_{entry['workload']}_counters.txt"
    return out


def read_counters(kernel: str, workload: str):
    """Matrix-core busy and VALU x4 figures per launch of `kernel` from the committed
    counter summary, if the kernel source is unchanged since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("counters_json: "):
            d = json.loads(line[len("counters_json: "):])
            if d.get("kernel") == "kq_" + kernel and d.get("source_sha256_16") == source_hash(kernel):
                return d
    return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of HIP graphs")
    ap.add_argument("--no-secondary", action="store_true", help="skip workloads 2-4")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the read-ceiling sweep (profiling runs of one workload)")
    ap.add_argument("--only", type=int, default=None, help="measure only this workload")
    ap.add_argument("--summarize", action="store_true",
                    help="summarise rocprofv3 CSV output of a run of this script (no GPU)")
    ap.add_argument("--trace-csv", default=None)
    ap.add_argument("--fetch-csv", default=None)
    ap.add_argument("--write-csv", default=None)
    ap.add_argument("--counters-csv", default=None,
                    help="one --pmc pass with the MMQ counters (matrix-core busy, VALU instructions)")
    args = ap.parse_args(argv)

    if args.summarize:
        cfg = 1 if args.only is None else args.only
        if args.counters_csv:
            print(summarize_counters(cfg, args.counters_csv))
            return 0
        text, traffic = summarize(cfg, args.trace_csv, args.fetch_csv, args.write_csv)
        print(text)
        if traffic:
            print("traffic_json: " + json.dumps(traffic))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the k-quant "
              "matmul library runs on one MI355X).", file=sys.stderr)
        return 2

    import torch

    import q6_q8_matmul_amd as kq

    kq.lib()
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    use_graph = not args.no_graph

    secondary = {}
    failed = False
    main_cfg = 1
    cfgs = [args.only] if args.only is not None else ([1] if args.no_secondary else [1, 2, 3, 4, 5, 6, 7, 8, 9])
    result = None
    # The read-ceiling sweep runs first: about a second of streaming that
    # also takes the engine clock off its idle level before any workload is
    # timed (measured: the first workload of a fresh process otherwise runs
    # at a median 1.6 GHz against 2.3 GHz for the later ones).
    ceiling = stream_read_ceiling() if 1 in cfgs and not args.no_ceiling else None
    for cfg in cfgs:
        if cfg in (5, 6):
            log(f"workload {cfg}: fused producers")
            secondary[f"cfg{cfg}"] = measure_producers(cfg)
            torch.cuda.empty_cache()
            continue
        if cfg == 8:
            log(f"workload {cfg}: separate vs segmented GEMV launches")
            secondary[f"cfg{cfg}"] = measure_segmented(cfg)
            torch.cuda.empty_cache()
            continue
        prefill = cfg in (4, 9)
        steps = args.steps if not prefill else max(20, args.steps // 10)
        warm = args.warmup if not prefill else max(5, args.warmup // 4)
        log(f"workload {cfg}: {steps} steps, {warm} warm-up, graphs={use_graph}")
        wl, ms, durs, clocks = measure(cfg, steps, warm, use_graph)
        per_op = []
        for i, op in enumerate(wl.ops):
            label, kind, avg_ms, med_ms, min_ms, str_ms = [d for d in durs if d[0] == op["label"]][0]
            e = {"op": op["label"], "kernel": "kq_" + op["op"], "shape": [op["m"], op["k"], op.get("batch", op.get("n"))],
                 "avg_us": round(avg_ms * 1e3, 2), "median_us": round(med_ms * 1e3, 2),
                 "min_us": round(min_ms * 1e3, 2), "stream_median_us": round(str_ms * 1e3, 2)}
            if op["op"].startswith("mmq"):
                tops = wl.op_ops(i) / (avg_ms * 1e-3) / 1e12
                e["tops"] = round(tops, 2)
                e["frac_int8_peak"] = round(tops / INT8_PEAK_TOPS, 4)
                e["frac_int8_peak_stream"] = round(wl.op_ops(i) / (str_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)
            else:
                gbps = wl.host[op["w"]].nbytes / (avg_ms * 1e-3) / 1e9
                e["weight_GBps"] = round(gbps, 1)
                e["frac_hbm"] = round(gbps / HBM_PEAK_GBPS, 4)
                e["frac_hbm_stream"] = round(wl.host[op["w"]].nbytes / (str_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
            per_op.append(e)
        if any(op["op"].startswith("gemv") for op in wl.ops):
            floors = read_floors_us(wl)
            for e in per_op:
                if e["op"] in floors:
                    e["read_floor_us"], e["read_floor_form"] = floors[e["op"]]
                    e["frac_of_read_floor"] = round(e["read_floor_us"] / e["avg_us"], 4)
        quant = [{"op": d[0], "avg_us": round(d[2] * 1e3, 2), "median_us": round(d[3] * 1e3, 2),
                  "min_us": round(d[4] * 1e3, 2)} for d in durs if d[1] == "quantize"]
        step_rate = wl.weight_bytes_step / (ms * 1e-3) / 1e9
        entry = {"workload": wl.wl["name"], "ms_per_step": round(ms, 5),
                 "weight_bytes_per_step": wl.weight_bytes_step, "weight_copies": wl.ncopies,
                 "steps_per_graph": cycle_len(wl.ncopies) if use_graph else None,
                 "step_weight_GBps": round(step_rate, 1), "kernels": per_op, "quantize": quant,
                 "timing": "kernel figures: mean, median and min over 5 interleaved rounds of graph "
                           "replays (frac_* from the mean); stream_median_us / *_stream: the same launches "
                           "issued straight to the stream in the same rounds (median)",
                 "clock_power": clocks}
        if prefill:
            tot_ops = sum(wl.op_ops(i) for i in range(len(wl.ops)))
            entry["step_int8_TOPS"] = round(tot_ops / (ms * 1e-3) / 1e12, 2)
        if cfg == main_cfg:
            # roofline of the dominant kernel: kq_gemv_q4k over the step's 4 launches
            tot_b = sum(wl.op_bytes(i) for i in range(len(wl.ops)))
            tot_t = sum([d for d in durs if d[0] == op["label"]][0][2] for op in wl.ops) * 1e-3
            achieved = tot_b / tot_t / 1e9
            tr = read_traffic("gemv_q4k", wl.wl["name"])
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                        "traffic": tr["hbm_bytes_per_launch"] if tr else None,
                        "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled)",
                        "kernel": "kq_gemv_q4k",
                        "algorithmic_bytes_per_launch": round(tot_b / len(wl.ops)),
                        "avg_launch_us": round(tot_t * 1e6 / len(wl.ops), 2)}
            result = {
                "metric": METRIC,
                "value": round(step_rate, 1),
                "unit": "GB/s",
                "n_gpus": 1,
                "steps": steps,
                "warmup": warm,
                "ms_per_step": round(ms, 5),
                "higher_is_better": True,
                "scaling": "weak",
                "vs_baseline": None,
                "dtype": "int8",
                "data": "synthetic",
                "config": {"workload": wl.wl["name"],
                           "shapes": "attn_out 4096x4096; gate and up 14336x4096 each, one launch over "
                                     "their contiguous 28672 rows; down 4096x14336",
                           "batch": 1, "weight_format": "Q4_K", "activation_format": "q8_1",
                           "hip_graphs": use_graph,
                           "steps_per_graph": cycle_len(wl.ncopies) if use_graph else None},
                "roofline": roofline,
            }
            if ceiling:
                ceiling["gemv_frac_of_ceiling"] = round(achieved / ceiling["GBps"], 4)
                result["stream_read_ceiling"] = ceiling
            if not args.no_cpu:
                log(f"cpu baseline (~{args.cpu_seconds} s)")
                cb, parity = cpu_baseline(wl, args.cpu_seconds)
                parity["ok"] = bool(parity["q8_1_bitexact"]
                                    and parity["max_err_over_den"] <= parity["tolerance"])
                if not parity["ok"]:   # the timing of a wrong result is no measurement
                    log(f"PARITY FAILED against the oracle: {parity}")
                    failed = True
                result["cpu_baseline"] = cb
                result["parity_vs_oracle"] = parity
            result["kernels"] = per_op
            result["quantize"] = quant
            result["weight_copies"] = wl.ncopies
            result["timing"] = entry["timing"]
            result["clock_power"] = clocks
        else:
            secondary[f"cfg{cfg}"] = entry
        del wl
        torch.cuda.empty_cache()
        if cfg in (3, 9):
            log(f"workload {cfg}: raw vs split Q6_K layout")
            secondary[f"cfg{cfg}_split_layout"] = measure_split(cfg)
            torch.cuda.empty_cache()
        if cfg in (4, 9):
            log(f"workload {cfg}: products with and without the K split")
            secondary[f"cfg{cfg}_k_split"] = measure_ksplit(cfg)
            torch.cuda.empty_cache()
    mmq = mmq_roofline(secondary.get("cfg4"))
    if result is None:
        result = {"metric": METRIC}
    if mmq:
        result["roofline_mmq"] = mmq
    if secondary:
        result["secondary"] = secondary
    print(json.dumps(result), flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main())
