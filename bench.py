#!/usr/bin/env python3
"""Benchmark of the k-quant matmul hot path on one MI355X.

Metric: Q4_K x q8_1 GEMV weight GB/s (fraction of HBM peak); prefill MMQ int8
TOPS (fraction of int8 MFMA peak).

A step is one Llama-3-8B-shaped decode pass at batch 1 (workload
"llama3_8b_decode_gemv_q4k_b1"): quantise the attention-output input and run
attn-out 4096x4096; quantise the FFN input and run gate and up 14336x4096
(one shared q8_1 activation); quantise the down input and run down
4096x14336.  ``value`` is the weight bytes of that pass (108,527,616) per
second of step time.  The weights rotate over enough device copies that the
footprint exceeds twice the 256 MB Infinity Cache, so every step streams its
weights from HBM.  Inputs are resident in HBM before the timed region.

The other workloads are measured the same way and reported under
``secondary``: batch-4 decode (fused QKV 6144x4096 and down 4096x14336 with
residual), the Q6_K output head 128256x4096 (batch 1 and 4), and the
Qwen2-7B prefill MMQ at 2048 tokens (gate/up 18944x3584, down 3584x18944,
QKV 4608x3584).

``roofline`` describes the dominant kernel of the step, kq_gemv_q4k: its
algorithmic bytes per launch (weights + q8_1 activation + f32 output) over
its average launch duration, measured with HIP events recorded on the launch
stream around every GEMV launch of an instrumented copy of the timed steps.

``cpu_baseline`` times the CPU oracle on the host cores on the same step and
also reports how far the GPU step outputs are from it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA (5.0 POPS)
MALL_BYTES = 256 * 2 ** 20      # Infinity Cache
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
        self.ops = self.wl["ops"]
        host = {}
        for name, kind, a, b in self.wl["tensors"]:
            host[name] = tensor(cfg, name)
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
        for op in self.ops:
            rows = op.get("batch", op.get("n"))
            self.y.append(torch.empty((rows, op["m"]), dtype=torch.float32, device="cuda"))
            if "residual" in op:
                self.res[op["residual"]] = torch.from_numpy(host[op["residual"]]).cuda()
        torch.cuda.synchronize()

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
            w = self.w[c][op["w"]]
            xq = self.xq[xn]
            y = self.y[i]
            if op["op"] == "gemv_q4k" or op["op"] == "gemv_q6k":
                res = self.res.get(op.get("residual"))
                fn = kq.kq_gemv_q4k if op["op"] == "gemv_q4k" else kq.kq_gemv_q6k
                out.append((op["label"], op["op"],
                            lambda fn=fn, w=w, xq=xq, y=y, res=res, op=op:
                            fn(w, xq, y, res, op["m"], op["k"], op["batch"])))
            else:
                out.append((op["label"], op["op"],
                            lambda w=w, xq=xq, y=y, op=op:
                            kq.kq_mmq_q4k(w, xq, y, op["m"], op["n"], op["k"])))
        return out

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


def build_graphs(wl: Workload):
    import torch

    graphs = []
    side = torch.cuda.Stream()
    for c in range(wl.ncopies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            wl.step(c)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def timed_steps(wl: Workload, steps: int, warmup: int, graphs=None):
    """Wall time per step (ms) over `steps` steps bracketed by events and
    synchronisation; weights rotate over the copies."""
    import torch

    run = (lambda c: graphs[c].replay()) if graphs else wl.step
    for i in range(warmup):
        run(i % wl.ncopies)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        run(i % wl.ncopies)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def kernel_durations(wl: Workload, steps: int):
    """Average duration (ms) of every launch of the step, from HIP events
    recorded on the launch stream around each launch; eager launches."""
    import torch

    stream = torch.cuda.current_stream()
    labels = None
    rec = []
    for i in range(steps):
        row = []
        for label, kind, fn in wl.launches(i % wl.ncopies):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            row.append((label, kind, a, b))
        rec.append(row)
    torch.cuda.synchronize()
    labels = [(l, k) for l, k, _, _ in rec[0]]
    avg = []
    for j, (label, kind) in enumerate(labels):
        d = [r[j][2].elapsed_time(r[j][3]) for r in rec]
        d.sort()
        avg.append((label, kind, sum(d) / len(d), d[len(d) // 2]))
    return avg


def measure(cfg: int, steps: int, warmup: int, use_graph: bool):
    import torch

    wl = Workload(cfg)
    wl.step(0)                      # first calls outside any capture
    torch.cuda.synchronize()
    graphs = build_graphs(wl) if use_graph else None
    ms = timed_steps(wl, steps, warmup, graphs)
    durs = kernel_durations(wl, max(5, min(steps, 50)))
    del graphs
    return wl, ms, durs


def cpu_baseline(wl: Workload, seconds: float):
    """The oracle on the host: the same step (quantise + every matmul of the
    workload) repeated until `seconds` have passed; also the GPU step
    outputs compared with the oracle's."""
    import numpy as np
    import torch

    import oracle

    oracle.build(force=False)
    threads = oracle.max_threads()
    reps = 0
    t0 = time.perf_counter()
    outs = None
    while True:
        xq = {xn: oracle.quantize_q8_1(wl.host[xn]) for xn in wl.x}
        outs = []
        for op in wl.ops:
            kind = "q4k" if op["op"] in ("gemv_q4k", "mmq_q4k") else "q6k"
            rows = op.get("batch", op.get("n"))
            res = wl.host.get(op.get("residual")) if "residual" in op else None
            outs.append(oracle.matmul(kind, wl.host[op["w"]], xq[op["x"]], op["m"], rows, op["k"],
                                      residual=res))
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
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
        "kind": "oracle",
        "sample": f"the whole step ({wl.wl['name']}: q8_1 quantisation of every input plus every "
                  f"matmul, f64 dequantise-then-dot) repeated {reps}x in {dt:.1f} s",
    }, {"q8_1_bitexact": bool(q_ok), "max_err_over_den": worst, "tolerance": 1e-5}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of HIP graphs")
    ap.add_argument("--no-secondary", action="store_true", help="skip workloads 2-4")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", type=int, default=None, help="measure only this workload")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the k-quant "
              "matmul runs on one MI355X; sharding is described in DESIGN.md).", file=sys.stderr)
        return 2

    import torch

    import q6_q8_matmul_amd as kq

    kq.lib()
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    use_graph = not args.no_graph

    secondary = {}
    main_cfg = 1
    cfgs = [args.only] if args.only is not None else ([1] if args.no_secondary else [1, 2, 3, 4])
    result = None
    for cfg in cfgs:
        steps = args.steps if cfg != 4 else max(3, args.steps // 20)
        warm = args.warmup if cfg != 4 else max(1, args.warmup // 10)
        log(f"workload {cfg}: {steps} steps, {warm} warm-up, graphs={use_graph}")
        wl, ms, durs = measure(cfg, steps, warm, use_graph)
        per_op = []
        for i, op in enumerate(wl.ops):
            label, kind, avg_ms, med_ms = [d for d in durs if d[0] == op["label"]][0]
            e = {"op": op["label"], "kernel": "kq_" + op["op"], "shape": [op["m"], op["k"], op.get("batch", op.get("n"))],
                 "avg_us": round(avg_ms * 1e3, 2), "median_us": round(med_ms * 1e3, 2)}
            if op["op"] == "mmq_q4k":
                tops = wl.op_ops(i) / (avg_ms * 1e-3) / 1e12
                e["tops"] = round(tops, 2)
                e["frac_int8_peak"] = round(tops / INT8_PEAK_TOPS, 4)
            else:
                gbps = wl.host[op["w"]].nbytes / (avg_ms * 1e-3) / 1e9
                e["weight_GBps"] = round(gbps, 1)
                e["frac_hbm"] = round(gbps / HBM_PEAK_GBPS, 4)
            per_op.append(e)
        quant = [{"op": d[0], "avg_us": round(d[2] * 1e3, 2)} for d in durs if d[1] == "quantize"]
        step_rate = wl.weight_bytes_step / (ms * 1e-3) / 1e9
        entry = {"workload": wl.wl["name"], "ms_per_step": round(ms, 5),
                 "weight_bytes_per_step": wl.weight_bytes_step, "weight_copies": wl.ncopies,
                 "step_weight_GBps": round(step_rate, 1), "kernels": per_op, "quantize": quant}
        if cfg == 4:
            tot_ops = sum(wl.op_ops(i) for i in range(len(wl.ops)))
            entry["step_int8_TOPS"] = round(tot_ops / (ms * 1e-3) / 1e12, 2)
        if cfg == main_cfg:
            # roofline of the dominant kernel: kq_gemv_q4k over the step's 4 launches
            tot_b = sum(wl.op_bytes(i) for i in range(len(wl.ops)))
            tot_t = sum([d for d in durs if d[0] == op["label"]][0][2] for op in wl.ops) * 1e-3
            achieved = tot_b / tot_t / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                        "kernel": "kq_gemv_q4k",
                        "algorithmic_bytes_per_step": tot_b,
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
                           "shapes": "attn_out 4096x4096, gate 14336x4096, up 14336x4096, down 4096x14336",
                           "batch": 1, "weight_format": "Q4_K", "activation_format": "q8_1",
                           "hip_graphs": use_graph},
                "roofline": roofline,
            }
            if not args.no_cpu:
                log(f"cpu baseline (~{args.cpu_seconds} s)")
                cb, parity = cpu_baseline(wl, args.cpu_seconds)
                result["cpu_baseline"] = cb
                result["parity_vs_oracle"] = parity
            result["kernels"] = per_op
            result["quantize"] = quant
            result["weight_copies"] = wl.ncopies
        else:
            secondary[f"cfg{cfg}"] = entry
        del wl
        torch.cuda.empty_cache()
    if result is None:
        result = {"metric": METRIC, "secondary": secondary}
    elif secondary:
        result["secondary"] = secondary
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
