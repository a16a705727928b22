"""Host logic of bench.py (no GPU).

* The source hash that keys the committed HBM-traffic records ignores
  comments and whitespace but not code.
* The counter summary turns a counter collection into matrix-core and VALU
  busy fractions, int8 MFMA work against 2*M*N*K and the engine clock; the
  traffic summary scales FETCH_SIZE / WRITE_SIZE by the run's own weight
  copies; the trace summary gives per-launch medians.  Each is checked on a
  small synthetic collection whose answers are known by construction.
"""
import csv
import json

import bench


def test_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    import q6_q8_matmul_amd.build as build

    (tmp_path / "a.hip").write_text("int f(int x) { return x + 1; } // one\n/* a\n block */\n")
    (tmp_path / "b.hip").write_text("// header\nint f(int x)  {\n  return x + 1;   // uno\n}\n")
    (tmp_path / "c.hip").write_text("int f(int x) { return x + 2; } // one\n")
    hdr = tmp_path / "q6_q8_matmul_amd" / "csrc" / "kq_device.h"
    hdr.parent.mkdir(parents=True)
    hdr.write_text("inline int g() { return 3; }  // shared\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"a": "a.hip", "b": "b.hip", "c": "c.hip"})
    ha = bench.source_hash("a")
    assert ha == bench.source_hash("b")
    assert ha != bench.source_hash("c")
    # the shared device header and the compiler flags are part of the key
    hdr.write_text("/* shared */ inline int g() {\n return 3; }\n")
    assert bench.source_hash("a") == ha
    hdr.write_text("inline int g() { return 4; }\n")
    assert bench.source_hash("a") != ha
    hdr.write_text("inline int g() { return 3; }\n")
    monkeypatch.setattr(build, "HIPCC_FLAGS", build.HIPCC_FLAGS + ["-O2"])
    assert bench.source_hash("a") != ha


def _collection(path, steps, ghz, mfma_busy, valu_x4, mops_factor, lds=None):
    """Counter rows for `steps` steps of workload 9 (quantise, v, quantise,
    down): each MMQ dispatch lasts 100 us at `ghz` on every XCD."""
    dur_ns = 100_000
    cyc = ghz * dur_ns                       # per XCD
    simd_cycles = 4 * 256 * cyc
    shapes = {"v": (512, 2048, 3584), "down": (3584, 2048, 18944)}
    fields = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
              "Start_Timestamp", "End_Timestamp"]
    rows, disp, t0 = [], 0, 1_000_000
    for _ in range(steps):
        for label in ("quantize x_in", "v", "quantize x_down", "down"):
            disp += 1
            if label.startswith("quantize"):
                name = "kq::(anonymous namespace)::quantize_q8_1_kernel(float const*, int)"
                vals = {"GRBM_GUI_ACTIVE": 8 * 2.0 * 5_000}
                dur = 5_000
            else:
                name = "void kq::(anonymous namespace)::mmq_q6k_kernel<4, false>(unsigned char const*)"
                m, n, k = shapes[label]
                vals = {"SQ_INSTS_VALU_MFMA_MOPS_I8": mops_factor * 2 * m * n * k / 512,
                        "SQ_VALU_MFMA_BUSY_CYCLES": mfma_busy * simd_cycles,
                        "SQ_ACTIVE_INST_VALU": valu_x4 * simd_cycles / 4,
                        "SQ_INSTS_MFMA": 1.0, "SQ_INSTS_VALU": 1.0,
                        "GRBM_GUI_ACTIVE": 8 * cyc}
                if lds is not None:           # (busy, bank-conflict) fractions of CU-cycles
                    vals["SQ_LDS_IDX_ACTIVE"] = lds[0] * 256 * cyc
                    vals["SQ_LDS_BANK_CONFLICT"] = lds[1] * 256 * cyc
                dur = dur_ns
            for cname, v in vals.items():
                rows.append({"Correlation_Id": disp, "Dispatch_Id": disp, "Kernel_Name": name,
                             "Counter_Name": cname, "Counter_Value": f"{v:.6f}",
                             "Start_Timestamp": t0, "End_Timestamp": t0 + dur})
            t0 += dur + 1_000
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_counter_summary_fractions_work_and_clock(tmp_path):
    path = tmp_path / "run_counter_collection.csv"
    _collection(path, steps=3, ghz=2.0, mfma_busy=0.25, valu_x4=0.5, mops_factor=2)
    out = bench.summarize_counters(9, str(path))
    assert "3 steps matched" in out
    lines = out.split("\n")
    for label in ("v (mmq_q6k", "down (mmq_q6k"):
        i = next(j for j, l in enumerate(lines) if l.startswith(label))
        block = []
        for l in lines[i + 1:]:
            if not l.startswith("  "):
                break
            block.append(l)
        block = "\n".join(block)
        assert "MFMA busy   25.0 %" in block, block
        assert "VALU x4     50.0 %" in block, block
        assert "= 2.000 x 2MNK" in block, block
        assert "clock     2.000 GHz" in block, block
        assert "dispatch time 100.0 us" in block, block
    rec = [json.loads(l.split(": ", 1)[1]) for l in lines if l.startswith("counters_json: ")]
    assert len(rec) == 1 and rec[0]["kernel"] == "kq_mmq_q6k"
    assert rec[0]["launches"]["down"] == {"mfma_busy": 0.25, "valu_x4": 0.5, "clock_GHz": 2.0}


def _decode_run(path, counter, steps, per_label, copy_factor):
    """A counter collection of workload 1 (quantise + GEMV, three times per
    step) preceded by five copies of each weight tensor whose readings are
    `copy_factor` x their bytes; `per_label` gives each launch's bytes."""
    weights = [9437184, 66060288, 33030144]      # attn_out, gate|up, down
    fields = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
              "Start_Timestamp", "End_Timestamp"]
    rows, disp, t0 = [], 0, 1_000_000

    def add(name, nbytes, dur):
        nonlocal disp, t0
        disp += 1
        rows.append({"Correlation_Id": disp, "Dispatch_Id": disp, "Kernel_Name": name,
                     "Counter_Name": counter, "Counter_Value": f"{nbytes / 1024:.6f}",
                     "Start_Timestamp": t0, "End_Timestamp": t0 + dur})
        t0 += dur + 500

    for wb in weights:
        for _ in range(5):
            add("__amd_rocclr_copyBuffer", wb * copy_factor, 20_000)
    q = "kq::(anonymous namespace)::quantize_q8_1_kernel(float const*, int)"
    g = "void kq::gemv4::gemv_q4k_persistent<1, 1, 1, 8, kq::gemv4::Seg1>(kq::gemv4::Seg1)"
    for _ in range(steps):
        for lab in ("quantize x_attn", "attn_out", "quantize x_ffn", "gate|up", "quantize x_down", "down"):
            add(q if lab.startswith("quantize") else g, per_label[lab], 2_000 if lab.startswith("quantize") else 10_000)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_traffic_summary_scales_by_the_copies(tmp_path):
    alg, _ = bench._op_bytes(1)
    fetch = {lab: 4096.0 for lab in ("quantize x_attn", "quantize x_ffn", "quantize x_down")}
    write = dict(fetch)
    for lab in ("attn_out", "gate|up", "down"):
        fetch[lab] = alg[lab] * 1.01 / 2     # FETCH_SIZE reads half of the bytes moved
        write[lab] = 0.0
    _decode_run(tmp_path / "f.csv", "FETCH_SIZE", 4, fetch, 0.5)
    _decode_run(tmp_path / "w.csv", "WRITE_SIZE", 4, write, 1.0)
    text, traffic = bench.summarize(1, fetch_csv=str(tmp_path / "f.csv"), write_csv=str(tmp_path / "w.csv"))
    assert "4 steps matched" in text and "from 15 weight copies" in text
    assert traffic["fetch_scale"] == 2.0 and traffic["write_scale"] == 1.0
    assert sum(l.rstrip().endswith(" 1.0100") for l in text.split("\n")) == 3, text
    for lab in ("attn_out", "gate|up", "down"):
        assert traffic["fetch_bytes_raw"][lab] == round(fetch[lab])
        assert traffic["hbm_bytes"][lab] == round(2.0 * fetch[lab])
    assert abs(traffic["hbm_bytes_per_launch"] / traffic["algorithmic_bytes_per_launch"] - 1.01) < 1e-6
    assert traffic["source_sha256_16"] == bench.source_hash("gemv_q4k")


def test_trace_summary_medians(tmp_path):
    path = tmp_path / "trace.csv"
    per = {lab: 1.0 for lab in ("quantize x_attn", "attn_out", "quantize x_ffn", "gate|up",
                                "quantize x_down", "down")}
    _decode_run(path, "none", 5, per, 1.0)
    text, _ = bench.summarize(1, trace_csv=str(path))
    assert "5 steps matched" in text
    assert any(l.startswith("gate|up") and "10.00" in l for l in text.split("\n")), text
    assert any(l.startswith("quantize x_down") and "2.00" in l for l in text.split("\n")), text


def test_clock_power_reads_the_marked_level(tmp_path):
    sclk = tmp_path / "pp_dpm_sclk"
    sclk.write_text("S: 100Mhz\n0: 500Mhz\n1: 2400Mhz *\n")
    pw = tmp_path / "power1_input"
    pw.write_text("1234500000\n")
    cp = bench.ClockPower()
    cp.sclk, cp.power = str(sclk), str(pw)
    assert cp._read() == (2400, 1234.5)
    cp.samples = [(100, 240.0), (2400, 1200.0), (2100, 1300.0), (2300, 1250.0)]
    s = cp.summary()
    assert s["busy_samples"] == 3 and s["sclk_MHz_median"] == 2300 and s["sclk_MHz_min"] == 2100
    assert s["power_W_median"] == 1250.0 and s["power_W_max"] == 1300.0


def test_mmq_roofline_sums_ops_over_time():
    ks = [{"op": "gate", "kernel": "kq_mmq_q4k", "shape": [1000, 2000, 500], "avg_us": 1.0,
           "tops": 2000.0, "frac_int8_peak": 0.4},
          {"op": "v", "kernel": "kq_mmq_q6k", "shape": [5, 5, 5], "avg_us": 9.0},
          {"op": "down", "kernel": "kq_mmq_q4k", "shape": [1000, 2000, 500], "avg_us": 3.0,
           "tops": 666.7, "frac_int8_peak": 0.1333}]
    r = bench.mmq_roofline({"workload": "none_such", "kernels": ks})
    # 2 launches of 2*1000*2000*500 = 2e9 ops in 4 us: 1000 TOPS
    assert r["achieved"] == 1000.0 and r["frac"] == 0.2 and r["bound"] == "mfma"
    assert set(r["per_launch"]) == {"gate", "down"} and "counters" not in r


def test_run_steps_whole_graphs_then_singles():
    """run_steps covers steps 0..n-1 exactly once, copy i % ncopies for step
    i: whole multi-step graphs first, one-step graphs for the remainder."""
    import bench

    class WL:
        ncopies = 3

        def __init__(self):
            self.eager = []

        def step(self, c):
            self.eager.append(c)

    log = []

    class G:
        def __init__(self, steps):
            self.steps = steps

        def replay(self):
            log.extend(self.steps)

    wl = WL()
    spg = bench.cycle_len(wl.ncopies)
    assert spg % wl.ncopies == 0 and spg >= bench.GRAPH_MIN
    graphs = {"steps_per_graph": spg, "many": G([i % 3 for i in range(spg)]),
              "single": [G([c]) for c in range(3)]}
    for n in (0, 1, spg - 1, spg, 2 * spg + 5, 200):
        log.clear()
        bench.run_steps(wl, n, graphs)
        assert log == [i % 3 for i in range(n)], n
    bench.run_steps(wl, 7, None)
    assert wl.eager == [i % 3 for i in range(7)]


def test_summarize_lds_counters(tmp_path):
    """With the LDS counters in the collection, the summary reports the LDS
    busy and bank-conflict fractions of CU-cycles and records them."""
    path = tmp_path / "c.csv"
    _collection(path, steps=3, ghz=2.0, mfma_busy=0.25, valu_x4=0.5, mops_factor=2, lds=(0.3, 0.02))
    text = bench.summarize_counters(9, str(path))
    assert "LDS busy = SQ_LDS_IDX_ACTIVE" in text
    assert text.count("LDS busy    30.0 %   bank-conflict   2.0 %") == 2, text
    rec = [json.loads(l[len("counters_json: "):]) for l in text.splitlines() if l.startswith("counters_json: ")]
    assert rec[0]["launches"]["down"]["lds_busy"] == 0.3
    assert rec[0]["launches"]["down"]["lds_bank_conflict"] == 0.02


def test_copy_scale_unequal_copy_counts():
    """The counter scale comes from plain copies of the weight tensors; each
    tensor may be copied a different number of times (per-launch rotations
    clone the small ones more), so readings are matched by size, not rank."""
    import random

    sizes = [9_437_184, 66_060_288, 33_030_144]
    rng = random.Random(5)
    readings = [z * 0.5 * rng.uniform(0.996, 1.004)
                for z, n in ((9_437_184, 62), (66_060_288, 8), (33_030_144, 17)) for _ in range(n)]
    sc = bench._copy_scale(readings, sizes)
    assert sc is not None and abs(sc - 2.0) < 0.01
    # readings that match no size consistently give no scale
    assert bench._copy_scale([1.0, 3.3, 7.7, 12.1], sizes) is None
