"""Host logic of bench.py (no GPU).

* The source hash that keys the committed HBM-traffic records ignores
  comments and whitespace but not code.
* The counter summary turns a counter collection into matrix-core and VALU
  busy fractions, int8 MFMA work against 2*M*N*K and the engine clock; checked
  on a small synthetic collection whose answers are known by construction.
"""
import csv

import bench


def test_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    (tmp_path / "a.hip").write_text("int f(int x) { return x + 1; } // one\n/* a\n block */\n")
    (tmp_path / "b.hip").write_text("// header\nint f(int x)  {\n  return x + 1;   // uno\n}\n")
    (tmp_path / "c.hip").write_text("int f(int x) { return x + 2; } // one\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"a": "a.hip", "b": "b.hip", "c": "c.hip"})
    assert bench.source_hash("a") == bench.source_hash("b")
    assert bench.source_hash("a") != bench.source_hash("c")


def _collection(path, steps, ghz, mfma_busy, valu_busy, mops_factor):
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
                        "SQ_ACTIVE_INST_VALU": valu_busy * simd_cycles / 4,
                        "SQ_INSTS_MFMA": 1.0, "SQ_INSTS_VALU": 1.0,
                        "GRBM_GUI_ACTIVE": 8 * cyc}
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
    _collection(path, steps=3, ghz=2.0, mfma_busy=0.25, valu_busy=0.5, mops_factor=2)
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
        assert "VALU busy   50.0 %" in block, block
        assert "= 2.000 x 2MNK" in block, block
        assert "clock     2.000 GHz" in block, block
        assert "dispatch time 100.0 us" in block, block
