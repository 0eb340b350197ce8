"""Host logic behind the profile summaries: dispatches are dealt to workloads by
launch order, and the clock / MFMA-busy table is computed from the counters as
its header states (no GPU; synthetic rocprofv3 CSVs)."""
import csv
import os

import bench


def test_split_by_plan_deals_dispatches_in_launch_order():
    plan = [("w1", "gate_up", 2), ("w1", "down", 2), ("w2", "gate_up", 1)]
    dispatches = {"gate_up": [(5, 50.0), (1, 10.0), (9, 90.0)], "down": [(2, 20.0), (6, 60.0)]}
    out = bench.split_by_plan(plan, dispatches)
    assert out[("w1", "gate_up")] == [10.0, 50.0]
    assert out[("w2", "gate_up")] == [90.0]
    assert out[("w1", "down")] == [20.0, 60.0]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_busy_summary_clock_and_busy_share(tmp_path):
    d = tmp_path / "busy"
    d.mkdir()
    _write(d / "run_agent_info.csv", [
        {"Agent_Type": "CPU", "Num_Xcc": "0", "Simd_Count": "0"},
        {"Agent_Type": "GPU", "Num_Xcc": "8", "Simd_Count": "1024"}])
    sym = bench.KERNEL_SYMBOLS["gate_up"]
    ns = 1_000_000                      # a 1 ms dispatch
    cyc = 1.8e6                         # one XCD's active cycles: 1.8 GHz
    rows = [
        {"Dispatch_Id": 1, "Kernel_Name": f"wide::{sym}(x)", "Counter_Name": "GRBM_GUI_ACTIVE",
         "Counter_Value": 8 * cyc, "Start_Timestamp": 0, "End_Timestamp": ns},
        {"Dispatch_Id": 1, "Kernel_Name": f"wide::{sym}(x)",
         "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": 0.5 * 1024 * cyc,
         "Start_Timestamp": 0, "End_Timestamp": ns}]
    _write(d / "run_counter_collection.csv", rows)
    plan = [("wl", "gate_up", 1)]
    bench.busy_summary(str(tmp_path), "cmd PMC", plan, bench.split_by_plan, out_dir=str(tmp_path))
    text = open(os.path.join(tmp_path, "mfma_busy_llama8b.md")).read()
    row = next(line for line in text.splitlines() if line.startswith("| gate_up | wl |"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[2] == "1000.0"          # duration in us
    assert cells[3] == "1.80"            # GHz
    assert cells[4] == "50.0%"
    assert cells[5] == f"{bench.PEAK_BF16_TFLOPS * 1.8 / 2.4:.0f}"
