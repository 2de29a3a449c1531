"""Host logic of bench.py, on the CPU: the summaries it makes of rocprofv3 output (kernel
trace with the timed steps picked out by the marker launches, HBM bytes per launch from the
FETCH_SIZE/WRITE_SIZE counters scaled by the copy calibration, per-wave SQ counters), the
refusal of more than one GPU, and the oracle baseline over every fill of the step."""
import csv
import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
import bench  # noqa: E402

ZIG = bench.FILL_KERNELS["normal_f64"] + "(tk::ZigArgs)"
MARK = "void tk::k_vec_fill<tk::OpConst, 1, false>(tk::OpConst, unsigned long)"


def write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def trace_row(name, grid, start, dur):
    return {"Kernel_Name": name, "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
            "Start_Timestamp": start, "End_Timestamp": start + dur, "VGPR_Count": 32, "LDS_Block_Size": 0}


def test_trace_summary_takes_the_dispatches_between_the_markers(tmp_path):
    rows = [trace_row(ZIG, 33554432, 0, 400_000),               # warm-up, outside
            trace_row(MARK, 256, 1_000_000, 2_000),             # marker before the timed steps
            trace_row(ZIG, 33554432, 2_000_000, 350_000),
            trace_row(ZIG, 33554432, 3_000_000, 360_000),
            trace_row(MARK, 256, 4_000_000, 2_000),             # marker after
            trace_row(ZIG, 33554432, 5_000_000, 500_000)]       # after, outside
    write_csv(tmp_path / "x_kernel_trace.csv", rows)
    timed = bench.trace_summary(str(tmp_path), min_share=0.0, timed_only=True)
    line = [l for l in timed.splitlines() if "k_zig_table_pass" in l]
    assert len(line) == 1
    cells = [c.strip() for c in line[0].split("|")]
    assert cells[3] == "2" and cells[4] == "355.00"             # calls, average us
    assert "OpConst" not in timed                               # the markers themselves are left out
    every = bench.trace_summary(str(tmp_path), min_share=0.0)
    zig = [l for l in every.splitlines() if "k_zig_table_pass" in l][0]
    assert [c.strip() for c in zig.split("|")][3] == "4"


def counter_rows(kernel, grid, counter, values):
    return [{"Kernel_Name": kernel, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": v} for v in values]


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path):
    fetch, write = tmp_path / "fetch", tmp_path / "write"
    fetch.mkdir()
    write.mkdir()
    copy = bench.FILL_KERNELS["calib_copy"]
    u32 = bench.FILL_KERNELS["u32"] + "(tk::OpWord32<false>, unsigned long)"
    # the copy of 1 GiB reads half of it in FETCH_SIZE units (factor 2) and writes it whole
    write_csv(fetch / "f_counter_collection.csv",
              counter_rows(copy, 262144, "FETCH_SIZE", [524288.0] * 3) + counter_rows(u32, 67108864, "FETCH_SIZE", [10.0] * 3))
    write_csv(write / "w_counter_collection.csv",
              counter_rows(copy, 262144, "WRITE_SIZE", [1048576.0] * 3)
              + counter_rows(u32, 67108864, "WRITE_SIZE", [1048576.0 * 1.25] * 3))
    out = tmp_path / "rec.json"
    table = bench.pmc_summary(str(fetch), str(write), str(out))
    rec = json.load(open(out))
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    k = rec["kernels"]["u32"]
    assert k["traffic_bytes"] == pytest.approx(10 * 1024 * 2 + 1048576 * 1.25 * 1024)
    assert k["algorithmic_bytes"] == 4 << 28
    assert k["source_sha256"] == bench._sources_sha(bench.FILL_SOURCES["u32"])
    assert "| u32 |" in table and "1.2500" in table


def test_counter_summary_divides_instructions_by_waves(tmp_path):
    u64 = bench.FILL_KERNELS["u64"] + "(tk::OpWord64<false>, unsigned long)"
    write_csv(tmp_path / "s_counter_collection.csv",
              counter_rows(u64, 134217728, "SQ_WAVES", [2000.0]) + counter_rows(u64, 134217728, "SQ_INSTS_VALU", [94000.0])
              + counter_rows(u64, 134217728, "VALUBusy", [53.0]))
    table = bench.counter_summary(str(tmp_path))
    row = [l for l in table.splitlines() if l.startswith("| u64 |")][0]
    assert "47.0 / wave" in row and "53" in row


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_times_every_fill_of_the_step():
    rec = bench.cpu_baseline(1 << 12, 10)
    assert rec["kind"] == "oracle" and rec["unit"] == "GiB/s" and rec["value"] > 0
    assert rec["cores"] >= 1 and rec["single_core"]["cores"] == 1
    import tk_inputs as ti
    assert len(rec["per_fill"]) == len(bench._oracle_jobs(ti.normal_x(1 << 12)))
    for name, t in rec["per_fill"].items():
        assert t["all_cores_s"] >= 0 and t["single_core_s_scaled"] >= 0, name
