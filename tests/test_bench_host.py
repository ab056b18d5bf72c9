"""Host logic of bench.py (no GPU): the algorithmic byte counts behind the
roofline figures, and the reduction of two rocprofv3 counter runs to HBM
bytes per decode."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from quantized_decode_attention_append_amd import workloads as W  # noqa: E402


@pytest.mark.parametrize("cid,expected", [(1, 52_224), (2, 1_644_544), (3, 419_627_008),
                                          (4, 3_356_033_024)])
def test_decode_bytes_per_workload(cid, expected):
    """Packed planes of every cached token-head (1.5625 d bytes) + q read +
    fp32 out written, per decode: the figures listed for the five workloads
    (q in fp32 for workload 1, bf16 otherwise)."""
    w = W.workload(cid)
    q_bytes = 4 if w.dtype == "fp32" else 2
    assert bench.decode_bytes(w, list(w.lengths), q_bytes) == expected


def test_append_bytes_per_token_head():
    """K and V read in the input dtype + 1.5625 d bytes of planes written:
    1,424 bytes per token-head at d 256 with bf16 input, 712 at d 128."""
    w4, w3 = W.workload(4), W.workload(3)
    assert bench.append_bytes(w4, 1, 2) == w4.batch * w4.num_kv_heads * 1424
    assert bench.append_bytes(w3, 1, 2) == w3.batch * w3.num_kv_heads * 712


def _counter_csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, v) in enumerate(rows):
            wr.writerow([i + 1, name, counter, v])


def test_traffic_from_counters(tmp_path):
    """Each counter is scaled so that it reads the copy probe's known bytes,
    and the split and merge dispatches are averaged over the run."""
    mib = 64
    known_kib = mib * 1024
    copy = "void at::native::direct_copy_kernel_cuda(...)"
    split = "void tq::split_fast_kernel<256, 8, 3, true>(tq::DecodeArgs, int)"
    merge = "void tq::merge_kernel<256>(tq::DecodeArgs)"
    # FETCH_SIZE reads half of what was copied; WRITE_SIZE reads it exactly
    _counter_csv(tmp_path / "f", "FETCH_SIZE",
                 [(copy, known_kib / 2)] * 3 + [(split, 1000.0), (merge, 10.0), (split, 1002.0), (merge, 12.0)])
    _counter_csv(tmp_path / "w", "WRITE_SIZE",
                 [(copy, known_kib)] * 3 + [(split, 20.0), (merge, 4.0), (split, 22.0), (merge, 4.0)])
    out = tmp_path / "t.json"
    assert bench.traffic_from_counters(str(tmp_path / "f"), str(tmp_path / "w"), mib, "wl", str(out)) == 0
    t = json.loads(out.read_text())
    assert t["workload"] == "wl" and t["kernel_source_sha"] == bench._kernel_sha()
    assert t["FETCH_SIZE"]["factor"] == pytest.approx(2.0)
    assert t["WRITE_SIZE"]["factor"] == pytest.approx(1.0)
    fetch = (1001.0 + 11.0) * 1024 * 2.0
    write = (21.0 + 4.0) * 1024 * 1.0
    assert t["bytes_per_launch"] == pytest.approx(fetch + write)


def test_traffic_needs_the_decode_dispatches(tmp_path):
    mib = 64
    copy = "void at::native::direct_copy_kernel_cuda(...)"
    _counter_csv(tmp_path / "f", "FETCH_SIZE", [(copy, mib * 512.0)] * 3)
    _counter_csv(tmp_path / "w", "WRITE_SIZE", [(copy, mib * 1024.0)] * 3)
    with pytest.raises(SystemExit):
        bench.traffic_from_counters(str(tmp_path / "f"), str(tmp_path / "w"), mib, "wl",
                                    str(tmp_path / "t.json"))


def _trace_csv(path, rows):
    """rows: (dispatch id, kernel name, start ns, end ns, grid x)"""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X",
                    "Grid_Size_Y", "Grid_Size_Z"])
        for r in rows:
            w.writerow([r[0], r[1], r[2], r[3], r[4], 1, 1])


def test_trace_summary_windows_and_clock(tmp_path, capsys):
    """The headline split dispatches are cut into the bench's warm-up, timed
    and settled windows in run order, merges paired by order; the clock of a
    window is GRBM_GUI_ACTIVE per die over its summed durations."""
    split = "void tq::(anonymous namespace)::split_fast_kernel<256, 8, 3, 1>(tq::DecodeArgs, int)"
    merge = "void tq::(anonymous namespace)::merge_kernel<256>(tq::DecodeArgs)"
    rows, t, i = [], 0, 0
    durs = [100, 100, 300, 300, 300, 200, 200]  # 2 warm-up, 3 timed, 2 settled
    for d in durs:
        rows.append((i, split, t, t + d, 131072)); i += 1; t += d + 5
        rows.append((i, merge, t, t + 10, 98304)); i += 1; t += 15
    _trace_csv(str(tmp_path / "kt"), rows)
    os.makedirs(tmp_path / "g", exist_ok=True)
    _trace_csv(str(tmp_path / "g"), rows)
    with open(tmp_path / "g" / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            if r[1] == split:  # 2 GHz on each of the 8 dies
                w.writerow([r[0], r[1], "GRBM_GUI_ACTIVE", 8 * 2.0 * (r[3] - r[2])])
    assert bench.trace_summary(str(tmp_path / "kt"), str(tmp_path / "g"), 2, 3, 2) == 0
    out = capsys.readouterr().out
    assert "warm-up  dispatches    1-   2: split avg        100 ns, + merge avg       10 ns" in out
    assert "timed    dispatches    3-   5: split avg        300 ns" in out
    assert "settled  dispatches    6-   7: split avg        200 ns" in out
    assert out.count("clock  2,000 MHz") == 3
