"""Host logic of the profiling summaries: kernel-name shortening, counter
calibration against the copy of known size, and the source hash that gates the
stored traffic figure in bench.py."""
import csv
import json
import os

from hybrid_linear_attention_gdn_amd import rocprof_summary as rs

HDR = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size", "Kernel_Id",
       "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
       "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
CHAIN = ("void gdn::mfma::(anonymous namespace)::scan_kernel<false, false, false, false>"
         "(gdn::mfma::(anonymous namespace)::ScanArgs)")
NEG = ("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)"
       "::{lambda()#2}, std::array<char*, 2ul> >(int, at::native::neg_kernel_cuda)")


def test_short_name():
    assert rs.short_name(CHAIN) == "scan_kernel<false, false, false, false>"
    assert rs.short_name("gdn::mfma::(anonymous namespace)::intra_kernel(unsigned short const*)") == "intra_kernel"
    assert rs.short_name(NEG).startswith("vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda")


def _counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(HDR)
        for i, (name, value) in enumerate(rows):
            w.writerow([i, i + 1, "Agent 1", 1, 1, 1, 64, 1, name, 256, 0, 0, 8, 0, 8, counter, value, 0, 1])


def test_traffic_calibration(tmp_path):
    # the copy of 4 MiB reads as half its size on FETCH_SIZE (2x factor) and exactly on WRITE_SIZE
    _counters(str(tmp_path / "f"), "FETCH_SIZE", [(CHAIN, 100.0), (CHAIN, 300.0), (NEG, 2048.0)])
    _counters(str(tmp_path / "w"), "WRITE_SIZE", [(CHAIN, 50.0), (CHAIN, 50.0), (NEG, 4096.0)])
    out_json, out_md = str(tmp_path / "t.json"), str(tmp_path / "t.md")
    rs.main(["traffic", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--copy-mib", "4",
             "--kernel", "scan_kernel", "--stage", "scan", "--workload", "w", "--fetch-command", "cf",
             "--write-command", "cw", "--json", out_json, "--md", out_md, "--launches-per-step", "3"])
    rec = json.load(open(out_json))
    assert rec["calibration"]["fetch_factor"] == 2.0 and rec["calibration"]["write_factor"] == 1.0
    assert rec["fetch_bytes_per_launch"] == 200 * 1024 * 2       # mean 200 KiB, doubled
    assert rec["write_bytes_per_launch"] == 50 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["bytes_per_step"] == 3 * rec["bytes_per_launch"]
    assert rec["source_hash"] == rs.kernel_source_hash("scan", True)
    assert "cf" in open(out_md).read()


def test_source_hash_tracks_the_kernel_files():
    a = rs.kernel_source_hash("scan", True)
    b = rs.kernel_source_hash("portable", False)
    assert a != b and len(a) == 16
    assert rs.kernel_source_hash("scan", True) == a


def test_source_hash_ignores_comments_and_layout():
    a = rs._code_only("int x = 1; // note\n/* block\n comment */  int  y = 2;\n")
    assert a == "int x = 1; int y = 2;"
    assert rs._code_only("a //c\nb") != rs._code_only("a b c")


def test_counters_table(tmp_path, capsys):
    # two counters per dispatch, two dispatches of one kernel and one of another;
    # kernels whose counters are all zero are left out of the table
    d = tmp_path / "c"
    os.makedirs(d)
    with open(d / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(HDR)
        rows = [(1, CHAIN, "MfmaUtil", 10.0), (1, CHAIN, "LdsBankConflict", 0.5),
                (2, CHAIN, "MfmaUtil", 20.0), (2, CHAIN, "LdsBankConflict", 0.25),
                (3, NEG, "MfmaUtil", 0.0), (3, NEG, "LdsBankConflict", 0.0)]
        for i, name, counter, value in rows:
            w.writerow([i, i, "Agent 1", 1, 1, 1, 64, 1, name, 256, 0, 0, 8, 0, 8, counter, value, 0, 1])
    rs.main(["counters", str(d), "--command", "rocprofv3 --pmc MfmaUtil LdsBankConflict -- x"])
    out = capsys.readouterr().out
    assert "rocprofv3 --pmc MfmaUtil LdsBankConflict -- x" in out
    assert "| `scan_kernel<false, false, false, false>` | 2 | 15 | 0.375 |" in out
    assert "neg_kernel" not in out
    assert "MfmaUtil:" in out and "LdsBankConflict:" in out


def test_window_mean_takes_the_timed_dispatches_in_start_order(tmp_path):
    """Dispatches listed out of start order; other kernels interleaved; the
    window counts only the named kernel's dispatches, ordered by start."""
    d = tmp_path / "kt"
    os.makedirs(d)
    rows = []  # (name, start, end): durations 10, 20, ..., 60 us at starts 0, 100, ..., 500 us
    for i in range(6):
        rows.append((CHAIN, 100_000 * i, 100_000 * i + 10_000 * (i + 1)))
        rows.append((NEG, 100_000 * i + 90_000, 100_000 * i + 95_000))
    rows.reverse()
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, (name, s, e) in enumerate(rows):
            w.writerow(["KERNEL_DISPATCH", i + 1, name, s, e])
    mean, total = rs.window_mean_us(str(d), "scan_kernel", 2, 3)
    assert total == 6 and abs(mean - 40.0) < 1e-9  # dispatches 2, 3, 4: 30, 40, 50 us
    import pytest
    with pytest.raises(SystemExit):
        rs.window_mean_us(str(d), "scan_kernel", 4, 3)
