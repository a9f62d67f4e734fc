"""Host checks of the profiler summaries (no GPU): the kernel-trace tail
statistics, the calibrated HBM traffic and the SQ-derived fractions, on
small synthetic rocprofv3 CSV files, and bench.py's use of the committed
traffic summary (only when it was taken on the current kernel source)."""

import csv
import importlib.util
import os

import pytest

from sparse_mla_decode_gather_amd import rocprof_summary as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEC = "void smla::(anonymous namespace)::decode_hd_kernel<false, false, false, false, true, false>(smla::DecodeParams)"
COMB = "smla::(anonymous namespace)::combine_kernel(smla::CombineParams)"
COPY = "void at::native::copy_kernel(float*)"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _trace(tmp_path, durations, combine=None):
    rows, t = [], 1000
    for i, d in enumerate(durations):
        rows.append([i + 1, DEC, t, t + d])
        t += d + 50
        if combine is not None:
            rows.append([1000 + i, COMB, t, t + combine[i]])
            t += combine[i] + 50
    _write(str(tmp_path / "trace" / "run_kernel_trace.csv"),
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    _write(str(tmp_path / "trace" / "run_kernel_stats.csv"),
           ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
           [[DEC, len(durations), sum(durations) / len(durations), min(durations),
             max(durations), 90.0]])
    return str(tmp_path / "trace")


def test_tail_is_the_last_k_dispatches(tmp_path):
    # settling launches first (slow), then the timed ones
    d = _trace(tmp_path, [400] * 20 + [250, 260, 270, 280])
    out = rs.timed_tail(d, 4)
    vals = dict(line.split(": ") for line in out.splitlines() if not line.startswith("#"))
    assert vals["tail_dispatches"] == "4"
    assert float(vals["tail_average_ns"]) == pytest.approx(265.0)
    assert vals["tail_min_ns"] == "250" and vals["tail_max_ns"] == "280"
    assert "the last 4 of 24 dispatches of decode_hd_kernel<" in out
    full = rs.stats(d, "cmd")
    assert full.splitlines()[1] == "# command: cmd"
    assert "decode_hd_kernel<false, false, false, false, true, false> | 24 |" in full


def test_tail_reports_the_combine_kernel_too(tmp_path):
    d = _trace(tmp_path, [100, 110, 120], combine=[10, 20, 30])
    vals = dict(line.split(": ") for line in rs.timed_tail(d, 2).splitlines()
                if not line.startswith("#"))
    assert float(vals["tail_average_ns"]) == pytest.approx(115.0)
    assert float(vals["combine_tail_average_ns"]) == pytest.approx(25.0)


def test_tail_needs_k_dispatches(tmp_path):
    d = _trace(tmp_path, [100, 110])
    with pytest.raises(ValueError):
        rs.timed_tail(d, 3)


def _counters(path, rows):
    _write(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)


def test_traffic_calibrates_by_the_copy(tmp_path):
    gib = 1 << 30
    # FETCH_SIZE reads half the copy's bytes, WRITE_SIZE all of them; the
    # decode's counters are split over two rows per dispatch (summed)
    f_rows, w_rows = [], []
    for i in range(5):
        f_rows += [[i, DEC, "FETCH_SIZE", 300.0], [i, DEC, "FETCH_SIZE", 200.0]]
        w_rows += [[i, DEC, "WRITE_SIZE", 64.0]]
    for i in range(3):
        f_rows.append([100 + i, COPY, "FETCH_SIZE", gib / 2 / 1024])
        w_rows.append([100 + i, COPY, "WRITE_SIZE", gib / 1024])
    _counters(str(tmp_path / "f" / "run_counter_collection.csv"), f_rows)
    _counters(str(tmp_path / "w" / "run_counter_collection.csv"), w_rows)
    out = rs.traffic(str(tmp_path / "f"), str(tmp_path / "w"), gib, "cmd")
    vals = dict(line.split(": ") for line in out.splitlines() if not line.startswith("#"))
    assert vals["fetch_calibration_factor"] == "0.5000"
    assert vals["write_calibration_factor"] == "1.0000"
    assert int(vals["fetch_bytes_per_launch"]) == 500 * 1024 * 2
    assert int(vals["write_bytes_per_launch"]) == 64 * 1024
    assert int(vals["traffic_bytes_per_launch"]) == 500 * 2048 + 64 * 1024
    assert vals["kernel_source_digest"] == rs.kernel_source_digest()


def test_sq_fractions(tmp_path):
    rows = []
    for i in range(3):
        rows += [[i, DEC, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0],
                 [i, DEC, "GRBM_GUI_ACTIVE", 8 * 1000.0],
                 [i, DEC, "SQ_WAIT_ANY", 25.0], [i, DEC, "SQ_WAVE_CYCLES", 100.0]]
    _counters(str(tmp_path / "s" / "run_counter_collection.csv"), rows)
    out = rs.sq([str(tmp_path / "s")], "cmd")
    assert "MFMA busy fraction of SIMD cycles = 0.500" in out
    assert "(SQ_WAIT_ANY / SQ_WAVE_CYCLES) = 0.250" in out


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_uses_traffic_only_on_the_current_source(tmp_path):
    bench = _bench()
    good = tmp_path / "good.txt"
    good.write_text("# x\ntraffic_bytes_per_launch: 1234\n"
                    f"kernel_source_digest: {rs.kernel_source_digest()}\n")
    stale = tmp_path / "stale.txt"
    stale.write_text("# x\ntraffic_bytes_per_launch: 1234\nkernel_source_digest: 0000\n")
    bench.COUNTERS = str(good)
    assert bench.measured_traffic() == 1234.0
    bench.COUNTERS = str(stale)
    assert bench.measured_traffic() is None
    bench.COUNTERS = str(tmp_path / "missing.txt")
    assert bench.measured_traffic() is None


def test_digest_ignores_comments_and_layout():
    code = 'int a = 1;\nfloat b = a * 2;  // scale\nconst char* s = "x // y";\n'
    same = '/* header */\nint a = 1;   float b = a * 2;\nconst char* s = "x // y";  // s\n'
    other = 'int a = 1;\nfloat b = a * 3;\nconst char* s = "x // y";\n'
    assert rs._code_only(code) == rs._code_only(same)
    assert rs._code_only(code) != rs._code_only(other)
    assert '"x // y"' in rs._code_only(code)
