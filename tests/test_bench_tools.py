"""The benchmark's measurement helpers on the CPU: the phases it reads from
per-work-group timestamps, and the summaries it writes from rocprofv3 output
(counter passes calibrated on a copy of known size, kernel statistics), each
on small hand-made inputs whose answers are known."""
import argparse
import csv
import json

import numpy as np
import pytest

import bench


def stamps(rows):
    """A stamps array as the stamped kernels write it: per work-group the four
    100 MHz stamps, the XCD and the compute unit id (8 slots)."""
    st = np.zeros((len(rows), 8), dtype=np.int64)
    for g, (t0, t1, t2, t3, xcd) in enumerate(rows):
        st[g, :5] = (t0, t1, t2, t3, xcd)
    return st


def test_stamp_stats_reads_the_phases():
    # ticks of 10 ns; the earliest start is the origin
    base = 10_000_000
    rows = [(base + 0, base + 300, base + 320, base + 4000, 0),     # start 0, staging 3 us, regs 0.2, stream 36.8
            (base + 20, base + 360, base + 380, base + 4100, 1),    # start 0.2, staging 3.4
            (base + 40, base + 340, base + 360, base + 4400, 1)]    # the last to end: 44 us
    s = bench.stamp_stats(stamps(rows), 3)
    assert s["span"] == pytest.approx(44.0)
    assert s["start_spread"] == pytest.approx(0.4)
    assert s["staging"] == pytest.approx(3.0)          # median of 3.0, 3.4, 3.0
    assert s["to_registers"] == pytest.approx(0.2)
    assert s["weight_stream"] == pytest.approx(37.2)   # median of 36.8, 37.2, 40.4
    assert s["end_median"] == pytest.approx(41.0)
    assert s["end_first"] == pytest.approx(40.0)
    assert s["xcd_end_median"] == {0: pytest.approx(40.0), 1: pytest.approx(42.5)}


def test_stamp_stats_ignores_slots_past_the_grid():
    st = np.vstack([stamps([(100, 200, 210, 1100, 3)]), np.full((5, 8), 7, dtype=np.int64)])
    s = bench.stamp_stats(st, 1)
    assert s["span"] == pytest.approx(10.0) and s["xcd_end_median"] == {3: pytest.approx(10.0)}


def write_counters(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for d, name, counter, value in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_per_dispatch_adds_the_rows_of_a_dispatch(tmp_path):
    p = tmp_path / "c.csv"
    write_counters(p, [(1, "k", "FETCH_SIZE", 10.0), (1, "k", "FETCH_SIZE", 5.5), (1, "k", "WRITE_SIZE", 99.0),
                       (2, "j", "FETCH_SIZE", 3.0)])
    assert bench.pmc_per_dispatch(str(p), "FETCH_SIZE") == {1: ("k", 15.5), 2: ("j", 3.0)}
    assert bench.pmc_per_dispatch(str(p), "WRITE_SIZE") == {1: ("k", 99.0)}


def pmc_args(fetch, write, **kw):
    a = dict(dominant="kq::qgemv1_dma_kernel<12, 2, 1024, true, 64>", launch_class="w1+w3", workload="unit",
             m=1, pmc_command="rocprofv3 --pmc ...", summarize_pmc=[str(fetch), str(write)])
    a.update(kw)
    return argparse.Namespace(**a)


def test_summarize_pmc_calibrates_on_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    monkeypatch.setattr(bench, "library_hash", lambda: "0123456789abcdef")
    dom = "void kq::qgemv1_dma_kernel<12, 2, 1024, true, 64>(kq::Segs, long, int, int, int, float const*)"
    copy_kib = bench.CALIB_BYTES / 1024 / 2.0          # the counter reads half the copy's bytes: factor 2
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    write_counters(fetch, [(1, "void at::native::copy_kernel", "FETCH_SIZE", copy_kib),
                           (2, "void at::native::copy_kernel", "FETCH_SIZE", 10.0),      # a small copy: not the reference
                           (3, dom, "FETCH_SIZE", 1000.0), (4, dom, "FETCH_SIZE", 1200.0),
                           (5, "void kq::qgemv1_dma_kernel<12, 4, 512, false, 64>(...)", "FETCH_SIZE", 7.0)])
    write_counters(write, [(1, "void at::native::copy_kernel", "WRITE_SIZE", copy_kib / 2.0),   # factor 4
                           (3, dom, "WRITE_SIZE", 3.0), (4, dom, "WRITE_SIZE", 5.0)])
    assert bench.summarize_pmc(pmc_args(fetch, write)) == 0
    r = json.loads((tmp_path / "profiles" / "traffic_unit.json").read_text())
    assert r["fetch_factor"] == pytest.approx(2.0) and r["write_factor"] == pytest.approx(4.0)
    assert r["fetch_bytes_per_launch"] == int(1100.0 * 1024 * 2.0)
    assert r["write_bytes_per_launch"] == int(4.0 * 1024 * 4.0)
    assert r["bytes_per_launch"] == int(1100.0 * 1024 * 2.0 + 4.0 * 1024 * 4.0)
    assert r["fetch_dispatches"] == 2 and r["library_sha256_16"] == "0123456789abcdef" and r["m"] == 1


def test_summarize_pmc_needs_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    monkeypatch.setattr(bench, "library_hash", lambda: "0")
    f = tmp_path / "f.csv"
    write_counters(f, [(3, "void kq::qgemv1_dma_kernel<12, 2, 1024, true, 64>(x)", "FETCH_SIZE", 1.0)])
    with pytest.raises(SystemExit, match="copy"):
        bench.summarize_pmc(pmc_args(f, f))


def test_summarize_trace_averages_the_dominant_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    stats = tmp_path / "kernel_stats.csv"
    rows = [("kq::qgemv1_dma_kernel<12, 2, 1024, true, 64>(kq::Segs, ...)", 40, 45000.0 * 40, 44000, 46000, 40.0),
            ("kq::qgemv1_kernel<14, 1, 1024, false, 64>(kq::Segs, ...)", 40, 36000.0 * 40, 35000, 37000, 32.0)]
    with open(stats, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        for name, calls, total, mn, mx, pct in rows:
            w.writerow([name, calls, total, total / calls, mn, mx, pct])
    line = tmp_path / "bench.json"
    line.write_text("noise\n" + json.dumps({"ms_per_step": 8.4, "value": 5150.0, "unit": "GB/s", "parity": "pass",
                                            "launch_classes": [{"launch": "w1+w3", "per_step": 80, "avg_us": 45.0,
                                                                "GBps": 5872.0, "frac": 0.734}]}) + "\n")
    args = argparse.Namespace(summarize_trace=str(stats), profile_name="unit_profile", pmc_command="rocprofv3 ...",
                              dominant="kq::qgemv1_dma_kernel<12, 2, 1024, true, 64>", bench_line=str(line))
    assert bench.summarize_trace(args) == 0
    text = (tmp_path / "profiles" / "unit_profile.txt").read_text()
    assert "dominant kernel kq::qgemv1_dma_kernel<12, 2, 1024, true, 64>: 40 calls, average 45000 ns" in text
    assert "w1+w3" in text and "parity pass" in text
