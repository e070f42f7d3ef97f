"""Host-side logic of the benchmark that needs no GPU: the one-GPU guard, the source hash that
decides whether a stored HBM-traffic figure still belongs to a kernel, the calibration of the
FETCH_SIZE / WRITE_SIZE counters by the probe copy, and the rocprofv3 summaries (synthetic CSV
files in the layout rocprofv3 writes)."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


@pytest.fixture
def fake_csrc(tmp_path, monkeypatch):
    d = tmp_path / "csrc"
    d.mkdir()
    (d / "k_x.hip").write_text('#include "dev.hpp"\n#include "launch.hpp"\n__global__ void k() {}\n')
    (d / "dev.hpp").write_text("// device helper v1\n")
    (d / "launch.hpp").write_text("// host declarations v1\n")
    monkeypatch.setattr(bench, "CSRC", str(d))
    return d


def test_source_hash_follows_the_kernel_and_its_device_headers_only(fake_csrc):
    h0 = bench._source_hash("k_x.hip")
    (fake_csrc / "launch.hpp").write_text("// host declarations v2\n")      # host-only header
    assert bench._source_hash("k_x.hip") == h0
    (fake_csrc / "dev.hpp").write_text("// device helper v2\n")             # included device header
    h1 = bench._source_hash("k_x.hip")
    assert h1 != h0
    (fake_csrc / "k_x.hip").write_text((fake_csrc / "k_x.hip").read_text() + "// comment\n")
    assert bench._source_hash("k_x.hip") != h1                           # any edit of the kernel file


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(fake_csrc, tmp_path, monkeypatch):
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps({"k": {"source": "k_x.hip", "source_sha256": bench._source_hash("k_x.hip"),
                                    "fetch_bytes": 1000, "write_bytes": 24}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.traffic_for("k") == 1024
    assert bench.traffic_for("missing") is None
    (fake_csrc / "dev.hpp").write_text("// changed\n")
    assert bench.traffic_for("k") is None


def _pmc_rows(counter, entries):
    return [{"Kernel_Name": k, "Grid_Size": str(g), "Counter_Name": counter, "Counter_Value": str(v)}
            for k, g, v in entries]


def test_traffic_entry_scales_each_counter_by_the_probe_copy(fake_csrc, tmp_path):
    kern = "void ssn::(anonymous namespace)::k_x<1>"
    copy = bench.COPY_KERNEL
    # the 2 GiB probe copy reads as 1 GiB on FETCH_SIZE (factor 2) and 2 GiB on WRITE_SIZE (factor 1);
    # a smaller copy with the same grid must not be taken for the probe
    fetch = _pmc_rows("FETCH_SIZE", [(copy, 131072, 1 << 20), (copy, 131072, 1000.0), (kern + "(int)", 4096, 300.0),
                                     (kern + "(int)", 4096, 500.0), (kern + "(int)", 8192, 9.0)])
    write = _pmc_rows("WRITE_SIZE", [(copy, 131072, 1 << 21), (kern + "(int)", 4096, 64.0)])
    _write_csv(str(tmp_path / "f" / "run" / "run_counter_collection.csv"), fetch)
    _write_csv(str(tmp_path / "w" / "run" / "run_counter_collection.csv"), write)
    e = bench.traffic_entry(str(tmp_path / "f"), str(tmp_path / "w"), kern, 4096, "k_x.hip", "s.md")
    assert e["fetch_calibration"] == 2.0 and e["write_calibration"] == 1.0
    assert e["fetch_bytes"] == int(400.0 * 1024 * 2.0)          # average of the two dispatches at that grid
    assert e["write_bytes"] == 64 * 1024
    assert e["source_sha256"] == bench._source_hash("k_x.hip")
    with pytest.raises(SystemExit):
        bench.traffic_entry(str(tmp_path / "f"), str(tmp_path / "w"), kern, 1, "k_x.hip", "s.md")


def test_trace_summary_lists_kernels_by_total_time_and_by_grid(tmp_path):
    d = tmp_path / "trace" / "run"
    _write_csv(str(d / "run_kernel_stats.csv"), [
        {"Name": "void ssn::(anonymous namespace)::k_a(int)", "Calls": "2", "TotalDurationNs": "3000",
         "AverageNs": "1500", "MinNs": "1000", "MaxNs": "2000", "Percentage": "75.0"},
        {"Name": "void ssn::(anonymous namespace)::k_b(int)", "Calls": "1", "TotalDurationNs": "1000",
         "AverageNs": "1000", "MinNs": "1000", "MaxNs": "1000", "Percentage": "25.0"}])
    tr = [{"Kernel_Name": "void ssn::(anonymous namespace)::k_a(int)", "Grid_Size_X": "256", "Grid_Size_Y": "1",
           "Grid_Size_Z": "1", "Start_Timestamp": str(t0), "End_Timestamp": str(t0 + dt)}
          for t0, dt in ((0, 1000), (5000, 2000))]
    _write_csv(str(d / "run_kernel_trace.csv"), tr)
    out = tmp_path / "s.md"
    bench.summarize("trace", str(out), [str(tmp_path / "trace")], "rocprofv3 --kernel-trace ...")
    text = out.read_text()
    assert "rocprofv3 --kernel-trace ..." in text
    assert text.index("k_a(int)") < text.index("k_b(int)")                  # larger total first
    assert "| `void ssn::(anonymous namespace)::k_a(int)` | 2 | 1.50 | 1.00 | 2.00 | 75.00 |" in text
    # per grid: median (upper of two) 2.00 us, mean 1.50 us, min 1.00 us
    assert "| `ssn::k_a` | 256 | 2 | 2.00 | 1.50 | 1.00 |" in text


def test_counter_summary_averages_each_counter_per_kernel_and_grid(tmp_path):
    a, b = "void ssn::(anonymous namespace)::k_a(int)", "void ssn::(anonymous namespace)::k_b(int)"
    _write_csv(str(tmp_path / "f" / "run" / "run_counter_collection.csv"),
               _pmc_rows("FETCH_SIZE", [(a, 256, 10.0), (a, 256, 30.0), (a, 512, 7.0), (b, 64, 1.0)]))
    _write_csv(str(tmp_path / "s" / "run" / "run_counter_collection.csv"),
               _pmc_rows("SQ_INSTS_MFMA", [(a, 256, 4.0), (a, 256, 4.0)]))
    out = tmp_path / "c.md"
    bench.summarize("pmc", str(out), [str(tmp_path / "f"), str(tmp_path / "s")], "rocprofv3 --pmc ...")
    text = out.read_text()
    assert "| kernel | grid | dispatches | FETCH_SIZE | SQ_INSTS_MFMA |" in text
    assert f"| `{a}` | 256 | 2 | 20.0 | 4.0 |" in text       # mean of the two dispatches per counter
    assert f"| `{a}` | 512 | 1 | 7.0 |  |" in text            # a counter not read for that grid stays empty
    assert f"| `{b}` | 64 | 1 | 1.0 |  |" in text
