"""bench.py's host logic (CPU only): the one-GPU rule, the kernel-source
hash that keeps stale counter figures out of the bench line, the CPU
baseline's fields, and the profile summarizer on small synthetic rocprofv3
CSV files whose counters and durations are known."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
from workloads import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// a comment\n__global__ void k(float *x) { x[0] = 1.0f; }\n/* block\n comment */\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    h0 = bench.source_hash()
    src.write_text("// another comment\n__global__   void k(float *x)\n{ x[0] = 1.0f; }  // tail\n")
    assert bench.source_hash() == h0
    src.write_text("__global__ void k(float *x) { x[0] = 2.0f; }\n")
    assert bench.source_hash() != h0


def test_measured_traffic_needs_the_current_kernel_source(tmp_path, monkeypatch):
    rec = {"w": {"bytes_per_launch": 123, "source_sha256_16": "0123456789abcdef"}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    monkeypatch.setattr(bench, "source_hash", lambda: "0123456789abcdef")
    assert bench.measured_traffic("w") == 123
    assert bench.measured_traffic("other") is None
    monkeypatch.setattr(bench, "source_hash", lambda: "fedcba9876543210")
    assert bench.measured_traffic("w") is None


def test_committed_traffic_records_are_consistent():
    """Each committed counter record names the kernel source it was taken on
    and holds traffic close to the algorithmic bytes (scaled state reads its
    inputs twice); the bench line uses only those whose source is current."""
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert rec
    for name, r in rec.items():
        assert len(r["source_sha256_16"]) == 16
        assert r["bytes_per_launch"] == pytest.approx(r["ratio"] * r["algorithmic_bytes_per_launch"], rel=1e-4)
        assert 0.99 < r["ratio"] < (1.6 if "scaled" in name else 1.01)
        want = r["bytes_per_launch"] if r["source_sha256_16"] == bench.source_hash() else None
        assert bench.measured_traffic(name) == want


def test_cpu_baseline_reports_the_oracle_on_the_host():
    import oracle

    try:
        oracle.default()
    except Exception as e:  # the oracle library is built by __graft_entry__.build()
        pytest.skip(f"oracle library not built: {e}")
    r = bench.cpu_baseline(workloads()["tiny"], 5100, 3)  # whole tensors: all three
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert 1 <= r["cores"] <= 16
    assert "x 3 steps" in r["sample"] and "5,103 elements" in r["sample"]


def _write_csv(path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)


def test_profile_summary_from_synthetic_counters(tmp_path, monkeypatch):
    """tiny: 5,103 elements x 28 B.  The calibration kernel's counters read
    half (FETCH) and all (WRITE) of its known bytes, so the factors are 2 and
    1; the update's raw counters are set to the algorithmic bytes under those
    factors, so the summary must find traffic = algorithmic exactly."""
    w = workloads()["tiny"]
    n = sum(w.sizes)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "profiles" / "traffic.json"))
    (tmp_path / "profiles").mkdir()
    upd = "void (anonymous namespace)::adam_update<(anonymous namespace)::Config<1, 0, 0, 1, {}> >(...)"
    cal = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, X>>(...)"
    blocks = 10
    _write_csv(tmp_path / "trace" / "run_kernel_stats.csv",
               [dict(Name=upd.format("false"), Calls=4, AverageNs=1000, MinNs=900, MaxNs=1100),
                dict(Name=cal, Calls=1, AverageNs=500, MinNs=500, MaxNs=500)])
    trace = []
    for capt, dur in (("false", 1000), ("true", 1100)):
        for i in range(4):
            trace.append(dict(Kernel_Name=upd.format(capt), Start_Timestamp=10_000 * i,
                              End_Timestamp=10_000 * i + dur, Grid_Size_X=blocks * 128, Workgroup_Size_X=128))
    _write_csv(tmp_path / "trace" / "run_kernel_trace.csv", trace)
    known_kib = n * 4 / 1024
    read_kib, write_kib = n * 16 / 1024, n * 12 / 1024
    for which, upd_val, cal_val in (("fetch", read_kib / 2, known_kib / 2), ("write", write_kib, known_kib)):
        _write_csv(tmp_path / which / "run_counter_collection.csv",
                   [dict(Kernel_Name=upd.format("false"), Grid_Size=blocks * 128, Workgroup_Size=128,
                         Counter_Value=upd_val),
                    dict(Kernel_Name=cal, Grid_Size=4096, Workgroup_Size=256, Counter_Value=cal_val)])
    log = tmp_path / "trace.log"
    log.write_text("progress line\n" + json.dumps({
        "value": 1.0, "unit": "GB/s", "ms_per_step": 0.002,
        "roofline": {"launch_ms_mean": 0.001, "achieved": 1.0},
        "capturable": {"launch_ms_mean": 0.0011}}) + "\n")
    bench.summarize_profiles(w, str(tmp_path / "trace"), str(tmp_path / "fetch"), str(tmp_path / "write"),
                             str(log))
    trace_txt = (tmp_path / "profiles" / "adam_update_tiny_kernel_trace.txt").read_text()
    assert "update, regular" in trace_txt and "update, capturable" in trace_txt
    assert trace_txt.count("events / trace 1.0000") == 2
    pmc_txt = (tmp_path / "profiles" / "adam_update_tiny_pmc.txt").read_text()
    assert "FETCH factor 2.0000, WRITE factor 1.0000" in pmc_txt
    assert "measured / algorithmic = 1.0000" in pmc_txt
    rec = json.loads((tmp_path / "profiles" / "traffic.json").read_text())["tiny"]
    assert rec["bytes_per_launch"] == n * 28 and rec["ratio"] == 1.0
    assert rec["source_sha256_16"] == bench.source_hash()


def test_profile_summary_splits_the_two_buffer_launches(tmp_path, monkeypatch):
    """A run that also timed the two-buffer step ends with its launches (the
    bench line gives their number, warmup + steps): the summary reports them
    apart, with their own event / trace comparison and traffic."""
    w = workloads()["tiny"]
    n = sum(w.sizes)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "profiles" / "traffic.json"))
    (tmp_path / "profiles").mkdir()
    upd = "void (anonymous namespace)::adam_update<(anonymous namespace)::Config<1, 0, 0, 1, {}> >(...)"
    cal = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, X>>(...)"
    blocks = 10
    _write_csv(tmp_path / "trace" / "run_kernel_stats.csv",
               [dict(Name=upd.format("false"), Calls=7, AverageNs=900, MinNs=800, MaxNs=1000)])
    # 4 in-place launches of 1000 ns, 2 capturable ones, then 3 two-buffer launches of 800 ns
    trace = [dict(Kernel_Name=upd.format("false"), Start_Timestamp=10_000 * i, End_Timestamp=10_000 * i + 1000,
                  Grid_Size_X=blocks * 128, Workgroup_Size_X=128) for i in range(4)]
    trace += [dict(Kernel_Name=upd.format("true"), Start_Timestamp=50_000 + 10_000 * i,
                   End_Timestamp=50_000 + 10_000 * i + 1100, Grid_Size_X=blocks * 128, Workgroup_Size_X=128)
              for i in range(2)]
    trace += [dict(Kernel_Name=upd.format("false"), Start_Timestamp=90_000 + 10_000 * i,
                   End_Timestamp=90_000 + 10_000 * i + 800, Grid_Size_X=blocks * 128, Workgroup_Size_X=128)
              for i in range(3)]
    _write_csv(tmp_path / "trace" / "run_kernel_trace.csv", trace[::-1])  # any row order
    line = {"value": 1.0, "unit": "GB/s", "ms_per_step": 0.002, "warmup": 1, "steps": 2,
            "roofline": {"launch_ms_mean": 0.001, "achieved": 1.0}, "capturable": {"launch_ms_mean": 0.0011},
            "two_buffer_state": {"ms_per_step": 0.0009, "launch_ms_mean": 0.0008}}
    for name in ("trace", "fetch", "write"):
        (tmp_path / f"{name}.log").write_text(json.dumps(line) + "\n")
    known_kib = n * 4 / 1024
    read_kib, write_kib = n * 16 / 1024, n * 12 / 1024
    for which, upd_val, tb_val, cal_val in (("fetch", read_kib / 2, read_kib * 0.55, known_kib / 2),
                                            ("write", write_kib, write_kib, known_kib)):
        rows = [dict(Dispatch_Id=1, Kernel_Name=cal, Grid_Size=4096, Workgroup_Size=256, Counter_Value=cal_val)]
        rows += [dict(Dispatch_Id=2 + i, Kernel_Name=upd.format("false"), Grid_Size=blocks * 128,
                      Workgroup_Size=128, Counter_Value=upd_val) for i in range(4)]
        rows += [dict(Dispatch_Id=6 + i, Kernel_Name=upd.format("false"), Grid_Size=blocks * 128,
                      Workgroup_Size=128, Counter_Value=tb_val) for i in range(3)]
        _write_csv(tmp_path / which / "run_counter_collection.csv", rows[::-1])
    bench.summarize_profiles(w, str(tmp_path / "trace"), str(tmp_path / "fetch"), str(tmp_path / "write"),
                             str(tmp_path / "trace.log"), str(tmp_path / "fetch.log"), str(tmp_path / "write.log"))
    trace_txt = (tmp_path / "profiles" / "adam_update_tiny_kernel_trace.txt").read_text()
    assert "update, two-buffer state" in trace_txt
    assert trace_txt.count("events / trace 1.0000") == 3
    assert "false> [two-buffer]" in trace_txt
    pmc_txt = (tmp_path / "profiles" / "adam_update_tiny_pmc.txt").read_text()
    assert "measured / algorithmic = 1.0000" in pmc_txt
    assert "two-buffer state (the runs' last 3 update launches)" in pmc_txt
    rec = json.loads((tmp_path / "profiles" / "traffic.json").read_text())["tiny"]
    assert rec["ratio"] == 1.0
    assert rec["two_buffer_bytes_per_launch"] == round((read_kib * 0.55 * 2 + write_kib) * 1024)


def test_measured_traffic_of_the_two_buffer_step(tmp_path, monkeypatch):
    rec = {"w": {"bytes_per_launch": 123, "two_buffer_bytes_per_launch": 125,
                 "source_sha256_16": "0123456789abcdef"}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    monkeypatch.setattr(bench, "source_hash", lambda: "0123456789abcdef")
    assert bench.measured_traffic("w", "two_buffer_bytes_per_launch") == 125
    monkeypatch.setattr(bench, "source_hash", lambda: "fedcba9876543210")
    assert bench.measured_traffic("w", "two_buffer_bytes_per_launch") is None
