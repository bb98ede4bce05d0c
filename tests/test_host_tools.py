"""Host-side measurement tools (CPU): the kernel-trace and counter summaries the committed
profiles are made with, bench.py's gate on counter figures taken on an older kernel source,
and its refusal of more than one GPU."""

import csv
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from displaced_patch_parallelism_amd.diag import trace_summary, traffic  # noqa: E402


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _trace_rows():
    # (start ns, kernel, duration us); written out of order to check the time ordering
    spec = [(3000, "void dp::(anonymous namespace)::foo_kernel<1>(dp::Args)", 30.0),
            (1000, "void dp::(anonymous namespace)::foo_kernel<1>(dp::Args)", 10.0),
            (500, "bar", 5.0),
            (2000, "void dp::(anonymous namespace)::foo_kernel<1>(dp::Args)", 20.0)]
    return [{"Kernel_Name": k, "Start_Timestamp": s, "End_Timestamp": s + int(d * 1000)} for s, k, d in spec]


def test_trace_durations_and_table(tmp_path):
    path = tmp_path / "run_kernel_trace.csv"
    _write_csv(path, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], _trace_rows())
    durs = trace_summary.kernel_durations(str(path))
    foo = "void dp::(anonymous namespace)::foo_kernel<1>(dp::Args)"
    assert durs[foo] == [10.0, 20.0, 30.0]          # dispatch order, whatever the file order
    assert durs["bar"] == [5.0]
    assert trace_summary.short_name(foo) == "foo_kernel<1>"

    lines = trace_summary.table(str(path)).splitlines()
    assert lines[0].startswith("| kernel | dispatches | median us")
    # largest total first: foo 60 us of 65
    assert lines[2] == "| `foo_kernel<1>` | 3 | 20.000 | 20.000 | 10.000 | 30.000 | 92.3 |"
    assert lines[3] == "| `bar` | 1 | 5.000 | 5.000 | 5.000 | 5.000 | 7.7 |"
    # a directory holding the trace reads the same
    assert trace_summary.table(str(tmp_path)) == "\n".join(lines)
    # --skip drops each kernel's first dispatches (and kernels with no more than that)
    skipped = trace_summary.table(str(path), skip=1).splitlines()
    assert skipped[2] == "| `foo_kernel<1>` | 2 | 25.000 | 25.000 | 20.000 | 30.000 | 100.0 |"
    assert len(skipped) == 3


def _counter_dir(tmp_path, name, rows):
    d = tmp_path / name
    d.mkdir()
    _write_csv(d / "run_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
               rows)
    return str(d)


def test_traffic_summarize_scales_by_the_copy(tmp_path):
    k = "conv_kernel(args)"
    # two dispatches, each reported in two rows (summed per dispatch); another kernel is ignored
    fetch = _counter_dir(tmp_path, "f", [
        {"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": 100},
        {"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": 50},
        {"Dispatch_Id": 2, "Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": 250},
        {"Dispatch_Id": 3, "Kernel_Name": "other", "Counter_Name": "FETCH_SIZE", "Counter_Value": 9999}])
    write = _counter_dir(tmp_path, "w", [
        {"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": "WRITE_SIZE", "Counter_Value": 300},
        {"Dispatch_Id": 2, "Kernel_Name": k, "Counter_Name": "WRITE_SIZE", "Counter_Value": 300}])
    # the 64 MiB calibration copy: FETCH_SIZE counts half of the bytes, WRITE_SIZE all of them
    cfetch = _counter_dir(tmp_path, "cf", [
        {"Dispatch_Id": i, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 32768} for i in range(3)])
    cwrite = _counter_dir(tmp_path, "cw", [
        {"Dispatch_Id": i, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
         "Counter_Value": 65536} for i in range(3)])
    out = traffic.summarize("conv_kernel", fetch, write, cfetch, cwrite, 64)
    assert out["fetch_kib_per_dispatch"] == 200.0 and out["fetch_dispatches"] == 2
    assert out["write_kib_per_dispatch"] == 300.0 and out["write_dispatches"] == 2
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    assert out["hbm_bytes_per_launch"] == (200 * 2 + 300) * 1024
    with pytest.raises(SystemExit):
        traffic.per_dispatch(fetch, "missing_kernel", "FETCH_SIZE")


def _load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_reports_traffic_only_for_the_counted_source(tmp_path, monkeypatch):
    bench = _load_bench()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "displaced_patch_parallelism_amd" / "csrc" / "k_conv.hip"
    src.parent.mkdir(parents=True)
    src.write_bytes(b"// kernel source as counted\n")
    (tmp_path / "profiles").mkdir()
    assert bench.traffic_for("conv", "c1") is None                      # no table
    table = {"conv/c1": {"hbm_bytes_per_launch": 123456,
                         "source_sha256_16": hashlib.sha256(src.read_bytes()).hexdigest()[:16]}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(table))
    assert bench.traffic_for("conv", "c1") == 123456
    assert bench.traffic_for("conv", "c4a") is None                     # not counted
    src.write_bytes(b"// kernel source changed since\n")
    assert bench.traffic_for("conv", "c1") is None                      # stale counts


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr and r.stdout == ""
