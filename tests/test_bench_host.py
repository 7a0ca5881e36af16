"""Host-side pieces of bench.py: the counter summary that feeds
roofline.traffic, and its invalidation when the kernel sources change."""
import csv
import io
import json
import os
import re
from contextlib import redirect_stdout

import pytest

import bench


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, v) in enumerate(rows):
            w.writerow([i, name, counter, v])


def test_summary_scales_by_the_calibration_copy(tmp_path):
    g1 = "void moe::(anonymous namespace)::gemm_big_kernel<true, 64, 2, 8>(moe::(anonymous namespace)::GemmParams)"
    cp = "__amd_rocclr_copyBuffer"
    # the copy reads 1 GiB but FETCH_SIZE shows half of it; a smaller copy is ignored
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(cp, 10.0), (g1, 1000.0), (g1, 3000.0),
                                                   (cp, 524288.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(cp, 1048576.0), (g1, 500.0), (g1, 500.0)])
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"))
    rec = json.loads(re.search(r"```json\n(.*?)\n```", buf.getvalue(), re.S).group(1))
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    k = rec["kernels"]["v3_prefill"]["gemm_gate_up"]
    assert k["dispatches"] == 2
    assert k["bytes"] == 2000 * 1024 * 2 + 500 * 1024
    assert rec["source_digest"] == bench.source_digest()


def test_recorded_traffic_requires_matching_sources(tmp_path, monkeypatch):
    rec = {"source_digest": bench.source_digest(),
           "kernels": {"v3_prefill": {"gemm_gate_up": {"bytes": 123.0}}}}
    p = tmp_path / "t.md"
    p.write_text("text\n```json\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.recorded_traffic("v3_prefill", "gemm_gate_up") == 123.0
    assert bench.recorded_traffic("v3_decode", "gemm_gate_up") is None
    rec["source_digest"] = "0" * 16
    p.write_text("```json\n" + json.dumps(rec) + "\n```\n")
    assert bench.recorded_traffic("v3_prefill", "gemm_gate_up") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic("v3_prefill", "gemm_gate_up") is None


def test_multi_gpu_request_exits(monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
