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
    g1 = "void moe::(anonymous namespace)::gemm_big_kernel<true, 8, false>(moe::(anonymous namespace)::GemmParams)"
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


def test_algorithmic_work_of_the_v3_batches():
    """The FLOPs and bytes the roofline lines divide by, from the layer's
    definition: gate/up does 4·d·I per routed or shared row (8.66 TFLOP at
    16 384 tokens, top-8 + 1 shared), the layer adds the down GEMM's 2·d·I
    per row and the router's 2·d·E per token; decode reads W1 and W3 of
    every touched expert and of the shared one."""
    import numpy as np
    from synth import workloads as wl
    w = wl.WORKLOADS["v3_prefill"]
    counts = np.zeros(w.E, dtype=np.int64)
    counts[:43] = 1                                    # 43 touched experts
    a = bench.algorithmic(w, counts)
    rows = w.T * (w.K + w.Ks)
    assert a["g1_flops"] == 4.0 * w.d * w.I * rows == 8658654068736.0
    assert a["layer_flops"] == 6.0 * w.d * w.I * rows + 2.0 * w.T * w.d * w.E
    assert a["touched"] == 43
    wd = wl.WORKLOADS["v3_decode"]
    cd = np.ones(wd.E, dtype=np.int64)
    ad = bench.algorithmic(wd, cd)
    w13 = (wd.E + wd.Ks) * 2 * wd.I * wd.d * 2         # bf16 W1 + W3, routed and shared
    assert ad["g1_bytes"] == w13 + 2 * wd.T * wd.d + 2 * wd.T * (wd.K + wd.Ks) * wd.I
    # 8-bit: one byte per routed weight plus a 4-byte scale per weight row
    a8 = bench.algorithmic_fp8(wd, cd)
    assert a8["g1_bytes"] == (wd.E * (2 * wd.I * wd.d + 4 * 2 * wd.I) + wd.Ks * 2 * 2 * wd.I * wd.d
                              + 2 * wd.T * wd.d + 2 * wd.T * (wd.K + wd.Ks) * wd.I)


def test_layer_roofline_time_of_one_expert():
    """An expert of n rows costs max(6·d·I·n / peak, bytes / bandwidth) in
    the layer roofline: a one-expert, one-token layer is bandwidth-bound by
    its 3·d·I bf16 weights."""
    import dataclasses

    import numpy as np
    from synth import workloads as wl
    base = wl.WORKLOADS["tiny"]
    w = dataclasses.replace(base, T=1, d=512, E=1, I=256, K=1, Ks=0, Is=256)
    t = bench.layer_roofline_ms(w, np.array([1]))
    bw = bench.PEAK_HBM_GBS * 1e9
    weights = 6.0 * w.d * w.I
    expect = (max(2.0 * w.d * w.E / (bench.PEAK_BF16_TFLOPS * 1e12), (2.0 * w.d + 2.0 * w.E * w.d) / bw)
              + (weights + 1 * (2.0 * w.d + 4.0 * w.I + 2.0 * w.d)) / bw
              + (2 + 1 + 0) * w.d * 2.0 / bw) * 1e3
    assert abs(t - expect) <= 1e-12 * expect


def test_backward_work_counts():
    """The backward's algorithmic FLOPs: per routed or shared row 12 d I
    (dH 2, dX 4, dW2 2, dW1+dW3 4), plus the router's 4 T E d; at the V3
    prefill shape that is 26.10 TFLOP, twice the forward layer."""
    import numpy as np

    from synth import workloads as wl
    w = wl.WORKLOADS["v3_prefill"]
    bw = bench.backward_work(w, np.zeros(w.E))
    rows = w.T * (w.K + w.Ks)
    assert bw["flops"]["bwd_dx"] == 4.0 * w.d * w.I * rows
    assert bw["total_flops"] == 12.0 * w.d * w.I * rows + 4.0 * w.T * w.E * w.d
    assert abs(bw["total_flops"] / 1e12 - 26.096) < 0.001
    assert bw["dw13_bytes"] == 2 * 2 * (w.E + w.Ks) * w.I * w.d + 2 * 2 * rows * w.I + 2 * rows * w.d


def test_tile_cover_hits_every_tile():
    import numpy as np

    from synth import workloads as wl
    w = wl.WORKLOADS["16b_zipf"]
    g = np.random.default_rng(0)
    idx = np.stack([g.choice(w.E, w.K, replace=False, p=None) for _ in range(w.T)]).astype(np.int32)
    tok = bench.tile_cover(idx, w)
    for e in range(w.E):
        rows = np.nonzero((idx == e).any(axis=1))[0]       # the group's rows, in token order
        for m0 in range(0, rows.size, 256):
            assert np.intersect1d(rows[m0:m0 + 256], tok).size > 0, (e, m0)
    for m0 in range(0, w.T, 256):                          # shared groups: every token in order
        assert np.any((tok >= m0) & (tok < m0 + 256))


def test_summary_keeps_instances_apart(tmp_path):
    """The training forward's gate/up instance (it also writes the
    pre-activations) does not land in the forward's slot, and the backward
    kinds map to their own slots."""
    ns = "void moe::(anonymous namespace)::"
    g1 = ns + "gemm_big_kernel<true, 8, false>(moe::(anonymous namespace)::GemmParams)"
    g1z = ns + "gemm_big_kernel<true, 8, true>(moe::(anonymous namespace)::GemmParams)"
    dw13 = ns + "bwd_gemm_kernel<4>(moe::(anonymous namespace)::BwdParams)"
    cp = "__amd_rocclr_copyBuffer"
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(cp, 524288.0), (g1, 100.0), (g1z, 900.0),
                                                   (dw13, 40.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(cp, 1048576.0), (g1, 10.0), (g1z, 90.0),
                                                   (dw13, 4.0)])
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"))
    rec = json.loads(re.search(r"```json\n(.*?)\n```", buf.getvalue(), re.S).group(1))
    assert rec["kernels"]["v3_prefill"]["gemm_gate_up"]["bytes"] == 100 * 1024 * 2 + 10 * 1024
    assert rec["kernels"]["v3_prefill_bwd"]["bwd_dw13"]["bytes"] == 40 * 1024 * 2 + 4 * 1024
    assert set(rec["kernels"]) == {"v3_prefill", "v3_prefill_bwd"}
