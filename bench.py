#!/usr/bin/env python3
"""Throughput of the DeepSeekMoE layer forward on one MI355X.

One step = one full pass of the layer (router, permutation, gate/up GEMM
with SwiGLU, down GEMM, combine) over one batch already resident in HBM.

Headline workload: the DeepSeek-V3-shape prefill batch (T=16384 tokens,
d=7168, 256 routed + 1 shared experts of inter 2048, top-8, Zipf(1.2) logit
bias) — MFMA-bound.  The same layer on a 256-token decode batch (HBM-bound)
is measured in the same run and reported under "decode", and both batches
again with 8-bit (E4M3, per-row scaled) routed weights under "prefill_fp8"
and "decode_fp8"; the smaller layer shapes (2B: 63 experts of 896, top-7;
16B: 64 experts of 1408, top-6, with and without a Zipf(1.1) bias, and the
tiny 16-expert layer) are summarised under "other_configs" with both roofline
fractions.  The training side (moe_forward_train + moe_backward: input,
weight, centroid and gate gradients for a seeded upstream gradient) is timed
on the prefill and decode batches under "backward", with the dominant
backward kernel against its roofline.  Inputs are
seeded synthetic data (bf16, N(0,1) activations, N(0,0.006) weights; the
8-bit codes are drawn as bit fields with per-row scales of a similar size).

Prints ONE JSON line:
  value            tokens/s of the whole layer (T / ms_per_step)
  roofline         the dominant kernel (gemm_gate_up): algorithmic FLOPs (or
                   bytes, decode) per launch / its mean duration from HIP
                   events recorded around it on its own stream during the
                   timed steps (only that kernel is recorded there), against
                   the MI355X peak; the other kernels' times (kernel_ms) come
                   from ten further steps recorded kernel by kernel
  cpu_baseline     the fp64 oracle on a bounded token sample of the same
                   batch, on the host cores (a reported baseline, not a target)
  hbm_read_ceiling the practical HBM read rate measured in the same run (a
                   plain streaming-read kernel), beside the nominal 8 TB/s
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/s; % of MFMA (prefill) / HBM (decode) roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "fine_grained_mixture_router_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_v3_prefill_decode.md")
CALIB_BYTES = 1 << 30         # the calibration copy: 1 GiB read + 1 GiB written
# kernel-name prefix -> (workload, slot) in a default run (prefill on the
# 256x256 tile, decode on the 32x256 tile, the 8-bit batches on the 8-bit
# instances of each)
COUNTER_KERNELS = {                 # kernel instance -> (workload, slot); names match whole
    "gemm_big_kernel<true, 8, false>": ("v3_prefill", "gemm_gate_up"),
    "gemm_big_kernel<false, 8, false>": ("v3_prefill", "gemm_down"),
    "grouped_gemm_kernel<32, 256, 1, 4, true, false>": ("v3_decode", "gemm_gate_up"),
    "grouped_gemm_kernel<32, 256, 1, 4, false, false>": ("v3_decode", "gemm_down"),
    "grouped_gemm_kernel<32, 256, 1, 4, true, true>": ("v3_decode_fp8", "gemm_gate_up"),
    "grouped_gemm_kernel<32, 256, 1, 4, false, true>": ("v3_decode_fp8", "gemm_down"),
    "gemm_big_q8_kernel<true, false>": ("v3_prefill_fp8", "gemm_gate_up"),
    "gemm_big_q8_kernel<false, false>": ("v3_prefill_fp8", "gemm_down"),
    "gemm_big_q8_kernel<true, true>": ("v3_prefill_fp8_act8", "gemm_gate_up"),
    "gemm_big_q8_kernel<false, true>": ("v3_prefill_fp8_act8", "gemm_down"),
    # the backward of the prefill batch (counter runs take it on that batch only)
    "bwd_gemm_kernel<0>": ("v3_prefill_bwd", "bwd_dh"),
    "bwd_gemm_kernel<1>": ("v3_prefill_bwd", "bwd_dx"),
    "bwd_gemm_kernel<2>": ("v3_prefill_bwd", "bwd_dx_router"),
    "bwd_gemm_kernel<3>": ("v3_prefill_bwd", "bwd_dw2"),
    "bwd_gemm_kernel<4>": ("v3_prefill_bwd", "bwd_dw13"),
    "bwd_gemm_kernel<5>": ("v3_prefill_bwd", "bwd_dc"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="v3_prefill")
    ap.add_argument("--decode", default="v3_decode",
                    help="second workload on the same layer weights ('' to skip)")
    ap.add_argument("--configs", default="tiny,2b,16b,16b_zipf",
                    help="smaller layer shapes summarised under other_configs ('' to skip)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the batches with 8-bit routed weights")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training-side (backward) measurements")
    ap.add_argument("--backward-on", default="prefill,decode",
                    help="batches whose training step is measured (the counter runs take "
                         "'prefill' alone, so that each backward kernel's counters are one size's)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the oracle CPU baseline (0 to skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with a 1 GiB device-to-device copy (the reference dispatch that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-kernels", metavar="TRACE_DIR",
                    help="print the per-kernel time table of a rocprofv3 --kernel-trace --stats "
                         "run and exit")
    return ap.parse_args()


DIGEST_SOURCES = ("common.h", "gemm.hip", "permute.hip", "backward.hip")   # the GEMMs, their tile order


def source_digest():
    """Digest of the code (comments and blank space removed) of the sources
    that decide the GEMMs' memory traffic: recorded counters describe these
    kernels only."""
    h = hashlib.sha256()
    for n in DIGEST_SOURCES:
        with open(os.path.join(CSRC, n)) as f:
            code = f.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(n.encode())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def _counter_means(run_dir, counter):
    """Mean value per dispatch of `counter`, per kernel name, from a rocprofv3
    counter_collection.csv under run_dir."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    vals = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return vals


def summarize_counters(fetch_dir, write_dir):
    """Traffic of the GEMM kernels from FETCH_SIZE and WRITE_SIZE runs (KiB
    per dispatch), scaled by what the same counters read for the 1 GiB
    calibration copy (the largest copy dispatch of each run)."""
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")

    def copy_max(vals):
        c = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs]
        if not c:
            raise SystemExit("no calibration copy dispatch found (run with --calibrate-copy)")
        return max(c)

    f_fetch = CALIB_BYTES / (copy_max(fetch) * 1024)
    f_write = CALIB_BYTES / (copy_max(write) * 1024)
    kern = {}
    for name in set(fetch) | set(write):
        short = re.sub(r"^void |\(.*$", "", name.replace("moe::(anonymous namespace)::", ""))
        if short not in COUNTER_KERNELS:
            continue
        wl_name, slot = COUNTER_KERNELS[short]
        fk = sum(fetch.get(name, [0])) / max(len(fetch.get(name, [])), 1)
        wk = sum(write.get(name, [0])) / max(len(write.get(name, [])), 1)
        kern.setdefault(wl_name, {})[slot] = dict(
            kernel=short, dispatches=len(fetch.get(name, [])), fetch_kib=round(fk, 1),
            write_kib=round(wk, 1), bytes=round(fk * 1024 * f_fetch + wk * 1024 * f_write))
    rec = dict(source_digest=source_digest(),
               calibration=dict(copy_bytes=CALIB_BYTES, fetch_scale=round(f_fetch, 4),
                                write_scale=round(f_write, 4)),
               kernels=kern)
    print("| workload | slot | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes |")
    print("|---|---|---|---:|---:|---:|---:|")
    for wl_name in sorted(kern):
        for slot, k in sorted(kern[wl_name].items()):
            print(f"| {wl_name} | {slot} | `{k['kernel']}` | {k['dispatches']} | {k['fetch_kib']:.0f} "
                  f"| {k['write_kib']:.0f} | {k['bytes'] / 1e9:.3f} GB |")
    print()
    print("```json")
    print(json.dumps(rec, indent=1))
    print("```")


def summarize_kernels(trace_dir):
    """Per-kernel time table (markdown) from the kernel_stats.csv of a
    rocprofv3 --kernel-trace --stats run."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows += list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("| kernel | calls | mean us | min us | max us | % of GPU time |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        name = re.sub(r"^void |\(.*$", "", r["Name"].replace("moe::(anonymous namespace)::", ""))
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
              f"{float(r['Percentage']):.2f} |")


def recorded_traffic(workload, slot):
    """Bytes per launch of `slot` on `workload` from the committed counter
    summary, or None when there is none or it was taken on other sources."""
    try:
        txt = open(TRAFFIC_FILE).read()
        rec = json.loads(re.search(r"```json\n(.*?)\n```", txt, re.S).group(1))
    except (OSError, AttributeError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    k = rec.get("kernels", {}).get(workload, {}).get(slot)
    return None if k is None else float(k["bytes"])


def hit_stats(idx, E):
    """Expert load of one batch: touched experts, max/mean rows, and the
    expert-hit entropy over ln(E) (the load diagnostic of the DeepSeek-V2
    explainer page, section 6)."""
    import numpy as np
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.float64)
    p = counts[counts > 0] / counts.sum()
    ent = float(-(p * np.log(p)).sum())
    return dict(touched=int((counts > 0).sum()), max_rows=int(counts.max()),
                min_rows=int(counts.min()), min_rows_touched=int(counts[counts > 0].min()),
                mean_rows=float(counts.mean()), entropy_over_lnE=ent / math.log(E) if E > 1 else 1.0,
                active_ratio=float((counts > 0).mean()))


def algorithmic_fp8(w, counts):
    """As algorithmic(), with the routed weights at one byte each plus one
    fp32 scale per weight row; shared experts stay bf16."""
    touched = int((counts > 0).sum())
    rows_r, rows_s = w.T * w.K, w.T * w.Ks
    g1_flops = 4.0 * w.d * (rows_r * w.I + rows_s * w.Is)
    g2_flops = 2.0 * w.d * (rows_r * w.I + rows_s * w.Is)
    layer_flops = 2.0 * w.T * w.d * w.E + g1_flops + g2_flops
    wb_r = 3 * w.I * w.d + 4 * (2 * w.I + w.d)
    wb_s = 2 * 3 * w.Is * w.d
    layer_bytes = (touched * wb_r + w.Ks * wb_s + 2 * w.E * w.d + 2 * 2 * w.T * w.d)
    g1_bytes = (touched * (2 * w.I * w.d + 4 * 2 * w.I) + w.Ks * 2 * 2 * w.Is * w.d
                + 2 * w.T * w.d + 2 * (rows_r * w.I + rows_s * w.Is))
    return dict(touched=touched, g1_flops=g1_flops, layer_flops=layer_flops,
                g1_bytes=float(g1_bytes), layer_bytes=float(layer_bytes))


def algorithmic(w, counts):
    """Algorithmic work of the layer and of its gate/up GEMM for one batch.

    Per row of a routed (shared) expert the gate/up GEMM does 4*d*I (4*d*Is)
    FLOPs; the down GEMM 2*d*I; the router 2*d*E per token.  Bytes: every
    touched expert's weights once (bf16), the shared weights, the centroids,
    x and out; the gate/up GEMM reads W1 and W3 of the touched experts and
    the shared ones, x once and writes H."""
    touched = int((counts > 0).sum())
    rows_r, rows_s = w.T * w.K, w.T * w.Ks
    g1_flops = 4.0 * w.d * (rows_r * w.I + rows_s * w.Is)
    g2_flops = 2.0 * w.d * (rows_r * w.I + rows_s * w.Is)
    layer_flops = 2.0 * w.T * w.d * w.E + g1_flops + g2_flops
    wb_r = 2 * 3 * w.I * w.d           # one routed expert's W1, W3, W2 in bytes
    wb_s = 2 * 3 * w.Is * w.d
    layer_bytes = (touched * wb_r + w.Ks * wb_s + 2 * w.E * w.d + 2 * 2 * w.T * w.d)
    g1_bytes = (touched * 2 * 2 * w.I * w.d + w.Ks * 2 * 2 * w.Is * w.d + 2 * w.T * w.d
                + 2 * (rows_r * w.I + rows_s * w.Is))
    return dict(touched=touched, g1_flops=g1_flops, layer_flops=layer_flops,
                g1_bytes=float(g1_bytes), layer_bytes=float(layer_bytes))


def dev(a):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def per_launch_ms(kernels):
    """{kernel: mean ms per launch} of the kernels that ran (a layer launches
    only the kernels its shape and flags need)."""
    return {k: round(ms / n, 4) for k, (ms, n) in kernels.items() if n > 0}


def time_workload(w, D, host_x, steps, warmup, act8=False):
    """Warm up, then time exactly `steps` forwards with HIP events around the
    whole region and around every kernel.  Returns timings and routing.
    act8: the 8-bit-weight forward with 8-bit activations (MOE_FLAG_ACT8)."""
    import torch

    import fine_grained_mixture_router_amd as moe
    x = dev(host_x)
    bias = None if D.get("bias") is None else D["bias"]
    shape = moe.make_shape(w.T, w.d, w.E, w.I, w.K, w.Ks, w.Is, act8=act8)
    ws = torch.empty(moe.workspace_size(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    gate = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")

    def step():
        if "q1" in D:
            moe.forward_fp8(x, D["C"], D["q1"], D["s1"], D["q3"], D["s3"], D["q2"], D["s2"],
                            D["ws1"], D["ws3"], D["ws2"], K=w.K, bias=bias, act8=act8, out=out,
                            topk_idx=idx, topk_gate=gate, workspace=ws)
        else:
            moe.forward(x, D["C"], D["w1"], D["w3"], D["w2"], D["ws1"], D["ws3"], D["ws2"],
                        K=w.K, bias=bias, out=out, topk_idx=idx, topk_gate=gate, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps record events around the gate/up GEMM only (each
    # recorded kernel adds two event records, a few microseconds each)
    moe.profile_begin(steps, kernels=["gemm_gate_up"])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    timed = moe.profile_end()
    # the per-kernel split from a few more steps, every kernel recorded
    split_steps = max(1, min(steps, 10))
    moe.profile_begin(split_steps)
    for _ in range(split_steps):
        step()
    torch.cuda.synchronize()
    kernels = moe.profile_end()
    kernels["gemm_gate_up"] = timed["gemm_gate_up"]
    return dict(ms_per_step=total_ms / steps, kernels=kernels, out=out, idx=idx.cpu().numpy(),
                gate=gate.cpu().numpy())


BWD_SLOTS = ("bwd_lists", "bwd_dh", "bwd_router", "bwd_dx_router", "bwd_dx", "bwd_dx_combine",
             "bwd_dw2", "bwd_dw13", "bwd_dc")


def backward_work(w, counts):
    """Algorithmic FLOPs (and, for the weight-gradient GEMMs, bytes) of one
    backward.  Per routed (shared) row: dH = dO W2 2·d·I, dX = [dA|dB]
    [W1;W3] 4·d·I, dW2 2·d·I, dW1+dW3 4·d·I; the router's dL·C and dL^T x
    2·T·E·d each.  dW13 bytes: the dW1 and dW3 of every expert written once
    (bf16) plus the rows of dZ and x it reads."""
    rows_i = w.T * w.K * w.I + w.T * w.Ks * w.Is
    f = dict(bwd_dh=2.0 * w.d * rows_i, bwd_dx=4.0 * w.d * rows_i, bwd_dw2=2.0 * w.d * rows_i,
             bwd_dw13=4.0 * w.d * rows_i, bwd_dx_router=2.0 * w.T * w.E * w.d,
             bwd_dc=2.0 * w.T * w.E * w.d)
    total = sum(f.values())
    dw13_bytes = (2 * 2 * (w.E * w.I + w.Ks * w.Is) * w.d            # dW1, dW3 written
                  + 2 * 2 * rows_i + 2 * w.T * (w.K + w.Ks) * w.d)     # dZ and x rows read
    return dict(flops=f, total_flops=total, dw13_bytes=float(dw13_bytes))


def time_backward(w, D, host_x, steps, warmup):
    """The training side on one batch: moe_forward_train, then `steps` timed
    moe_backward calls on its state (a seeded upstream gradient), each
    backward kernel recorded with HIP events on the call's stream in ten
    further calls."""
    import torch

    import fine_grained_mixture_router_amd as moe
    from synth import workloads as wl
    x = dev(host_x)
    dout = dev(wl.gen_dout(w, host_x.shape[0]))
    bias = D.get("bias")
    args = (x, D["C"], D["w1"], D["w3"], D["w2"], D["ws1"], D["ws3"], D["ws2"])
    shape = moe.make_shape(w.T, w.d, w.E, w.I, w.K, w.Ks, w.Is)
    state = torch.empty(moe.train_state_size(shape), dtype=torch.uint8, device="cuda")
    ws = torch.empty(moe.backward_workspace_size(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    outs = dict(dx=torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda"),
                dw1=torch.empty_like(D["w1"]), dw3=torch.empty_like(D["w3"]),
                dw2=torch.empty_like(D["w2"]), dws1=torch.empty_like(D["ws1"]),
                dws3=torch.empty_like(D["ws3"]), dws2=torch.empty_like(D["ws2"]),
                dC=torch.empty((w.E, w.d), dtype=torch.float32, device="cuda"))

    def fwd():
        return moe.forward_train(*args, K=w.K, bias=bias, out=out, state=state)[1]

    st = fwd()
    for _ in range(warmup):
        fwd()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fwd()
    e1.record()
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / steps

    def bwd():
        moe.backward(*args, dout=dout, state=st, workspace=ws, **outs)

    for _ in range(warmup):
        bwd()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        bwd()
    e1.record()
    torch.cuda.synchronize()
    bwd_ms = e0.elapsed_time(e1) / steps
    split = max(1, min(steps, 10))
    moe.profile_begin(split, kernels=list(BWD_SLOTS))
    for _ in range(split):
        bwd()
    torch.cuda.synchronize()
    kern = moe.profile_end()
    del state, ws, outs
    torch.cuda.empty_cache()
    return dict(fwd_train_ms=fwd_ms, bwd_ms=bwd_ms,
                kernel_ms={k: round(kern[k][0] / max(kern[k][1], 1), 4) for k in BWD_SLOTS
                           if kern[k][1] > 0})


def backward_line(w, r, counts):
    """The backward's summary for the JSON line: its own throughput and its
    dominant kernel against the roofline (MFMA for many rows per expert; the
    weight-gradient writes, HBM, for few)."""
    bw = backward_work(w, counts)
    km = r["kernel_ms"]
    dom = max((k for k in km if k in bw["flops"]), key=lambda k: km[k])
    t = km[dom] / 1e3
    if regime(w) == "mfma" or dom != "bwd_dw13":
        # traffic: HBM bytes per launch from the counter runs (taken on the
        # prefill batch's backward; none for other batches)
        tr = recorded_traffic(w.name + "_bwd", dom)
        ach = bw["flops"][dom] / t / 1e12
        roof = dict(kernel=dom, bound="mfma", achieved=round(ach, 1), peak=PEAK_BF16_TFLOPS,
                    unit="TFLOP/s", frac=round(ach / PEAK_BF16_TFLOPS, 4),
                    traffic=None if tr is None else round(tr),
                    algorithmic_flops=bw["flops"][dom], mean_launch_ms=km[dom])
        if dom == "bwd_dw13":
            roof["algorithmic_bytes"] = bw["dw13_bytes"]
    else:
        ach = bw["dw13_bytes"] / t / 1e9
        roof = dict(kernel=dom, bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS,
                    unit="GB/s", frac=round(ach / PEAK_HBM_GBS, 4), traffic=None,
                    algorithmic_bytes=bw["dw13_bytes"], mean_launch_ms=km[dom])
    tf = bw["total_flops"] / (r["bwd_ms"] / 1e3) / 1e12
    return {"workload": w.name, "T": w.T, "ms_per_backward": round(r["bwd_ms"], 4),
            "ms_per_forward_train": round(r["fwd_train_ms"], 4),
            "train_step_tokens_per_s": round(w.T / ((r["bwd_ms"] + r["fwd_train_ms"]) / 1e3), 1),
            "backward_tflops": round(tf, 1), "backward_mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "roofline": roof, "kernel_ms": km}


def layer_roofline_ms(w, counts):
    """Lower bound on the layer's time with every piece at the better of its
    two ceilings (2.5 PFLOP/s, 8 TB/s): the router, each routed or shared
    expert as max(FLOPs / peak, bytes / bandwidth) — an expert of n rows does
    6·d·I·n FLOPs and moves its 3·d·I bf16 weights plus n rows of x, H
    (written, then read) and Y — and the combine's (2 + K + Ks)·d bf16 per
    token.  Few-row experts are bandwidth-bound even in a prefill batch."""
    peak, bw = PEAK_BF16_TFLOPS * 1e12, PEAK_HBM_GBS * 1e9
    t = max(2.0 * w.T * w.d * w.E / peak, (2.0 * w.T * w.d + 2.0 * w.E * w.d) / bw)
    groups = [(int(n), w.I) for n in counts if n > 0] + [(w.T, w.Is)] * w.Ks
    for n, inter in groups:
        f = 6.0 * w.d * inter * n
        b = 6.0 * w.d * inter + n * (2.0 * w.d + 4.0 * inter + 2.0 * w.d)
        t += max(f / peak, b / bw)
    t += (2 + w.K + w.Ks) * w.T * w.d * 2.0 / bw
    return t * 1e3


def hbm_read_ceiling(nbytes=8 << 30, passes=5):
    """The device's practical HBM read rate: one pass of 16-byte loads over
    an nbytes buffer (the library's stream-read kernel), timed with events."""
    import torch

    import fine_grained_mixture_router_amd as moe
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    moe.stream_read(buf)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(passes):
        moe.stream_read(buf)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / passes
    del buf
    return dict(gbs=round(nbytes / (ms / 1e3) / 1e9, 1), bytes=nbytes, passes=passes,
                ms_per_pass=round(ms, 4))


def regime(w):
    """Few rows per expert (under 64 on average) stream each weight once and
    are HBM-bound; larger batches are MFMA-bound."""
    return "hbm" if w.T * w.K < 64 * w.E else "mfma"


def roofline(kind, work, kernels, workload):
    """The gate/up GEMM against its roofline.  `traffic` is the HBM bytes per
    launch from the committed counter summary (FETCH_SIZE + WRITE_SIZE,
    calibrated), null when that summary is of other kernel sources."""
    ms, n = kernels["gemm_gate_up"]
    avg_s = ms / max(n, 1) / 1e3
    traffic = recorded_traffic(workload, "gemm_gate_up")
    common = dict(traffic=traffic, algorithmic_bytes=work["g1_bytes"],
                  mean_launch_ms=round(ms / max(n, 1), 4), launches=n)
    if kind == "mfma":
        ach = work["g1_flops"] / avg_s / 1e12
        return dict(kernel="gemm_gate_up", bound="mfma", achieved=round(ach, 1),
                    peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(ach / PEAK_BF16_TFLOPS, 4),
                    **common)
    ach = work["g1_bytes"] / avg_s / 1e9
    return dict(kernel="gemm_gate_up", bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS,
                unit="GB/s", frac=round(ach / PEAK_HBM_GBS, 4), **common)


def tile_cover(idx, w, bm=256):
    """Tokens whose rows touch every (group, bm-row tile) of the GEMM work
    lists (the token on each tile's last row), in token order."""
    import numpy as np
    picks = set()
    for e in range(w.E):
        toks = np.nonzero((idx == e).any(axis=1))[0]
        for m0 in range(0, toks.size, bm):
            picks.add(int(toks[min(m0 + bm, toks.size) - 1]))
    if w.Ks:
        for m0 in range(0, w.T, bm):
            picks.add(min(m0 + bm, w.T) - 1)
    return np.array(sorted(picks), dtype=np.int64)


def routing_check(w, L, res):
    """Every token's routing against the oracle: index sets equal wherever
    the oracle's K-th vs (K+1)-th score margin exceeds 1e-5; the tokens
    under that margin are counted (exempt), not checked."""
    import numpy as np

    import oracle
    ri, _, rm = oracle.route(L["x"], L["C"], L["bias"], w.K)
    ok = rm > 1e-5
    gi = np.sort(res["idx"], axis=1)
    mism = int((np.sort(ri, axis=1) != gi)[ok].any(axis=1).sum())
    return dict(tokens=int(w.T), margin_exempt=int((~ok).sum()), set_mismatches=mism)


def cpu_baseline(w, L, res, seconds):
    """The fp64 oracle, as it stands, timed on the host cores for about
    `seconds` of wall clock on tokens that put a row in every work-list tile
    of the GEMMs (in token order; the whole set when the budget allows);
    also a spot parity check of the GPU output on those tokens."""
    import numpy as np

    import oracle
    import synth
    got_bits = res["out"].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    order = tile_cover(res["idx"], w)
    done = 0
    errs, mism = [], 0
    t0 = time.time()
    chunk = 16
    threads = 0
    ref_rows = []
    while done < order.size and (time.time() - t0) < seconds:
        tok = order[done:done + chunk]
        r = oracle.forward(L["x"][tok], L["C"], L["bias"], L["w1"], L["w3"], L["w2"], L["ws1"],
                           L["ws3"], L["ws2"], w.K)
        threads = r["threads"]
        ok = r["margin"] > 1e-5
        for j, t in enumerate(tok):
            if ok[j] and set(res["idx"][t].tolist()) != set(r["idx"][j].tolist()):
                mism += 1
        ref_rows.append((tok, r["out"]))
        done += len(tok)
    dt = time.time() - t0
    toks = np.concatenate([t for t, _ in ref_rows])
    ref = np.concatenate([o for _, o in ref_rows])
    got = synth.bf16_to_f64(got_bits[toks])
    rel = float(np.abs(got - ref).max() / np.sqrt(np.mean(ref ** 2)))
    return (dict(value=round(done / dt, 2), unit="tokens/s", cores=int(threads), kind="oracle",
                 sample=f"{done} of the {order.size} tokens of the {w.name} batch that put a row "
                        f"in every (group, 256-row tile) of the GEMM work lists, full layer in "
                        f"fp64 (routing + {w.K} routed + {w.Ks} shared SwiGLU experts per token), "
                        f"{dt:.1f} s"),
            dict(tokens=int(done), tiles_covered=bool(done == order.size),
                 max_err_over_rms=rel, routing_set_mismatches=int(mism)))


def main():
    args = parse()
    if args.summarize_kernels:
        summarize_kernels(args.summarize_kernels)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library runs the layer on a single MI355X and has "
              "no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fine_grained_mixture_router_amd as moe  # noqa: F401  (fails loudly if unbuilt)
    from synth import workloads as wl

    w = wl.WORKLOADS[args.workload]
    t_gen = time.time()
    L = wl.gen_all(w)
    D = {k: (None if v is None else dev(v)) for k, v in L.items() if k != "x"}
    gen_s = time.time() - t_gen
    print(f"[bench] inputs of {w.name} generated and uploaded in {gen_s:.1f} s", file=sys.stderr,
          flush=True)

    res = time_workload(w, D, L["x"], args.steps, args.warmup)
    counts = np.bincount(res["idx"].ravel(), minlength=w.E)
    work = algorithmic(w, counts)
    ms = res["ms_per_step"]
    line = {
        "metric": METRIC,
        "value": round(w.T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; bf16 N(0,1) activations, N(0,0.006) weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "I": w.I, "K": w.K,
                   "Ks": w.Ks, "Is": w.Is, "zipf_s": w.zipf_s, "parallelism": "single GPU"},
        "roofline": roofline(regime(w), work, res["kernels"], w.name),
        "layer": {"tflops": round(work["layer_flops"] / (ms / 1e3) / 1e12, 1),
                  "mfma_frac": round(work["layer_flops"] / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "kernel_ms": per_launch_ms(res["kernels"]),
                  "roofline_ms": round(layer_roofline_ms(w, counts), 4),
                  "frac_of_roofline": round(layer_roofline_ms(w, counts) / ms, 4),
                  "load": hit_stats(res["idx"], w.E)},
    }
    print(f"[bench] {w.name}: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    Q8 = None
    if not args.no_fp8:
        # the same prefill batch with 8-bit routed weights (shared experts bf16)
        Q8 = dict(zip(("q1", "s1", "q3", "s3", "q2", "s2"),
                      (dev(a) for a in wl.gen_routed_fp8(w))))
        P8 = {k: v for k, v in D.items() if k not in ("w1", "w3", "w2")}
        P8.update(Q8)
        rp = time_workload(w, P8, L["x"], args.steps, args.warmup)
        cp = np.bincount(rp["idx"].ravel(), minlength=w.E)
        kp = algorithmic_fp8(w, cp)
        msp = rp["ms_per_step"]
        line["prefill_fp8"] = {
            "workload": w.name + " (8-bit E4M3 routed weights, per-row fp32 scales; shared bf16)",
            "T": w.T, "value": round(w.T / (msp / 1e3), 1), "unit": "tokens/s",
            "ms_per_step": round(msp, 4), "speedup_vs_bf16": round(ms / msp, 3),
            "mfma_dtype": "bf16 (codes widened exactly before the products)",
            "note": "with bf16 activations the 8-bit weights only halve the bytes each tile "
                    "moves, and the products still run on the bf16 MFMA; prefill_fp8_act8 adds "
                    "8-bit activations and runs the routed gate/up on the FP8 MFMA",
            "roofline": roofline("mfma", kp, rp["kernels"], w.name + "_fp8"),
            "kernel_ms": per_launch_ms(rp["kernels"]),
        }
        # the same with 8-bit activations (MOE_FLAG_ACT8): the routed gate/up
        # and down products on the FP8 MFMA (32x32x64, E4M3 x E4M3), the
        # shared expert bf16
        ra = time_workload(w, P8, L["x"], args.steps, args.warmup, act8=True)
        msa = ra["ms_per_step"]
        g1r = 4.0 * w.d * w.I * w.T * w.K                 # routed gate/up FLOPs (FP8)
        g1s = 4.0 * w.d * w.Is * w.T * w.Ks               # shared gate/up FLOPs (bf16)
        mixed_peak = (g1r + g1s) / (g1r / (2 * PEAK_BF16_TFLOPS) + g1s / PEAK_BF16_TFLOPS)
        ga_ms, ga_n = ra["kernels"]["gemm_gate_up"]
        ga_s = ga_ms / max(ga_n, 1) / 1e3
        ach = (g1r + g1s) / ga_s / 1e12
        tr = recorded_traffic(w.name + "_fp8_act8", "gemm_gate_up")
        line["prefill_fp8_act8"] = {
            "workload": w.name + " (8-bit E4M3 routed weights and activations: per-row "
                                 "power-of-two activation scales for x and h; shared expert bf16)",
            "T": w.T, "value": round(w.T / (msa / 1e3), 1), "unit": "tokens/s",
            "ms_per_step": round(msa, 4), "speedup_vs_bf16": round(ms / msa, 3),
            "mfma_dtype": "fp8 (routed gate/up and down, v_mfma_f32_32x32x64_f8f6f4); bf16 for "
                          "the shared expert",
            "roofline": dict(kernel="gemm_gate_up", bound="mfma", achieved=round(ach, 1),
                             peak=round(mixed_peak, 1), unit="TFLOP/s",
                             frac=round(ach / mixed_peak, 4),
                             traffic=None if tr is None else round(tr),
                             peak_note="routed FLOPs at the 5.0 PF FP8 peak, the shared expert's "
                                       "at the 2.5 PF bf16 peak; the quantisation of x is its "
                                       "own kernel (act8_x in kernel_ms)",
                             mean_launch_ms=round(ga_s * 1e3, 4), launches=ga_n),
            "kernel_ms": per_launch_ms(ra["kernels"]),
        }
        del P8
        print(f"[bench] {w.name} fp8: {msp:.3f} ms/step, with 8-bit activations {msa:.3f} ms/step",
              file=sys.stderr, flush=True)

    if args.decode:
        wd = wl.WORKLOADS[args.decode]
        assert (wd.d, wd.E, wd.I, wd.Ks, wd.Is, wd.wseed) == (w.d, w.E, w.I, w.Ks, w.Is, w.wseed)
        xd = wl.gen_x(wd)
        Dd = dict(D, bias=None if wd.zipf_s == 0 else dev(wl.gen_bias(wd)))
        rd = time_workload(wd, Dd, xd, args.steps, args.warmup)
        cd = np.bincount(rd["idx"].ravel(), minlength=wd.E)
        wk = algorithmic(wd, cd)
        msd = rd["ms_per_step"]
        line["decode"] = {
            "workload": wd.name, "T": wd.T, "value": round(wd.T / (msd / 1e3), 1),
            "unit": "tokens/s", "ms_per_step": round(msd, 4),
            "roofline": roofline(regime(wd), wk, rd["kernels"], wd.name),
            "layer_gbs": round(wk["layer_bytes"] / (msd / 1e3) / 1e9, 1),
            "layer_hbm_frac": round(wk["layer_bytes"] / (msd / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernel_ms": per_launch_ms(rd["kernels"]),
            "roofline_ms": round(layer_roofline_ms(wd, cd), 4),
            "frac_of_roofline": round(layer_roofline_ms(wd, cd) / msd, 4),
            "load": hit_stats(rd["idx"], wd.E),
        }
        print(f"[bench] {wd.name}: {msd:.3f} ms/step", file=sys.stderr, flush=True)

        if not args.no_fp8:
            # the same decode batch with 8-bit routed weights (shared experts bf16)
            if Q8 is None:   # the decode batch shares the prefill batch's weights
                Q8 = dict(zip(("q1", "s1", "q3", "s3", "q2", "s2"),
                              (dev(a) for a in wl.gen_routed_fp8(wd))))
            D8 = {k: v for k, v in Dd.items() if k not in ("w1", "w3", "w2")}
            D8.update(Q8)
            r8 = time_workload(wd, D8, xd, args.steps, args.warmup)
            c8 = np.bincount(r8["idx"].ravel(), minlength=wd.E)
            k8 = algorithmic_fp8(wd, c8)
            ms8 = r8["ms_per_step"]
            line["decode_fp8"] = {
                "workload": wd.name + " (8-bit E4M3 routed weights, per-row fp32 scales; shared bf16)",
                "T": wd.T, "value": round(wd.T / (ms8 / 1e3), 1), "unit": "tokens/s",
                "ms_per_step": round(ms8, 4), "speedup_vs_bf16": round(msd / ms8, 3),
                "roofline": roofline(regime(wd), k8, r8["kernels"], wd.name + "_fp8"),
                "layer_gbs": round(k8["layer_bytes"] / (ms8 / 1e3) / 1e9, 1),
                "layer_hbm_frac": round(k8["layer_bytes"] / (ms8 / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                "kernel_ms": per_launch_ms(r8["kernels"]),
            }
            del D8
            torch.cuda.empty_cache()
            print(f"[bench] {wd.name} fp8: {ms8:.3f} ms/step", file=sys.stderr, flush=True)

    if not args.no_backward:
        # the training side on the same batches: forward_train, then backward
        bl = {}
        rb = time_backward(w, D, L["x"], args.steps, args.warmup)
        bl["prefill"] = backward_line(w, rb, counts)
        print(f"[bench] {w.name} backward: {rb['bwd_ms']:.3f} ms", file=sys.stderr, flush=True)
        if args.decode and "decode" in args.backward_on.split(","):
            rbd = time_backward(wd, Dd, xd, args.steps, args.warmup)
            bl["decode"] = backward_line(wd, rbd, cd)
            print(f"[bench] {wd.name} backward: {rbd['bwd_ms']:.3f} ms", file=sys.stderr,
                  flush=True)
        line["backward"] = bl

    if args.configs:
        # the smaller shapes: layer TFLOP/s against the MFMA peak and
        # algorithmic bytes/s against the HBM peak, both reported
        others = {}
        for name in [c for c in args.configs.split(",") if c]:
            wc = wl.WORKLOADS[name]
            Lc = wl.gen_all(wc)
            Dc = {k: (None if v is None else dev(v)) for k, v in Lc.items() if k != "x"}
            rc = time_workload(wc, Dc, Lc["x"], args.steps, args.warmup)
            cc = np.bincount(rc["idx"].ravel(), minlength=wc.E)
            kc = algorithmic(wc, cc)
            msc = rc["ms_per_step"]
            tf = kc["layer_flops"] / (msc / 1e3) / 1e12
            gbs = kc["layer_bytes"] / (msc / 1e3) / 1e9
            others[name] = {
                "T": wc.T, "d": wc.d, "E": wc.E, "I": wc.I, "K": wc.K, "Ks": wc.Ks,
                "zipf_s": wc.zipf_s, "ms_per_step": round(msc, 4),
                "tokens_per_s": round(wc.T / (msc / 1e3), 1),
                "tflops": round(tf, 1), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "roofline_ms": round(layer_roofline_ms(wc, cc), 4),
                "frac_of_roofline": round(layer_roofline_ms(wc, cc) / msc, 4),
                "kernel_ms": per_launch_ms(rc["kernels"]),
            }
            del Dc, Lc
            torch.cuda.empty_cache()
            print(f"[bench] {name}: {msc:.3f} ms/step", file=sys.stderr, flush=True)
        line["other_configs"] = others

    ceil = hbm_read_ceiling()
    line["hbm_read_ceiling"] = ceil
    for key in ("decode", "decode_fp8"):
        if key in line:
            r = line[key]["roofline"]
            r["frac_of_read_ceiling"] = round(r["achieved"] / ceil["gbs"], 4)
            line[key]["layer_frac_of_read_ceiling"] = round(line[key]["layer_gbs"] / ceil["gbs"], 4)
    print(f"[bench] HBM read ceiling {ceil['gbs']:.0f} GB/s", file=sys.stderr, flush=True)

    if args.cpu_seconds > 0:
        base, spot = cpu_baseline(w, L, res, args.cpu_seconds)
        line["cpu_baseline"] = base
        spot["routing_all_tokens"] = routing_check(w, L, res)
        line["spot_parity"] = spot
    else:
        line["cpu_baseline"] = None
    if args.calibrate_copy:
        src = torch.ones(CALIB_BYTES // 2, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
