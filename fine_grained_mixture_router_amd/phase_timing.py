"""Where a many-rows GEMM tile spends its time: per-tile phase timestamps.

    python fine_grained_mixture_router_amd/build.py --phase      (on the build host)
    python fine_grained_mixture_router_amd/phase_timing.py       (on the GPU)

The measurement copy of the library (libmoe_phase.so, built with
-DMOE_PHASE_STAMPS) records, for each workgroup of the 256 x 256 GEMM tiles,
the shader clock (s_memtime) at the tile's start, once its first slice has
landed, after its main loop and after its epilogue's stores have been issued
(all taken by thread 0, i.e. wave 0).  This script runs the V3-shape prefill
layer through that copy (bf16, then 8-bit weights and activations on the FP8
tiles) and prints the median phases over each kind's workgroups (the bf16
kinds include the shared expert's tiles; the FP8 kinds are routed tiles
only), and the share of a tile's time that its MFMAs need: 2048 cycles per
slice for a SIMD's two waves (bf16: 4 k16 steps x 8 MFMAs x 32 cycles per
wave; FP8: 2 k64 steps x 8 MFMAs x 64 cycles per wave).
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

KINDS = ("bf16 gate/up", "bf16 down", "FP8 gate/up", "FP8 down")


def _swap_library(moe):
    """Point the binding at the measurement copy (same C ABI)."""
    path = os.path.join(HERE, "libmoe_phase.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: run build.py --phase first")
    csrc = os.path.join(HERE, "csrc")
    newest = max(os.path.getmtime(os.path.join(csrc, f)) for f in os.listdir(csrc))
    if newest > os.path.getmtime(path):
        raise SystemExit(f"{path} is older than the sources: run build.py --phase again")
    lib = ctypes.CDLL(path)
    for name in moe.EXPORTS:
        f0, f1 = getattr(moe._lib, name), getattr(lib, name)
        f1.restype, f1.argtypes = f0.restype, f0.argtypes
    moe._lib = lib
    return lib


def _read(lib):
    n = lib.moe_phase_slots()
    buf = (ctypes.c_ulonglong * n)()
    if lib.moe_phase_read(buf, n) != 0:
        raise SystemExit("reading the phase stamps failed")
    return np.frombuffer(buf, dtype=np.uint64).reshape(4, -1, 5).astype(np.int64)


def _summary(stamps, kind, slices):
    a = stamps[kind]
    a = a[(a[:, 0] > 0) & (a[:, 3] > a[:, 0])]
    pro, main, epi = a[:, 1] - a[:, 0], a[:, 2] - a[:, 1], a[:, 3] - a[:, 2]
    tot = a[:, 3] - a[:, 0]
    m = np.median
    return (f"| {KINDS[kind]} | {len(a)} | {m(pro):.0f} | {m(main):.0f} ({m(main) / slices:.0f} per slice) "
            f"| {m(epi):.0f} | {m(tot):.0f} | {slices * 2048 / m(tot):.0%} |")


def main():
    import torch

    import fine_grained_mixture_router_amd as moe
    from synth import workloads as wl

    lib = _swap_library(moe)
    w = wl.WORKLOADS["v3_prefill"]
    L = wl.gen_all(w)

    def dev(v):
        if v is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(v))
        return (t.view(torch.bfloat16) if v.dtype == np.uint16 else t).cuda()

    D = {k: dev(v) for k, v in L.items()}
    print("[phase] inputs on the device", flush=True)
    shape = moe.make_shape(w.T, w.d, w.E, w.I, w.K, w.Ks, w.Is)
    ws = torch.empty(moe.workspace_size(shape), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        moe.forward(D["x"], D["C"], D["w1"], D["w3"], D["w2"], D["ws1"], D["ws3"], D["ws2"], K=w.K,
                    bias=D["bias"], workspace=ws)
    torch.cuda.synchronize()
    bf = _read(lib)
    print("[phase] bf16 layer done", flush=True)
    del D["w1"], D["w3"], D["w2"], ws
    Q = dict(zip(("q1", "s1", "q3", "s3", "q2", "s2"), (dev(a) for a in wl.gen_routed_fp8(w))))
    shape8 = moe.make_shape(w.T, w.d, w.E, w.I, w.K, w.Ks, w.Is, act8=True)
    ws8 = torch.empty(moe.workspace_size(shape8), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        moe.forward_fp8(D["x"], D["C"], Q["q1"], Q["s1"], Q["q3"], Q["s3"], Q["q2"], Q["s2"],
                        D["ws1"], D["ws3"], D["ws2"], K=w.K, bias=D["bias"], act8=True, workspace=ws8)
    torch.cuda.synchronize()
    f8 = _read(lib)
    print("[phase] 8-bit layer done", flush=True)

    print(f"V3 prefill (T={w.T}, d={w.d}, I={w.I}); shader-clock cycles, medians over workgroups")
    print("| tile | workgroups | prologue | main loop | epilogue | total | MFMA-bound share |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    print(_summary(bf, 0, w.d // 64))
    print(_summary(bf, 1, w.I // 64))
    print(_summary(f8, 2, w.d // 128))
    print(_summary(f8, 3, w.I // 128))


if __name__ == "__main__":
    main()
