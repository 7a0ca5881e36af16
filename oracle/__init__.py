"""fp64 CPU oracle of the DeepSeekMoE layer forward.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The layer's own code never
imports it, and it shares no code with the HIP library.

oracle.c holds the definition (routing, SwiGLU experts, shared experts,
residual) in plain double-precision loops; ref_np.py is a second,
independent numpy float64 formulation used to cross-check it on small
shapes; cost.py holds the parameter/MAC accounting of one expert and the
expert-hit entropy diagnostic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

NO_RESIDUAL = 1
RENORM = 2      # gates divided by their sum over the K selected experts
SIGMOID = 4     # sigmoid affinities; the bias enters the selection only
ACT8 = 8        # routed products take 8-bit activations (per-row power-of-two scales)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("I", ctypes.c_int32), ("K", ctypes.c_int32), ("Ks", ctypes.c_int32),
                ("Is", ctypes.c_int32), ("flags", ctypes.c_uint32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.oracle_route.restype = i32
        L.oracle_route.argtypes = [ctypes.POINTER(_Shape), vp, i32, vp, vp, vp, vp, vp, vp, i32]
        L.oracle_forward.restype = i32
        L.oracle_forward.argtypes = [ctypes.POINTER(_Shape), vp, i32, vp, vp,
                                     vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, vp, vp, vp, vp, i32]
        L.oracle_forward_fp8.restype = i32
        L.oracle_forward_fp8.argtypes = [ctypes.POINTER(_Shape), vp, i32, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, i32]
        L.oracle_backward.restype = i32
        L.oracle_backward.argtypes = [ctypes.POINTER(_Shape), vp, i32, vp, vp,
                                      vp, vp, vp, vp, vp, vp,
                                      vp, ctypes.c_double, vp,
                                      vp, i32, vp, i32, i32, i32,
                                      vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, i32]
        L.oracle_e4m3.restype = ctypes.c_double
        L.oracle_e4m3.argtypes = [ctypes.c_uint8]
        L.oracle_act8_exponent.restype = i32
        L.oracle_act8_exponent.argtypes = [ctypes.c_double]
        L.oracle_e4m3_nearest.restype = ctypes.c_uint8
        L.oracle_e4m3_nearest.argtypes = [ctypes.c_double]
        L.oracle_bf16_nearest.restype = ctypes.c_uint16
        L.oracle_bf16_nearest.argtypes = [ctypes.c_double]
        L.oracle_quantize_act8.restype = None
        L.oracle_quantize_act8.argtypes = [vp, i32, i32, vp, vp]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a, shape):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    assert a.shape == tuple(shape), (a.shape, shape)
    return a


def _ptr_table(stack, n, shape, dtype=np.uint16):
    """Per-expert pointer table from a [n, ...] stack or a list of n arrays."""
    keep = []
    tbl = (ctypes.c_void_p * max(n, 1))()
    for i in range(n):
        a = np.ascontiguousarray(stack[i])
        assert a.dtype == dtype, a.dtype
        assert a.shape == tuple(shape), (a.shape, shape)
        keep.append(a)
        tbl[i] = a.ctypes.data
    return tbl, keep


def e4m3(code: int) -> float:
    """Value of an OCP FP8 E4M3 code (NaN for 0x7F / 0xFF)."""
    return float(lib().oracle_e4m3(int(code)))


def act8_exponent(amax: float) -> int:
    """Scale exponent of a row of 8-bit activations: the smallest integer e
    with amax <= 448 * 2^e (0 for amax = 0)."""
    return int(lib().oracle_act8_exponent(float(amax)))


def e4m3_nearest(y: float) -> int:
    """E4M3 code nearest to y (|y| <= 448), ties to the even code."""
    return int(lib().oracle_e4m3_nearest(float(y)))


def bf16_nearest(v: float) -> int:
    """Bits of the bf16 value nearest to v, ties to the even significand."""
    return int(lib().oracle_bf16_nearest(float(v)))


def quantize_act8(x_rows):
    """8-bit activations of bf16 rows (uint16 bits [n, d]): (codes uint8
    [n, d], scale exponents int32 [n]); row t's values are e4m3(codes) *
    2^exps[t]."""
    x_rows = np.ascontiguousarray(x_rows, dtype=np.uint16)
    n, d = x_rows.shape
    codes = np.zeros((n, d), np.uint8)
    exps = np.zeros(n, np.int32)
    lib().oracle_quantize_act8(_ptr(x_rows), n, d, _ptr(codes), _ptr(exps))
    return codes, exps


def _gating(renorm, sigmoid):
    return (RENORM if renorm else 0) | (SIGMOID if sigmoid else 0)


def route(x_rows, C, bias, K, nthreads=0, return_probs=False, renorm=False, sigmoid=False):
    """Routing (affinity, score, top-K) of the given token rows.

    x_rows: uint16 bf16 bits [n, d]; C: [E, d]; bias: float32 [E] or None.
    renorm / sigmoid select the gating variant (see oracle.c, steps 2-3).
    Returns idx int32 [n, K], gate float64 [n, K], margin float64 [n]
    (and the scores [n, E] when asked)."""
    x_rows = np.ascontiguousarray(x_rows)
    n, d = x_rows.shape
    E = C.shape[0]
    C = _u16(C, (E, d))
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    sh = _Shape(n, d, E, 0, K, 0, 0, _gating(renorm, sigmoid))
    idx = np.zeros((n, K), np.int32)
    gate = np.zeros((n, K), np.float64)
    margin = np.zeros(n, np.float64)
    probs = np.zeros((n, E), np.float64) if return_probs else None
    lib().oracle_route(ctypes.byref(sh), _ptr(x_rows), n, _ptr(C), _ptr(b), _ptr(idx),
                       _ptr(gate), _ptr(margin), _ptr(probs), int(nthreads))
    return (idx, gate, margin, probs) if return_probs else (idx, gate, margin)


def forward(x_rows, C, bias, w1, w3, w2, ws1, ws3, ws2, K, no_residual=False,
            forced_idx=None, nthreads=0, renorm=False, sigmoid=False):
    """Layer forward of the given token rows, in fp64.

    x_rows: [n, d] bf16 bits.  w1/w3: per routed expert [I, d] (a [E, I, d]
    stack or a list, entries may be None for experts never selected when
    forced_idx names the experts); w2: [d, I] each.  ws*: likewise for the
    K_s shared experts.  Returns a dict with out, shared, routed ([n, d]
    float64), idx, gate, margin and the thread count used."""
    x_rows = np.ascontiguousarray(x_rows)
    n, d = x_rows.shape
    E = C.shape[0]
    C = _u16(C, (E, d))
    Ks = 0 if ws1 is None else len(ws1)
    I = next(a.shape[0] for a in w1 if a is not None) if E else 0
    Is = ws1[0].shape[0] if Ks else 0
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)

    keep = []
    tw = []
    zero_i = np.zeros((I, d), np.uint16)
    zero_o = np.zeros((d, I), np.uint16)
    for stack, shp, z in ((w1, (I, d), zero_i), (w3, (I, d), zero_i), (w2, (d, I), zero_o)):
        lst = [z if stack[e] is None else stack[e] for e in range(E)]
        t, k = _ptr_table(lst, E, shp)
        tw.append(t)
        keep.append(k)
    ts = []
    for stack, shp in ((ws1, (Is, d)), (ws3, (Is, d)), (ws2, (d, Is))):
        t, k = _ptr_table(stack if Ks else [], Ks, shp)
        ts.append(t)
        keep.append(k)

    fi = None
    if forced_idx is not None:
        fi = np.ascontiguousarray(forced_idx, dtype=np.int32)
        assert fi.shape == (n, K)
        assert fi.size == 0 or (fi.min() >= 0 and fi.max() < E)

    sh = _Shape(n, d, E, I, K, Ks, Is,
                (NO_RESIDUAL if no_residual else 0) | _gating(renorm, sigmoid))
    out = np.zeros((n, d), np.float64)
    shared = np.zeros((n, d), np.float64)
    routed = np.zeros((n, d), np.float64)
    idx = np.zeros((n, K), np.int32)
    gate = np.zeros((n, K), np.float64)
    margin = np.zeros(n, np.float64)
    used = lib().oracle_forward(ctypes.byref(sh), _ptr(x_rows), n, _ptr(C), _ptr(b),
                                tw[0], tw[1], tw[2], ts[0], ts[1], ts[2], _ptr(fi),
                                _ptr(out), _ptr(shared), _ptr(routed), _ptr(idx), _ptr(gate),
                                _ptr(margin), int(nthreads))
    return dict(out=out, shared=shared, routed=routed, idx=idx, gate=gate, margin=margin,
                threads=int(used))


def forward_fp8(x_rows, C, bias, q1, s1, q3, s3, q2, s2, ws1, ws3, ws2, K, no_residual=False,
                forced_idx=None, nthreads=0, renorm=False, sigmoid=False, act8=False):
    """Layer forward with 8-bit routed weights, in fp64: q1/q3 uint8 [E, I, d]
    and q2 [E, d, I] E4M3 codes, s1/s3 float32 [E, I] and s2 [E, d] per-row
    scales (weight = e4m3(q) * scale); shared experts ws* in bf16 as for
    forward().  act8: the routed experts' products take 8-bit activations —
    x quantised per token, h = silu(W1 x) * W3 x rounded to bf16 and
    quantised per (token, expert) row (quantize_act8's rule) before W2.
    Returns the same dict as forward()."""
    x_rows = np.ascontiguousarray(x_rows)
    n, d = x_rows.shape
    E = C.shape[0]
    C = _u16(C, (E, d))
    I = q1.shape[1]
    Ks = 0 if ws1 is None else len(ws1)
    Is = ws1[0].shape[0] if Ks else 0
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    keep = []
    tq, ts_ = [], []
    for q, sc, shp in ((q1, s1, (I, d)), (q3, s3, (I, d)), (q2, s2, (d, I))):
        t, k = _ptr_table(q, E, shp, np.uint8)
        tq.append(t)
        keep.append(k)
        t, k = _ptr_table(np.ascontiguousarray(sc, dtype=np.float32), E, (shp[0],), np.float32)
        ts_.append(t)
        keep.append(k)
    tsh = []
    for stack, shp in ((ws1, (Is, d)), (ws3, (Is, d)), (ws2, (d, Is))):
        t, k = _ptr_table(stack if Ks else [], Ks, shp)
        tsh.append(t)
        keep.append(k)
    fi = None
    if forced_idx is not None:
        fi = np.ascontiguousarray(forced_idx, dtype=np.int32)
        assert fi.shape == (n, K)
    sh = _Shape(n, d, E, I, K, Ks, Is,
                (NO_RESIDUAL if no_residual else 0) | _gating(renorm, sigmoid) | (ACT8 if act8 else 0))
    out = np.zeros((n, d), np.float64)
    shared = np.zeros((n, d), np.float64)
    routed = np.zeros((n, d), np.float64)
    idx = np.zeros((n, K), np.int32)
    gate = np.zeros((n, K), np.float64)
    margin = np.zeros(n, np.float64)
    used = lib().oracle_forward_fp8(ctypes.byref(sh), _ptr(x_rows), n, _ptr(C), _ptr(b),
                                    tq[0], ts_[0], tq[1], ts_[1], tq[2], ts_[2],
                                    tsh[0], tsh[1], tsh[2], _ptr(fi),
                                    _ptr(out), _ptr(shared), _ptr(routed), _ptr(idx),
                                    _ptr(gate), _ptr(margin), int(nthreads))
    return dict(out=out, shared=shared, routed=routed, idx=idx, gate=gate, margin=margin,
                threads=int(used))


def backward(x_all, C, bias, w1, w3, w2, ws1, ws3, ws2, K, dout, *, alpha=0.0, tokens=None,
             experts=(), want_shared=False, want_dC=False, no_residual=False, forced_idx=None,
             renorm=False, sigmoid=False, nthreads=0):
    """Backward of the layer in fp64 (oracle.c, oracle_backward).

    x_all, dout: [T, d] bf16 bits — every token of the batch (the balance
    statistics and dC need all of them).  Weights as for forward().  alpha
    weighs the expert-level balance loss.  Returns a dict with, where asked:
    dx [n_tok, d], dgate [n_tok, K], idx [n_tok, K] for `tokens` (default
    all); dw1/dw3 [n_exp, I, d], dw2 [n_exp, d, I] for `experts`; dws1/dws3/
    dws2 for the shared experts (want_shared); dC [E, d] (want_dC); and
    counts [E], mean_score [E], bal (L_bal) and bal_alpha (alpha * L_bal)."""
    x_all = np.ascontiguousarray(x_all)
    T, d = x_all.shape
    E = C.shape[0]
    C = _u16(C, (E, d))
    dout = _u16(dout, (T, d))
    Ks = 0 if ws1 is None else len(ws1)
    I = next(a.shape[0] for a in w1 if a is not None) if E else 0
    Is = ws1[0].shape[0] if Ks else 0
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    keep = []
    tw = []
    zero_i = np.zeros((I, d), np.uint16)
    zero_o = np.zeros((d, I), np.uint16)
    for stack, shp, z in ((w1, (I, d), zero_i), (w3, (I, d), zero_i), (w2, (d, I), zero_o)):
        lst = [z if stack[e] is None else stack[e] for e in range(E)]
        t, k = _ptr_table(lst, E, shp)
        tw.append(t)
        keep.append(k)
    ts = []
    for stack, shp in ((ws1, (Is, d)), (ws3, (Is, d)), (ws2, (d, Is))):
        t, k = _ptr_table(stack if Ks else [], Ks, shp)
        ts.append(t)
        keep.append(k)
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, np.int32)
    assert tok.size == 0 or (tok.min() >= 0 and tok.max() < T and np.unique(tok).size == tok.size)
    ex = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
    assert ex.size == 0 or (ex.min() >= 0 and ex.max() < E)
    fi = None
    if forced_idx is not None:
        fi = np.ascontiguousarray(forced_idx, dtype=np.int32)
        assert fi.shape == (T, K)
    sh = _Shape(T, d, E, I, K, Ks, Is,
                (NO_RESIDUAL if no_residual else 0) | _gating(renorm, sigmoid))
    n, m = tok.size, ex.size
    r = dict(dx=np.zeros((n, d)), dgate=np.zeros((n, K)), idx=np.zeros((n, K), np.int32),
             dw1=np.zeros((m, I, d)), dw3=np.zeros((m, I, d)), dw2=np.zeros((m, d, I)),
             dws1=np.zeros((Ks, Is, d)) if want_shared else None,
             dws3=np.zeros((Ks, Is, d)) if want_shared else None,
             dws2=np.zeros((Ks, d, Is)) if want_shared else None,
             dC=np.zeros((E, d)) if want_dC else None,
             counts=np.zeros(E, np.int64), mean_score=np.zeros(E), bal=np.zeros(2))
    used = lib().oracle_backward(ctypes.byref(sh), _ptr(x_all), T, _ptr(C), _ptr(b),
                                 tw[0], tw[1], tw[2], ts[0], ts[1], ts[2],
                                 _ptr(dout), float(alpha), _ptr(fi),
                                 _ptr(tok), n, _ptr(ex), m, int(bool(want_shared)),
                                 int(bool(want_dC)),
                                 _ptr(r["dx"]), _ptr(r["dgate"]), _ptr(r["idx"]), _ptr(r["dw1"]),
                                 _ptr(r["dw3"]), _ptr(r["dw2"]), _ptr(r["dws1"]), _ptr(r["dws3"]),
                                 _ptr(r["dws2"]), _ptr(r["dC"]), _ptr(r["counts"]),
                                 _ptr(r["mean_score"]), _ptr(r["bal"]), int(nthreads))
    r["bal_alpha"] = float(r["bal"][1])
    r["bal"] = float(r["bal"][0])
    r["threads"] = int(used)
    return r
