"""Pins the bars of the expert-part parity checks (PART_TOL, PART_RMS_TOL in
helpers.py) to the arithmetic the kernels are specified to do.

The GPU path stores the SwiGLU output H and the expert output Y as bf16 and
rounds the returned part once to bf16 (the reading of the intermediate
precision in the design notes: bf16 operands, fp32 accumulation, bf16
intermediates).  This test emulates exactly those three roundings on top of
exact fp64 products — no GPU and no GPU code involved — on the token samples
the GPU tests draw, and measures how far the result lands from the oracle's
exact parts.  The bars must clear that error with room to spare, and must not
be so loose that a wrong expert, gate or row would still pass: a planted
mistake (one token's expert swapped) must fail them."""
import numpy as np
import pytest

import oracle
import synth
from oracle.ref_np import widen
from synth import workloads as wl

from helpers import GRAD_RMS_TOL, GRAD_TOL, PART_RMS_TOL, PART_TOL, rms


def _bf16(a):
    return synth.bf16_to_f64(synth.f32_to_bf16_rne(np.asarray(a, np.float32)))


def _ffn_rounded(X, w1, w3, w2):
    A = X @ widen(w1).T
    B = X @ widen(w3).T
    H = _bf16(A / (1.0 + np.exp(-A)) * B)          # rounding 1: H stored as bf16
    return _bf16(H @ widen(w2).T)                  # rounding 2: Y stored as bf16


def _emulate(L, tok, idx, gate, Ks):
    """Shared and routed parts with the GPU's rounding points; the returned
    part is rounded once more (rounding 3)."""
    X = widen(L["x"][tok])
    shared = np.zeros((len(tok), X.shape[1]))
    for s in range(Ks):
        shared += _ffn_rounded(X, L["ws1"][s], L["ws3"][s], L["ws2"][s])
    routed = np.zeros_like(shared)
    for e in np.unique(idx):
        r, k = np.nonzero(idx == e)
        routed[r] += gate[r, k][:, None] * _ffn_rounded(X[r], L["w1"][e], L["w3"][e], L["w2"][e])
    return _bf16(shared), _bf16(routed), _bf16(shared + routed)


def _ratios(got, ref):
    s = rms(ref)
    return float(np.abs(got - ref).max()) / s, rms(got - ref) / s


def _sample(T, n):
    # the draw of the GPU forward-parity test
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(T)
    s = np.sort(rng.choice(T, n, replace=False))
    s[0], s[-1] = 0, T - 1
    return np.unique(s)


@pytest.mark.parametrize("name,n", [("tiny", 128), ("2b", 128), ("16b_zipf", 48)])
def test_part_bars_cover_the_specified_roundings(name, n):
    w = wl.WORKLOADS[name]
    L = wl.gen_all(w)
    tok = _sample(w.T, n)
    ref = oracle.forward(L["x"][tok], L["C"], L["bias"], L["w1"], L["w3"], L["w2"], L["ws1"],
                         L["ws3"], L["ws2"], w.K, no_residual=True)
    sh, ro, de = _emulate(L, tok, ref["idx"], ref["gate"], w.Ks)
    worst = []
    for got, exact in ((sh, ref["shared"]), (ro, ref["routed"]), (de, ref["out"])):
        mx, rm = _ratios(got, exact)
        worst.append((mx, rm))
        assert mx <= PART_TOL / 1.4, (name, mx)
        assert rm <= PART_RMS_TOL / 2.5, (name, rm)
    # the bars sit within a small factor of what rounding alone costs
    assert max(m for m, _ in worst) >= PART_TOL / 5
    assert max(r for _, r in worst) >= PART_RMS_TOL / 8

    # a wrong expert for a single token must fail the RMS bar
    bad = ref["idx"].copy()
    t0 = 0
    spare = [e for e in range(w.E) if e not in bad[t0]]
    bad[t0, 0] = spare[0]
    _, ro_bad, _ = _emulate(L, tok, bad, ref["gate"], 0)
    mx, rm = _ratios(ro_bad, ref["routed"])
    assert mx > PART_TOL or rm > PART_RMS_TOL, (name, mx, rm)


# ---------------------------------------------------------------------------
# The backward.  Its specified rounding points: the saved pre-activations
# Z = [W1 x | W3 x] (bf16), the per-row dZ = [dA | dB] and g*H (bf16), the
# affinity gradients (bf16), each row's input gradient (bf16), and the bf16
# results dx, dW1, dW3, dW2; gate gradients and dC stay fp32.  Weight
# gradients are far more heavy-tailed than layer outputs (max/RMS up to ~9
# against ~4.5), so their max error is taken relative to max|ref|; the RMS
# bar is the parts' one.



def _silu(a):
    return a / (1.0 + np.exp(-a))


def _dsilu(a):
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def _emulate_backward(L, K, idx, gate, probs, experts):
    """dx, dgate, dW of `experts`, shared dW, dC with the GPU's rounding
    points (softmax gate, no renormalisation, alpha = 0)."""
    X, dO = widen(L["x"]), widen(L["dout"])
    T, d = X.shape
    E = L["C"].shape[0]
    dXr_sum = np.zeros((T, d))
    dgate = np.zeros((T, K))
    out = {}

    def one(rows, w1, w3, w2, g):
        Xr, dOr = X[rows], dO[rows]
        W1, W3, W2 = widen(w1), widen(w3), widen(w2)
        A, B = _bf16(Xr @ W1.T), _bf16(Xr @ W3.T)
        dHp = dOr @ W2
        Hb = _silu(A) * B
        dg = (dHp * Hb).sum(axis=1)
        dH = g[:, None] * dHp
        dA, dB = _bf16(dH * B * _dsilu(A)), _bf16(dH * _silu(A))
        gH = _bf16(g[:, None] * Hb)
        return dg, _bf16(dA @ W1 + dB @ W3), (_bf16(dA.T @ Xr), _bf16(dB.T @ Xr), _bf16(dOr.T @ gH))

    for e in range(E):
        r, k = np.nonzero(idx == e)
        if r.size == 0:
            continue
        dg, dxr, dws = one(r, L["w1"][e], L["w3"][e], L["w2"][e], gate[r, k])
        dgate[r, k] = dg
        np.add.at(dXr_sum, r, dxr)
        if e in experts:
            out[("dw", e)] = dws
    for s in range(len(L["ws1"])):
        _, dxr, dws = one(np.arange(T), L["ws1"][s], L["ws3"][s], L["ws2"][s], np.ones(T))
        dXr_sum += dxr
        out[("dws", s)] = dws
    ds = np.zeros_like(probs)
    np.put_along_axis(ds, idx, dgate, axis=1)
    dl = probs * (ds - (probs * ds).sum(axis=1, keepdims=True))
    dLb = _bf16(dl)
    out["dx"] = _bf16(dO + dLb @ widen(L["C"]) + dXr_sum)
    out["dgate"] = dgate
    out["dC"] = dLb.T @ X
    return out


def _grad_ratios(got, ref):
    return (float(np.abs(got - ref).max()) / float(np.abs(ref).max()),
            rms(got - ref) / rms(ref))


@pytest.mark.parametrize("name", ["tiny", "2b"])
def test_grad_bars_cover_the_specified_roundings(name):
    w = wl.WORKLOADS[name]
    L = wl.gen_all(w)
    L["dout"] = wl.gen_dout(w)
    idx, gate, _, probs = oracle.route(L["x"], L["C"], L["bias"], w.K, return_probs=True)
    experts = list(range(w.E)) if w.E <= 16 else [0, w.E // 2, w.E - 1]
    ref = oracle.backward(L["x"], L["C"], L["bias"], L["w1"], L["w3"], L["w2"], L["ws1"],
                          L["ws3"], L["ws2"], w.K, L["dout"], experts=experts, want_shared=True,
                          want_dC=True, forced_idx=idx)
    em = _emulate_backward(L, w.K, idx, gate, probs, set(experts))
    pairs = [("dx", em["dx"], ref["dx"]), ("dgate", em["dgate"], ref["dgate"]),
             ("dC", em["dC"], ref["dC"])]
    for q, e in enumerate(experts):
        for n, a in zip(("dw1", "dw3", "dw2"), em[("dw", e)]):
            pairs.append((n, a, ref[n][q]))
    for n, a in zip(("dws1", "dws3", "dws2"), em[("dws", 0)]):
        pairs.append((n, a, ref[n][0]))
    worst_mx = worst_rm = 0.0
    for n, a, r in pairs:
        mx, rm = _grad_ratios(a, r)
        worst_mx, worst_rm = max(worst_mx, mx), max(worst_rm, rm)
        assert mx <= GRAD_TOL / 2, (name, n, mx)
        assert rm <= GRAD_RMS_TOL / 2.5, (name, n, rm)
    # the bars are within a small factor of what the roundings cost
    assert worst_mx >= GRAD_TOL / 10 and worst_rm >= GRAD_RMS_TOL / 8, (worst_mx, worst_rm)
