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

from helpers import PART_RMS_TOL, PART_TOL, rms


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
