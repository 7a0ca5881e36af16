"""Pins of the oracle's two gating variants: gates renormalised over the
selected experts, and sigmoid affinities whose per-expert bias steers the
selection only.  Each check is fixed by the pages or by the mathematics, not
by re-running the oracle's own formula: printed-style closed forms, a
softmax over the selected logits (the explainer's routing code), brute force
over expert subsets, invariances, and the independent numpy formulation."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import ref_np

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "gating_examples.json")))
L1 = GOLD["logistic_1"]
E_ = math.e


def bf16(a):
    a = np.asarray(a, np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "hand inputs must be exact in bf16"
    return (u >> 16).astype(np.uint16)


def _eval(expr):
    return eval(expr, {"logistic_1": L1, "e": E_})  # closed forms from the golden file


@pytest.mark.parametrize("case", GOLD["cases"], ids=[c["name"] for c in GOLD["cases"]])
def test_hand_examples(case):
    x = bf16([GOLD["x"]])
    C = bf16(case["centroids"])
    bias = None if case["bias"] is None else np.asarray(case["bias"], np.float32)
    idx, gate, _ = oracle.route(x, C, bias, case["K"], renorm=case["renorm"],
                                sigmoid=case["sigmoid"])
    assert idx[0].tolist() == case["idx"]
    want = [_eval(g) for g in case["gate"]]
    assert np.allclose(gate[0], want, rtol=0, atol=1e-15)


def _rand(seed, n=24, d=64, E=16, scale=0.3, bias=True):
    rng = np.random.default_rng(seed)
    x = bf16(np.round(rng.normal(size=(n, d)) * 64) / 64)
    C = bf16(np.round(rng.normal(size=(E, d)) * scale * 64) / 64)
    b = (rng.normal(size=E) * 0.05).astype(np.float32) if bias else None
    return x, C, b


def _logits(x, C, b):
    L = ref_np.widen(x) @ ref_np.widen(C).T
    return L if b is None else L + b.astype(np.float64)[None, :]


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("K", [1, 3, 8])
def test_renorm_is_softmax_over_selected_logits(seed, K):
    """The explainer's routing: top-K of the logits, then a softmax over those
    K.  Selection is the same as without renormalisation."""
    x, C, b = _rand(seed)
    idx, gate, margin = oracle.route(x, C, b, K, renorm=True)
    idx0, gate0, _ = oracle.route(x, C, b, K)
    assert np.array_equal(idx, idx0)
    L = _logits(x, C, b)
    for t in range(x.shape[0]):
        if margin[t] <= 1e-12:
            continue
        top = np.argsort(-L[t], kind="stable")[:K]
        assert set(top.tolist()) == set(idx[t].tolist())
        z = np.exp(L[t, idx[t]] - L[t, idx[t]].max())
        assert np.allclose(gate[t], z / z.sum(), rtol=1e-12, atol=0)
        assert abs(gate[t].sum() - 1.0) < 1e-14
    if K == 1:
        assert np.all(gate == 1.0)


def test_renorm_with_all_experts_is_plain_softmax():
    x, C, b = _rand(4, E=8)
    _, g_r, _ = oracle.route(x, C, b, 8, renorm=True)
    _, g_p, _ = oracle.route(x, C, b, 8)
    assert np.allclose(g_r, g_p, rtol=1e-14, atol=0)


@pytest.mark.parametrize("seed", [5, 6])
@pytest.mark.parametrize("renorm", [False, True])
def test_sigmoid_gates_ignore_the_bias(seed, renorm):
    """Gates are the unbiased sigmoid scores of whichever experts the biased
    keys chose; shifting every bias by the same constant changes nothing."""
    x, C, b = _rand(seed)
    K = 4
    idx, gate, margin = oracle.route(x, C, b, K, sigmoid=True, renorm=renorm)
    S = 1.0 / (1.0 + np.exp(-(ref_np.widen(x) @ ref_np.widen(C).T)))
    for t in range(x.shape[0]):
        g = S[t, idx[t]]
        if renorm:
            g = g / g.sum()
        assert np.allclose(gate[t], g, rtol=1e-13, atol=0)
    idx2, gate2, _ = oracle.route(x, C, (b + np.float32(0.5)).astype(np.float32), K,
                                  sigmoid=True, renorm=renorm)
    ok = margin > 1e-9
    assert np.array_equal(idx[ok], idx2[ok])
    assert np.allclose(gate[ok], gate2[ok], rtol=1e-15, atol=0)


def test_sigmoid_zero_centroids_select_by_bias():
    """All affinities are 0, every score sigmoid(0) = 1/2: the bias alone
    orders the experts (ties to the lower index) and every gate is 1/2, or
    1/K renormalised."""
    rng = np.random.default_rng(7)
    E, K, d = 12, 5, 64
    x, _, _ = _rand(8, n=6, d=d, E=E)
    C = np.zeros((E, d), np.uint16)
    b = np.round(rng.normal(size=E) * 8).astype(np.float32) / 8
    b[3] = b[9]                                   # a tie, broken toward expert 3
    idx, gate, _ = oracle.route(x, C, b, K, sigmoid=True)
    want = np.argsort(-b.astype(np.float64), kind="stable")[:K]
    assert all(row.tolist() == want.tolist() for row in idx)
    assert np.all(gate == 0.5)
    _, g_r, _ = oracle.route(x, C, b, K, sigmoid=True, renorm=True)
    assert np.allclose(g_r, 1.0 / K, rtol=0, atol=1e-16)


@pytest.mark.parametrize("E,K", [(6, 2), (8, 3), (10, 4)])
def test_sigmoid_selection_brute_force(E, K):
    """The chosen set maximises the summed selection key over all subsets."""
    x, C, b = _rand(9, n=8, E=E)
    idx, _, margin = oracle.route(x, C, b, K, sigmoid=True)
    S = 1.0 / (1.0 + np.exp(-(ref_np.widen(x) @ ref_np.widen(C).T)))
    keys = S + b.astype(np.float64)[None, :]
    for t in range(x.shape[0]):
        if margin[t] <= 1e-12:
            continue
        best = max(itertools.combinations(range(E), K), key=lambda c: keys[t, list(c)].sum())
        assert set(best) == set(idx[t].tolist())
        assert np.all(np.diff(keys[t, idx[t]]) <= 0)      # descending key order


@pytest.mark.parametrize("renorm,sigmoid", [(True, False), (False, True), (True, True)])
def test_numpy_formulation_agrees(renorm, sigmoid):
    """The whole layer under each variant, against the independent numpy
    formulation (whole-matrix products, sort-based top-K)."""
    rng = np.random.default_rng(11)
    T, d, E, I, K, Ks = 20, 64, 8, 64, 3, 1
    x, C, b = _rand(12, n=T, d=d, E=E)

    def w(*shape):
        return bf16(np.round(rng.normal(size=shape) * 0.06 * 256) / 256)
    w1, w3, w2 = w(E, I, d), w(E, I, d), w(E, d, I)
    s1, s3, s2 = w(Ks, I, d), w(Ks, I, d), w(Ks, d, I)
    r = oracle.forward(x, C, b, w1, w3, w2, s1, s3, s2, K, renorm=renorm, sigmoid=sigmoid)
    n = ref_np.forward(x, C, b, w1, w3, w2, s1, s3, s2, K, renorm=renorm, sigmoid=sigmoid)
    ok = r["margin"] > 1e-9
    assert np.array_equal(r["idx"][ok], n["idx"][ok])
    assert np.allclose(r["gate"][ok], n["gate"][ok], rtol=1e-12, atol=0)
    scale = np.abs(n["out"]).max()
    assert np.abs(r["out"][ok] - n["out"][ok]).max() <= 1e-12 * scale


def test_forced_routing_renormalises_over_the_forced_experts():
    x, C, b = _rand(13, n=4, d=64, E=8)
    forced = np.array([[0, 1, 2], [7, 6, 5], [3, 0, 7], [1, 4, 2]], np.int32)
    rng = np.random.default_rng(14)
    z = lambda *s: bf16(np.round(rng.normal(size=s) * 16) / 256)
    w1, w3, w2 = z(8, 64, 64), z(8, 64, 64), z(8, 64, 64)
    r = oracle.forward(x, C, b, w1, w3, w2, None, None, None, 3, forced_idx=forced, renorm=True)
    L = _logits(x, C, b)
    for t in range(4):
        g = np.exp(L[t, forced[t]] - L[t].max())
        assert np.allclose(r["gate"][t], g / g.sum(), rtol=1e-12, atol=0)


@pytest.mark.parametrize("sigmoid", [False, True])
def test_margin_is_the_gap_in_selection_keys(sigmoid):
    """The near-tie margin is key_(K) - key_(K+1) of whatever orders the
    selection: the softmax score, or sigmoid score + bias."""
    x, C, b = _rand(15, n=10, E=12)
    K = 4
    _, _, margin = oracle.route(x, C, b, K, sigmoid=sigmoid)
    if sigmoid:
        S = 1.0 / (1.0 + np.exp(-(ref_np.widen(x) @ ref_np.widen(C).T)))
        keys = S + b.astype(np.float64)[None, :]
    else:
        keys = ref_np.softmax_scores(ref_np.widen(x), ref_np.widen(C), b)
    srt = -np.sort(-keys, axis=1)
    assert np.allclose(margin, srt[:, K - 1] - srt[:, K], rtol=1e-9, atol=1e-15)
