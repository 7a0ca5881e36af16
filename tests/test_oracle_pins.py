"""Pins of the fp64 oracle against facts the pages and mathematics fix.

Each test names what it pins; together they are chosen so that a plausible
slip in the oracle (W1/W3 swapped, W2 transposed, a sign in silu, a wrong
softmax axis, a gate applied to the wrong expert, a dropped shared or
residual term, a wrong tie-break) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import cost, ref_np
import synth
from synth import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def bf(a):
    """float values exactly representable in bf16 -> bf16 bit patterns."""
    a = np.asarray(a, dtype=np.float32)
    bits = synth.f32_to_bf16_rne(a)
    assert np.array_equal(synth.bf16_to_f64(bits), a.astype(np.float64)), "not bf16-exact"
    return bits


def rand_bf16(rng, shape, sigma):
    return synth.f32_to_bf16_rne((rng.standard_normal(shape) * sigma).astype(np.float32))


def rand_layer(rng, T, d, E, I, K, Ks, Is, sc=0.05, sx=1.0, cs=0.3):
    return dict(x=rand_bf16(rng, (T, d), sx), C=rand_bf16(rng, (E, d), cs),
                w1=rand_bf16(rng, (E, I, d), sc), w3=rand_bf16(rng, (E, I, d), sc),
                w2=rand_bf16(rng, (E, d, I), sc), ws1=rand_bf16(rng, (Ks, Is, d), sc),
                ws3=rand_bf16(rng, (Ks, Is, d), sc), ws2=rand_bf16(rng, (Ks, d, Is), sc))


def run(L, K, bias=None, **kw):
    return oracle.forward(L["x"], L["C"], bias, L["w1"], L["w3"], L["w2"],
                          L["ws1"], L["ws3"], L["ws2"], K, **kw)


# ---------------------------------------------------------------- P1
def test_p1_ptflops_expert_printout():
    """One bias-ful expert (7168 -> 2048) over 256 tokens reproduces every
    rounded figure of the youleyou page's ptflops printout."""
    g = _gold("ptflops_expert.json")
    i = g["input"]
    c = cost.expert_cost(i["dim"], i["inter"], i["tokens"], bias=i["bias"])
    assert c["params"] == 44_051_456
    assert c["w1_params"] == c["w3_params"] == 14_682_112
    assert c["w2_params"] == 14_687_232
    assert c["w1_macs"] == c["w3_macs"] == 3_758_620_672
    assert c["w2_macs"] == 3_759_931_392
    assert c["total_macs"] == 11_277_697_024
    lines = cost.ptflops_lines(c)
    for k, v in g["printed"].items():
        assert list(lines[k]) == v, (k, lines[k], v)
    # without biases the printout would read differently: the page counts them
    nb = cost.ptflops_lines(cost.expert_cost(7168, 2048, 256, bias=False))
    assert nb["expert"][0] != g["printed"]["expert"][0]


# ---------------------------------------------------------------- P2
@pytest.mark.parametrize("m,I", [(4, 3), (2, 5), (8, 2)])
def test_p2_segmentation_identity(m, I):
    """An FFN of inter m*I split into m experts of inter I (W1/W3 row blocks,
    W2 column blocks) sums back to the unsplit FFN; with zero centroids every
    score is 1/E exactly, so routing all E segments gives FFN_std / E."""
    rng = np.random.default_rng(100 + m)
    T, d = 9, 16
    std = rand_layer(rng, T, d, 1, m * I, 0, 1, m * I)
    W1, W3, W2 = std["ws1"][0], std["ws3"][0], std["ws2"][0]
    E = m
    seg = dict(x=std["x"], C=np.zeros((E, d), np.uint16),
               w1=np.stack([W1[j * I:(j + 1) * I] for j in range(m)]),
               w3=np.stack([W3[j * I:(j + 1) * I] for j in range(m)]),
               w2=np.stack([np.ascontiguousarray(W2[:, j * I:(j + 1) * I]) for j in range(m)]),
               ws1=np.zeros((0, I, d), np.uint16), ws3=np.zeros((0, I, d), np.uint16),
               ws2=np.zeros((0, d, I), np.uint16))
    a = run(seg, K=E, no_residual=True)
    dense = dict(std, C=np.zeros((1, d), np.uint16))
    b = run(dense, K=0, no_residual=True)
    assert np.all(a["gate"] == 1.0 / E)
    np.testing.assert_allclose(E * a["routed"], b["shared"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a["out"], a["routed"], rtol=0, atol=0)


# ---------------------------------------------------------------- P3
def test_p3_shared_only_is_dense_swiglu():
    """K = 0: the layer is the residual plus the dense SwiGLU FFNs of the
    shared experts (numpy float64 matrix products)."""
    rng = np.random.default_rng(3)
    T, d, Is, Ks = 7, 32, 24, 2
    L = rand_layer(rng, T, d, 4, 8, 0, Ks, Is)
    r = run(L, K=0)
    X = synth.bf16_to_f64(L["x"])
    ref = X.copy()
    for s in range(Ks):
        A = X @ synth.bf16_to_f64(L["ws1"][s]).T
        B = X @ synth.bf16_to_f64(L["ws3"][s]).T
        ref += ((A / (1 + np.exp(-A))) * B) @ synth.bf16_to_f64(L["ws2"][s]).T
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-13)
    assert np.all(r["routed"] == 0)


# ---------------------------------------------------------------- P4
def test_p4_topk_brute_force():
    """Top-K equals the best of all C(E,K) subsets (sum of scores) and is in
    descending score order; equals a full stable sort."""
    rng = np.random.default_rng(4)
    for trial in range(40):
        E = int(rng.integers(2, 11))
        K = int(rng.integers(1, E + 1))
        d = 8
        x = rand_bf16(rng, (3, d), 1.0)
        C = rand_bf16(rng, (E, d), 0.5)
        b = (rng.standard_normal(E) * 0.3).astype(np.float32) if trial % 2 else None
        idx, gate, margin, probs = oracle.route(x, C, b, K, return_probs=True)
        for t in range(3):
            p = probs[t]
            best = max(itertools.combinations(range(E), K), key=lambda s: sum(p[i] for i in s))
            assert set(idx[t].tolist()) == set(best)
            assert np.all(np.diff(p[idx[t]]) <= 0)
            assert idx[t].tolist() == sorted(range(E), key=lambda i: (-p[i], i))[:K]
            np.testing.assert_array_equal(gate[t], p[idx[t]])
            if K < E:
                rest = np.delete(p, idx[t])
                assert margin[t] == p[idx[t][-1]] - rest.max()
            else:
                assert margin[t] == np.inf
            assert abs(p.sum() - 1.0) < 1e-14


def test_p4_two_expert_softmax_closed_form():
    """Logits (0, 1): the scores are (1 - logistic(1), logistic(1))."""
    lg1 = _gold("hand_examples.json")["constants"]["logistic_1"]
    x = bf([[1, 0]])
    C = bf([[0, 0], [1, 0]])
    idx, gate, margin, probs = oracle.route(x, C, None, 1, return_probs=True)
    assert idx.tolist() == [[1]]
    assert abs(probs[0, 1] - lg1) < 1e-16 and abs(probs[0, 0] - (1 - lg1)) < 1e-16
    assert abs(margin[0] - (2 * lg1 - 1)) < 1e-15


# ---------------------------------------------------------------- P5
def test_p5_zero_centroids_tie_break():
    """All scores tie: the K lowest expert ids are chosen, in order, gate 1/E."""
    x = bf(np.ones((2, 4)))
    E, K = 16, 5
    idx, gate, margin = oracle.route(x, np.zeros((E, 4), np.uint16), None, K)
    assert idx.tolist() == [list(range(K))] * 2
    assert np.all(gate == 1.0 / E)
    assert np.all(margin == 0.0)


# ---------------------------------------------------------------- P6
def test_p6_zero_weights():
    rng = np.random.default_rng(6)
    L = rand_layer(rng, 5, 16, 4, 8, 2, 1, 8)
    X = synth.bf16_to_f64(L["x"])
    L0 = dict(L, w2=np.zeros_like(L["w2"]), ws2=np.zeros_like(L["ws2"]))
    assert np.array_equal(run(L0, K=2)["out"], X)
    Lz = {k: np.zeros_like(v) for k, v in L.items()}
    Lz["x"] = L["x"]
    assert np.all(run(Lz, K=2, no_residual=True)["out"] == 0)
    # K = K_s = 0: out == x exactly
    Ln = dict(L, ws1=L["ws1"][:0], ws3=L["ws3"][:0], ws2=L["ws2"][:0])
    assert np.array_equal(run(Ln, K=0)["out"], X)


# ---------------------------------------------------------------- P7
def _hand_case(case, g):
    lg1 = g["constants"]["logistic_1"]
    ex = {k: g[k] for k in ("expert_a", "expert_b")}
    d = case["d"]
    x = bf([g["x"]])
    if case["Ks"]:
        e = ex[case["shared"]]
        ws1, ws3, ws2 = bf([e["w1"]]), bf([e["w3"]]), bf([e["w2"]])
    else:
        ws1 = np.zeros((0, 1, d), np.uint16)
        ws3 = np.zeros((0, 1, d), np.uint16)
        ws2 = np.zeros((0, d, 1), np.uint16)
    if case["K"]:
        C = bf(case["centroids"])
        w1 = bf([ex[n]["w1"] for n in case["experts"]])
        w3 = bf([ex[n]["w3"] for n in case["experts"]])
        w2 = bf([ex[n]["w2"] for n in case["experts"]])
    else:
        C = np.zeros((1, d), np.uint16)
        w1 = w3 = np.zeros((1, 1, d), np.uint16)
        w2 = np.zeros((1, d, 1), np.uint16)
    bias = np.asarray(case["bias"], np.float32) if "bias" in case else None
    r = oracle.forward(x, C, bias, w1, w3, w2, ws1, ws3, ws2, case["K"])
    return r, lg1


def test_p7_hand_examples():
    """Closed forms with exact bf16 inputs (see tests/golden/hand_examples.json)."""
    g = _gold("hand_examples.json")
    S = None
    for case in g["cases"]:
        r, S = _hand_case(case, g)
        fa = np.array([2 * S * 1.0, 2 * S * 0.5])       # expert_a at x = (1, 0)
        fb = np.array([S, S])                            # expert_b at x = (1, 0)
        x = np.array([1.0, 0.0])
        if case["name"] == "shared_only":
            exp = x + fa
        elif case["name"] in ("routed_top1", "bias_top1"):
            exp = x + S * fa
        else:
            exp = x + S * fa + (1 - S) * fb
        np.testing.assert_allclose(r["out"][0], exp, rtol=1e-15, atol=1e-16, err_msg=case["name"])
        if case["K"]:
            assert r["idx"][0].tolist() == case["idx"]
            gates = [S if s == "logistic_1" else 1 - S for s in case["gate"]]
            np.testing.assert_allclose(r["gate"][0], gates, rtol=1e-15)
    # silu(1) itself
    assert S == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-16)


# ---------------------------------------------------------------- P8
def test_p8_permutation_invariances():
    rng = np.random.default_rng(8)
    T, d, E, I, K = 12, 16, 8, 8, 3
    L = rand_layer(rng, T, d, E, I, K, 1, 8)
    b = (rng.standard_normal(E) * 0.2).astype(np.float32)
    r = run(L, K, bias=b)
    perm = rng.permutation(T)
    r2 = run(dict(L, x=L["x"][perm]), K, bias=b)
    assert np.array_equal(r2["out"], r["out"][perm])
    assert np.array_equal(r2["idx"], r["idx"][perm])
    # relabel experts consistently
    q = rng.permutation(E)
    Lq = dict(L, C=L["C"][q], w1=L["w1"][q], w3=L["w3"][q], w2=L["w2"][q])
    rq = run(Lq, K, bias=b[q])
    assert np.all(r["margin"] > 1e-9)
    np.testing.assert_allclose(rq["out"], r["out"], rtol=1e-13, atol=1e-15)
    inv = np.argsort(q)
    assert np.array_equal(np.sort(q[rq["idx"]], 1), np.sort(r["idx"], 1))
    assert inv.shape == (E,)


# ---------------------------------------------------------------- P9
@pytest.mark.parametrize("N,m,Kstd,I", [(16, 4, 2, 1024), (4, 4, 1, 1024), (64, 8, 6, 2048)])
def test_p9_equal_cost_segmentation(N, m, Kstd, I):
    """Splitting N experts of inter I into N*m of inter I/m and routing m*K
    keeps parameters and per-token MACs exactly equal."""
    d = 1024
    a = cost.layer_cost(N, I, Kstd, 0, 0, d)
    b = cost.layer_cost(N * m, I // m, m * Kstd, 0, 0, d)
    assert a == b


def test_p9_layer_cost_exact_integers():
    """layer_cost against exact integers fixed elsewhere: one bias-free expert
    of the youleyou printout (dim 7168, inter 2048) has 3 * 7168 * 2048 =
    44 040 192 parameters (the printed 44.05 M minus its 2 * 2048 + 7168
    biases), so the V3-shape layer (256 routed + 1 shared, top-8) holds
    257 such experts and a token passes through 9 of them, one MAC per
    parameter.  Dropping d, I, K or the shared term changes these numbers."""
    one = 44_040_192
    assert cost.expert_cost(7168, 2048, 1, bias=False)["params"] == one
    assert cost.expert_cost(7168, 2048, 1, bias=True)["params"] - (2 * 2048 + 7168) == one
    v3 = cost.layer_cost(256, 2048, 8, 1, 2048, 7168)
    assert v3 == dict(params=257 * one, token_macs=9 * one)
    assert v3["params"] == 11_318_329_344
    # the tiny layer: 16 routed + 1 shared of inter 256 on d = 512, top-4
    assert cost.layer_cost(16, 256, 4, 1, 256, 512) == dict(params=17 * 393_216,
                                                            token_macs=5 * 393_216)
    # shared inter-dim distinct from the routed one, two shared experts
    assert cost.layer_cost(64, 1408, 6, 2, 704, 2048) == dict(
        params=64 * 3 * 2048 * 1408 + 2 * 3 * 2048 * 704,
        token_macs=6 * 3 * 2048 * 1408 + 2 * 3 * 2048 * 704)


# ---------------------------------------------------------------- P10
def test_p10_combinations():
    for c in _gold("combinations.json")["cases"]:
        assert math.comb(c["n"], c["k"]) == c["value"]


# ---------------------------------------------------------------- P11
def test_p11_hit_entropy_and_gate_invariants():
    g = _gold("hit_entropy.json")["cases"][0]
    E = g["num_experts"]
    idx = np.tile(np.arange(E), 5)
    ent, active, counts = cost.hit_entropy(idx, E)
    assert ent == pytest.approx(math.log(E), rel=1e-15)
    assert f"{cost.max_entropy(E):.2f}" == g["max_entropy_2dp"]
    assert active == 1.0
    # collapsed routing: entropy 0, one expert active
    ent0, act0, _ = cost.hit_entropy(np.zeros(40, int), E)
    assert ent0 == 0.0 and act0 == 1 / E
    # gate invariants on a random layer
    rng = np.random.default_rng(11)
    for K, E2 in ((3, 8), (8, 8)):
        L = rand_layer(rng, 20, 16, E2, 4, K, 0, 4)
        r = run(L, K)
        c = np.bincount(r["idx"].ravel(), minlength=E2)
        assert c.sum() == 20 * K
        assert np.all(r["gate"] > 0) and np.all(r["gate"] <= 1)
        s = r["gate"].sum(1)
        if K == E2:
            np.testing.assert_allclose(s, 1.0, rtol=1e-14)
        else:
            assert np.all(s < 1.0)


# ---------------------------------------------------------------- P12
def _np_vs_c(L, K, bias=None, no_residual=False):
    a = run(L, K, bias=bias, no_residual=no_residual)
    b = ref_np.forward(L["x"], L["C"], bias, L["w1"], L["w3"], L["w2"], L["ws1"], L["ws3"],
                       L["ws2"], K, no_residual=no_residual)
    assert np.array_equal(a["idx"], b["idx"])
    for k in ("out", "shared", "routed"):
        scale = max(np.abs(b[k]).max(), 1e-300)
        assert np.abs(a[k] - b[k]).max() <= 1e-12 * scale, k
    np.testing.assert_allclose(a["gate"], b["gate"], rtol=1e-12)


def test_p12_numpy_cross_check_tiny_workload():
    w = wl.WORKLOADS["tiny"]
    L = wl.gen_all(w)
    _np_vs_c(L, w.K, no_residual=True)
    _np_vs_c(L, w.K)


def test_p12_numpy_cross_check_random_shapes():
    rng = np.random.default_rng(12)
    for trial in range(6):
        T = int(rng.integers(1, 20))
        d = int(rng.choice([8, 16, 24]))
        E = int(rng.integers(1, 12))
        K = int(rng.integers(0, E + 1))
        Ks = int(rng.integers(0, 3))
        I = int(rng.integers(1, 9))
        Is = int(rng.integers(1, 9))
        L = rand_layer(rng, T, d, E, I, K, Ks, Is)
        b = (rng.standard_normal(E) * 0.5).astype(np.float32) if trial % 2 else None
        _np_vs_c(L, K, bias=b, no_residual=bool(trial % 3 == 0))


def test_forced_routing_matches_free_routing():
    """Forcing the oracle's own selection reproduces it exactly; forcing
    another selection changes only the routed part."""
    rng = np.random.default_rng(13)
    L = rand_layer(rng, 10, 16, 8, 8, 3, 1, 8)
    r = run(L, 3)
    f = run(L, 3, forced_idx=r["idx"])
    assert np.array_equal(f["out"], r["out"])
    other = (r["idx"] + 1) % 8
    g = run(L, 3, forced_idx=other)
    assert np.array_equal(g["shared"], r["shared"])
    assert not np.allclose(g["routed"], r["routed"])
