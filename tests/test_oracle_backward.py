"""Pins of the backward oracle (oracle.c, oracle_backward) against what
holds independently of it:

B1  central finite differences of a separate numpy fp64 forward of the
    objective sum(dout * out) + alpha * L_bal, for elements of x, every
    weight stack and the centroids, under every gating variant;
B2  torch.autograd through a plain torch fp64 formulation of the same layer
    (a different method: reverse-mode differentiation of the forward);
B3  closed forms in logistic(1) of tiny hand examples: the SwiGLU
    derivative silu'(z) = sig(z) (1 + z (1 - sig(z))) through a shared expert,
    and the two-expert softmax router;
B4  the balance statistics: counts sum to T K, hit rates f_e sum to E,
    softmax mean scores sum to 1; zero centroids give L_bal = 1 exactly and a
    closed-form centroid gradient;
B5  special cases: dout = 0 and alpha = 0 give all-zero gradients; W2 = 0
    gives zero gate gradients, zero dW1/dW3 and dx = dout.

The objective and the balance-loss reading are stated in oracle.c."""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle.ref_np import widen

rng0 = np.random.default_rng


def _bf(a):
    return synth.f32_to_bf16_rne(np.asarray(a, np.float32))


def _layer(seed, T=12, d=8, E=6, I=4, K=2, Ks=1, Is=3, sc=0.4, bias=True):
    g = rng0(seed)
    L = dict(x=_bf(g.standard_normal((T, d))), C=_bf(g.standard_normal((E, d)) * 0.5),
             w1=_bf(g.standard_normal((E, I, d)) * sc), w3=_bf(g.standard_normal((E, I, d)) * sc),
             w2=_bf(g.standard_normal((E, d, I)) * sc), ws1=_bf(g.standard_normal((Ks, Is, d)) * sc),
             ws3=_bf(g.standard_normal((Ks, Is, d)) * sc), ws2=_bf(g.standard_normal((Ks, d, Is)) * sc),
             dout=_bf(g.standard_normal((T, d))),
             bias=(g.standard_normal(E) * 0.3).astype(np.float32) if bias else None)
    return L, K


def _np_objective(P, K, idx, alpha, renorm, sigmoid, no_residual):
    """sum(dout * out) + alpha * sum_e f_e P_e for double-valued parameters P
    under the fixed routing idx (the numpy formulation, independent of
    oracle.c)."""
    X, C, dO = P["x"], P["C"], P["dout"]
    T, d = X.shape
    E = C.shape[0]
    b = P["bias"]
    A = X @ C.T
    if sigmoid:
        S = 1.0 / (1.0 + np.exp(-A))
    else:
        Lg = A + (0.0 if b is None else b[None, :])
        Lg = Lg - Lg.max(axis=1, keepdims=True)
        S = np.exp(Lg)
        S = S / S.sum(axis=1, keepdims=True)
    rows = np.arange(T)[:, None]
    G = S[rows, idx]
    if renorm:
        G = G / G.sum(axis=1, keepdims=True)

    def ffn(Xs, w1, w3, w2):
        a = Xs @ w1.T
        return ((a / (1.0 + np.exp(-a))) * (Xs @ w3.T)) @ w2.T

    out = np.zeros_like(X) if no_residual else X.copy()
    for s in range(P["ws1"].shape[0]):
        out = out + ffn(X, P["ws1"][s], P["ws3"][s], P["ws2"][s])
    for k in range(K):
        for e in np.unique(idx[:, k]):
            sel = idx[:, k] == e
            out[sel] += G[sel, k][:, None] * ffn(X[sel], P["w1"][e], P["w3"][e], P["w2"][e])
    counts = np.bincount(idx.ravel(), minlength=E)
    f = E * counts / (K * T)
    return float((dO * out).sum() + alpha * (f * S.mean(axis=0)).sum())


def _oracle_all(L, K, alpha, **kw):
    E = L["C"].shape[0]
    return oracle.backward(L["x"], L["C"], L["bias"], L["w1"], L["w3"], L["w2"], L["ws1"],
                           L["ws3"], L["ws2"], K, L["dout"], alpha=alpha, experts=range(E),
                           want_shared=True, want_dC=True, **kw)


VARIANTS = [dict(), dict(renorm=True), dict(sigmoid=True), dict(sigmoid=True, renorm=True),
            dict(no_residual=True)]


@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: "-".join(v) or "softmax")
@pytest.mark.parametrize("alpha", [0.0, 0.7])
def test_b1_finite_differences(var, alpha):
    L, K = _layer(11 + len(var) + int(alpha * 10))
    r = _oracle_all(L, K, alpha, **var)
    idx = oracle.route(L["x"], L["C"], L["bias"], K, renorm=var.get("renorm", False),
                       sigmoid=var.get("sigmoid", False))[0]
    assert np.array_equal(idx, r["idx"])
    P = {k: (None if v is None else (v.astype(np.float64) if k == "bias" else widen(v)))
         for k, v in L.items()}
    grads = dict(x=r["dx"], C=r["dC"], w1=r["dw1"], w3=r["dw3"], w2=r["dw2"], ws1=r["dws1"],
                 ws3=r["dws3"], ws2=r["dws2"])
    flags = dict(renorm=var.get("renorm", False), sigmoid=var.get("sigmoid", False),
                 no_residual=var.get("no_residual", False))
    g = rng0(5)
    h = 1e-5
    for name, G in grads.items():
        for _ in range(6):
            pos = tuple(int(g.integers(0, n)) for n in P[name].shape)
            orig = P[name][pos]
            P[name][pos] = orig + h
            up = _np_objective(P, K, idx, alpha, **flags)
            P[name][pos] = orig - h
            dn = _np_objective(P, K, idx, alpha, **flags)
            P[name][pos] = orig
            fd = (up - dn) / (2 * h)
            assert abs(G[pos] - fd) <= 1e-7 * (1 + abs(fd)), (name, pos, G[pos], fd)


def test_b2_autograd():
    torch = pytest.importorskip("torch")
    for var in VARIANTS:
        L, K = _layer(31, T=20, d=12, E=8, I=6, K=3, Ks=2, Is=5)
        alpha = 0.3
        r = _oracle_all(L, K, alpha, **var)
        idx = torch.from_numpy(r["idx"].astype(np.int64))
        P = {k: torch.tensor(v.astype(np.float64) if k == "bias" else widen(v),
                             requires_grad=k not in ("dout", "bias"))
             for k, v in L.items() if v is not None}
        X, C = P["x"], P["C"]
        A = X @ C.T
        if var.get("sigmoid"):
            S = torch.sigmoid(A)
        else:
            S = torch.softmax(A + P["bias"], dim=1)
        G = torch.gather(S, 1, idx)
        if var.get("renorm"):
            G = G / G.sum(dim=1, keepdim=True)

        def ffn(Xs, w1, w3, w2):
            return (torch.nn.functional.silu(Xs @ w1.T) * (Xs @ w3.T)) @ w2.T

        out = torch.zeros_like(X) if var.get("no_residual") else X
        for s in range(P["ws1"].shape[0]):
            out = out + ffn(X, P["ws1"][s], P["ws3"][s], P["ws2"][s])
        for k in range(K):
            Y = torch.stack([ffn(X[t:t + 1], P["w1"][int(idx[t, k])], P["w3"][int(idx[t, k])],
                                 P["w2"][int(idx[t, k])])[0] for t in range(X.shape[0])])
            out = out + G[:, k:k + 1] * Y
        E = C.shape[0]
        f = torch.bincount(idx.ravel(), minlength=E).double() * E / (K * X.shape[0])
        obj = (P["dout"] * out).sum() + alpha * (f * S.mean(dim=0)).sum()
        obj.backward()
        for name, key in (("x", "dx"), ("C", "dC"), ("w1", "dw1"), ("w3", "dw3"), ("w2", "dw2"),
                          ("ws1", "dws1"), ("ws3", "dws3"), ("ws2", "dws2")):
            ref = P[name].grad.numpy()
            assert np.allclose(r[key], ref, rtol=1e-11, atol=1e-13), (var, name)


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_b3_closed_forms():
    # shared-only SwiGLU: x = (1, 0), Ws1 = [[1, 0]], Ws3 = [[2, 0]], Ws2 = [[1], [0.5]],
    # dout = (1, 0).  h = 2 silu(1); d Lambda / dh = <dout, (1, 0.5)> = 1.
    s1 = _sig(1.0)
    silu1 = s1
    dsilu1 = s1 * (1.0 + (1.0 - s1))
    bf = lambda v: _bf(np.array(v, np.float32))
    x = bf([[1, 0]])
    E0 = np.zeros((1, 2), np.uint16)
    z = np.zeros((1, 1, 2), np.uint16)
    r = oracle.backward(x, E0, None, z, z, np.zeros((1, 2, 1), np.uint16), bf([[[1, 0]]]),
                        bf([[[2, 0]]]), bf([[[1], [0.5]]]), 0, bf([[1, 0]]), want_shared=True)
    assert r["dx"][0] == pytest.approx([1 + 2 * dsilu1 + 2 * silu1, 0.0], rel=1e-15, abs=0)
    assert r["dws1"][0] == pytest.approx(np.array([[2 * dsilu1, 0.0]]), rel=1e-15, abs=0)
    assert r["dws3"][0] == pytest.approx(np.array([[silu1, 0.0]]), rel=1e-15, abs=0)
    assert r["dws2"][0] == pytest.approx(np.array([[2 * silu1], [0.0]]), rel=1e-15, abs=0)

    # two-expert softmax router, top-1: C = [[1, 0], [0, 0]] gives logits (1, 0)
    # and scores s0 = sig(1), s1 = 1 - sig(1); expert 0 is W1 = W3 = [[1, 0]],
    # W2 = [[1], [0]], so y = (silu(1), 0) and dgate = silu(1).
    s0, s1_ = _sig(1.0), 1.0 - _sig(1.0)
    C = bf([[1, 0], [0, 0]])
    w13 = bf([[[1, 0]], [[0, 0]]])
    w2 = bf([[[1], [0]], [[0], [0]]])
    r = oracle.backward(x, C, None, w13, w13, w2, None, None, None, 1, bf([[1, 0]]),
                        experts=[0, 1], want_dC=True)
    assert r["idx"][0, 0] == 0
    dg = silu1
    assert r["dgate"][0, 0] == pytest.approx(dg, rel=1e-15)
    dx0 = 1.0 + s0 * (dsilu1 + silu1) + s0 * s1_ * dg
    assert r["dx"][0] == pytest.approx([dx0, 0.0], rel=1e-14, abs=0)
    assert r["dC"] == pytest.approx(np.array([[s0 * s1_ * dg, 0], [-s0 * s1_ * dg, 0]]),
                                    rel=1e-14, abs=0)
    # dW1 = da x^T with da = s0 * silu'(1); dW3 = s0 * silu(1); dW2 = s0 * dout h^T
    assert r["dw1"][0] == pytest.approx(np.array([[s0 * dsilu1, 0]]), rel=1e-14, abs=0)
    assert r["dw3"][0] == pytest.approx(np.array([[s0 * silu1, 0]]), rel=1e-14, abs=0)
    assert r["dw2"][0] == pytest.approx(np.array([[s0 * silu1], [0]]), rel=1e-14, abs=0)
    assert not r["dw1"][1].any() and not r["dw2"][1].any()


def test_b4_balance_statistics():
    L, K = _layer(41, T=40, d=16, E=8, I=4, K=3)
    r = _oracle_all(L, K, 0.5)
    assert r["counts"].sum() == 40 * K
    f = 8 * r["counts"] / (K * 40)
    assert f.sum() == pytest.approx(8, rel=1e-15)
    assert r["mean_score"].sum() == pytest.approx(1.0, rel=1e-14)
    assert r["bal"] == pytest.approx(float((f * r["mean_score"]).sum()), rel=1e-14)
    assert r["bal_alpha"] == pytest.approx(0.5 * r["bal"], rel=1e-15)
    # zero centroids: every score 1/E, experts 0..K-1 take every token:
    # f = E/K on them, so L_bal = K * (E/K) * (1/E) = 1 exactly; with
    # dout = 0 the only gradient is the balance term's,
    # dl_j = (alpha / (E T)) (f_j - 1), so dC_j = dl_j * sum_t x_t and dx = 0
    T, E, alpha = 40, 8, 0.5
    L["C"] = np.zeros_like(L["C"])
    L["bias"] = None
    L["dout"] = np.zeros_like(L["dout"])
    r = _oracle_all(L, K, alpha)
    assert list(r["counts"]) == [T] * K + [0] * (E - K)
    assert r["bal"] == 1.0
    fj = np.array([E / K] * K + [0.0] * (E - K))
    dl = alpha / (E * T) * (fj - 1.0)
    xs = widen(L["x"]).sum(axis=0)
    assert r["dC"] == pytest.approx(dl[:, None] * xs[None, :], rel=1e-12, abs=1e-15)
    assert np.abs(r["dx"]).max() == 0.0


def test_b5_special_cases():
    L, K = _layer(51)
    Z = dict(L, dout=np.zeros_like(L["dout"]))
    r = _oracle_all(Z, K, 0.0)
    for k in ("dx", "dgate", "dw1", "dw3", "dw2", "dws1", "dws3", "dws2", "dC"):
        assert not np.any(r[k]), k
    W = dict(L, w2=np.zeros_like(L["w2"]), ws2=np.zeros_like(L["ws2"]))
    r = _oracle_all(W, K, 0.0)
    assert not r["dgate"].any() and not r["dw1"].any() and not r["dw3"].any()
    assert not r["dC"].any()
    assert np.array_equal(r["dx"], widen(L["dout"]))
    assert r["dw2"].any()                    # dW2 = g dout h^T is not zero
