"""Second, independent fp64 formulation of the layer in numpy, for small shapes.

TEST INFRASTRUCTURE (see the package docstring).  Written as whole-matrix
products instead of per-token loops so that it shares no structure with
oracle.c; the two are compared to 1e-12 relative.

Definition followed: the generic top-K gate of "DeepSeekMoE 深度解读报告"
section 3.1 (softmax of token-centroid inner products, top scores kept
unnormalised), fine-grained routed experts and always-on shared experts
(sections 2.2, 2.3), SwiGLU experts w2(silu(w1 x) * w3 x) (the youleyou
page's Expert module), plus the residual.  Gating variants: gates
renormalised over the selected experts (the eliteato DeepSeek-V2 explainer's
routing code, section 3.1) and sigmoid affinities whose bias only steers the
selection (the youleyou page's auxiliary-loss-free remark).
"""
from __future__ import annotations

import numpy as np


def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sigmoid_scores(X, C, bias):
    """Sigmoid gate: scores sigmoid(X C^T) and selection keys scores + bias
    (the bias steers the choice only)."""
    S = 1.0 / (1.0 + np.exp(-(X @ C.T)))
    keys = S if bias is None else S + np.asarray(bias, np.float64)[None, :]
    return S, keys


def softmax_scores(X, C, bias):
    L = X @ C.T
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    L = L - L.max(axis=1, keepdims=True)
    P = np.exp(L)
    return P / P.sum(axis=1, keepdims=True)


def topk(P, K):
    """Indices of the K largest scores per row, descending, ties to the lower
    expert index (a stable sort of the negated scores)."""
    order = np.argsort(-P, axis=1, kind="stable")
    return order[:, :K]


def swiglu(X, W1, W3, W2):
    A = X @ W1.T
    B = X @ W3.T
    Hh = (A / (1.0 + np.exp(-A))) * B
    return Hh @ W2.T


def forward(x, C, bias, w1, w3, w2, ws1, ws3, ws2, K, no_residual=False, forced_idx=None,
            renorm=False, sigmoid=False):
    X = widen(x)
    Cd = widen(C)
    if sigmoid:
        P, keys = sigmoid_scores(X, Cd, bias)
    else:
        P = softmax_scores(X, Cd, bias)
        keys = P
    idx = topk(keys, K) if forced_idx is None else np.asarray(forced_idx)
    T, d = X.shape
    E = Cd.shape[0]
    G = np.zeros((T, E))
    rows = np.arange(T)[:, None]
    gate = P[rows, idx]
    if renorm:
        gate = gate / gate.sum(axis=1, keepdims=True)
    G[rows, idx] = gate
    shared = np.zeros((T, d))
    for s in range(0 if ws1 is None else len(ws1)):
        shared += swiglu(X, widen(ws1[s]), widen(ws3[s]), widen(ws2[s]))
    routed = np.zeros((T, d))
    for e in range(E):
        sel = G[:, e] != 0
        if sel.any():
            routed[sel] += G[sel, e][:, None] * swiglu(X[sel], widen(w1[e]), widen(w3[e]), widen(w2[e]))
    out = (0.0 if no_residual else X) + shared + routed
    return dict(out=out, shared=shared, routed=routed, idx=idx.astype(np.int32), gate=gate, probs=P)
