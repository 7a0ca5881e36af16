"""Parameter / MAC accounting of one SwiGLU expert, the segmentation
equal-cost identity, and the expert-hit entropy diagnostic.

TEST INFRASTRUCTURE (see the package docstring).

expert_cost follows the counting convention of the ptflops printout on the
youleyou page ("DeepSeek MoE模型优化与未来演进及字节超稀疏内存技术", the
Expert(dim=7168, inter_dim=2048) cost over a 256-token batch):
  - a Linear(in, out, bias) has in*out (+ out) parameters and costs
    T*in*out (+ T*out for the bias) multiply-accumulates;
  - the element-wise part of the expert counts one operation per
    intermediate element (T*inter), which is what makes the printed module
    share come out at 99.995 %.

hit_entropy is the load diagnostic of the DeepSeek-V2 explainer page
(eliteato.com, section 6): entropy of the per-expert hit distribution and the
fraction of experts hit at least once.
"""
from __future__ import annotations

import math

import numpy as np


def linear_cost(fan_in: int, fan_out: int, tokens: int, bias: bool):
    params = fan_in * fan_out + (fan_out if bias else 0)
    macs = tokens * fan_in * fan_out + (tokens * fan_out if bias else 0)
    return params, macs


def expert_cost(dim: int, inter: int, tokens: int, bias: bool = False) -> dict:
    """Exact integer counts for one expert w2(silu(w1 x) * w3 x)."""
    p1, m1 = linear_cost(dim, inter, tokens, bias)
    p2, m2 = linear_cost(inter, dim, tokens, bias)
    p3, m3 = linear_cost(dim, inter, tokens, bias)
    params = p1 + p2 + p3
    module_macs = m1 + m2 + m3
    elementwise = tokens * inter
    total = module_macs + elementwise
    return dict(params=params, w1_params=p1, w2_params=p2, w3_params=p3,
                w1_macs=m1, w2_macs=m2, w3_macs=m3, module_macs=module_macs,
                elementwise_macs=elementwise, total_macs=total)


def ptflops_lines(c: dict) -> dict:
    """The rounded strings a ptflops per-layer printout shows for these counts."""
    tot_p, tot_m = c["params"], c["total_macs"]

    def m(v):
        return f"{v / 1e6:.2f} M"

    def g(v):
        return f"{v / 1e9:.2f} GMac"

    def pct(a, b):
        return f"{100.0 * a / b:.3f}%"

    out = {"expert": (m(tot_p), pct(tot_p, tot_p), g(tot_m), pct(c["module_macs"], tot_m))}
    for name in ("w1", "w2", "w3"):
        out[name] = (m(c[name + "_params"]), pct(c[name + "_params"], tot_p),
                     g(c[name + "_macs"]), pct(c[name + "_macs"], tot_m))
    return out


def layer_cost(E: int, inter: int, K: int, Ks: int, Is: int, dim: int) -> dict:
    """Bias-free parameter count of a layer's experts and per-token expert
    MACs (router excluded)."""
    per = expert_cost(dim, inter, 1, False)
    per_s = expert_cost(dim, Is, 1, False) if Ks else None
    params = E * per["params"] + (Ks * per_s["params"] if Ks else 0)
    macs = K * per["module_macs"] + (Ks * per_s["module_macs"] if Ks else 0)
    return dict(params=params, token_macs=macs)


def hit_entropy(idx: np.ndarray, E: int):
    """(entropy, active_ratio, counts) of the expert hits in idx."""
    counts = np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.float64)
    tot = counts.sum()
    p = counts[counts > 0] / tot
    ent = float(-(p * np.log(p)).sum())
    return ent, float((counts > 0).mean()), counts


def max_entropy(E: int) -> float:
    return math.log(E)
