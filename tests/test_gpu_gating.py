"""Parity of the two gating variants on the GPU (flags MOE_FLAG_RENORM and
MOE_FLAG_SIGMOID, alone and together) against the fp64 oracle run with the
same variant: routing of every token, and the layer output, its
residual-free delta under the GPU's own routing, and run-to-run identity on
token samples."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl

from helpers import (bf16_bits, check_close, check_part, check_routing, gpu_forward, out_f64,
                     upload)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import fine_grained_mixture_router_amd as moe  # noqa: E402

VARIANTS = {"renorm": dict(renorm=True), "sigmoid": dict(sigmoid=True),
            "sigmoid_renorm": dict(sigmoid=True, renorm=True)}


def _log(msg):
    print(msg, flush=True)


def _bias(w, seed):
    """The workload's own bias, or (for unbiased workloads) a small seeded one
    that moves the sigmoid gate's choices without dominating them."""
    b = wl.gen_bias(w)
    if b is not None:
        return b
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(w.E) * 0.02).astype(np.float32)


def _keys(x, C, b, K, ref_idx, sigmoid, **kw):
    """The oracle's selection keys of its chosen experts, in order."""
    _, _, _, probs = oracle.route(x, C, b, K, return_probs=True, sigmoid=sigmoid, **kw)
    rows = np.arange(ref_idx.shape[0])[:, None]
    keys = probs[rows, ref_idx]
    if sigmoid and b is not None:
        keys = keys + b.astype(np.float64)[ref_idx]
    return keys


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", ["tiny", "2b", "16b_zipf"])
def test_route_variant(name, variant):
    w = wl.WORKLOADS[name]
    kw = VARIANTS[variant]
    _log(f"[gating] route {name} {variant}")
    x, C, b = wl.gen_x(w), wl.gen_centroids(w), _bias(w, w.T)
    D = upload({"x": x, "C": C, "bias": b})
    idx, gate = moe.route(D["x"], D["C"], K=w.K, bias=D["bias"], **kw)
    torch.cuda.synchronize()
    ri, rg, rm = oracle.route(x, C, b, w.K, **kw)
    keys = _keys(x, C, b, w.K, ri, **{"sigmoid": False, **kw})
    gi, gg = idx.cpu().numpy(), gate.cpu().numpy()
    exempt = check_routing(gi, gg, ri, rg, rm, w.K, ref_keys=keys)
    assert exempt < 0.1 * w.T
    if kw.get("renorm"):
        assert np.allclose(gg.sum(axis=1), 1.0, rtol=0, atol=1e-5)
    # a rerun in a routing scratch of 0xFF bytes is bit-identical
    shape = moe.make_shape(w.T, w.d, w.E, 64, w.K, **kw)
    junk = torch.full((moe.route_workspace_size(shape),), 0xFF, dtype=torch.uint8, device="cuda")
    idx2, gate2 = moe.route(D["x"], D["C"], K=w.K, bias=D["bias"], workspace=junk, **kw)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(gate2, gate)


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name,nsample", [("2b", 96), ("16b_zipf", 96)])
def test_forward_variant(name, nsample, variant):
    w = wl.WORKLOADS[name]
    kw = VARIANTS[variant]
    _log(f"[gating] forward {name} {variant}")
    L = wl.gen_all(w)
    L["bias"] = _bias(w, w.T)
    D = upload(L)
    out, idx, gate = gpu_forward(D, w.K, **kw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.T + 1)
    tok = np.unique(np.r_[0, rng.choice(w.T, nsample, replace=False), w.T - 1])
    ref = oracle.forward(L["x"][tok], L["C"], L["bias"], L["w1"], L["w3"], L["w2"], L["ws1"],
                         L["ws3"], L["ws2"], w.K, **kw)
    gi, gg = idx.cpu().numpy()[tok], gate.cpu().numpy()[tok]
    keys = _keys(L["x"][tok], L["C"], L["bias"], w.K, ref["idx"], **{"sigmoid": False, **kw})
    check_routing(gi, gg, ref["idx"], ref["gate"], ref["margin"], w.K, ref_keys=keys)
    check_close(synth.bf16_to_f64(bf16_bits(out)[tok]), ref["out"])

    dout, didx, _ = gpu_forward(D, w.K, no_residual=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(didx, idx)
    dref = oracle.forward(L["x"][tok], L["C"], L["bias"], L["w1"], L["w3"], L["w2"], L["ws1"],
                          L["ws3"], L["ws2"], w.K, no_residual=True, forced_idx=gi, **kw)
    check_part(out_f64(dout)[tok], dref["out"], "delta")

    # a rerun in a workspace of 0xFF bytes is bit-identical
    shape = moe.make_shape(w.T, w.d, w.E, w.I, w.K, w.Ks, w.Is, **kw)
    junk = torch.full((moe.workspace_size(shape),), 0xFF, dtype=torch.uint8, device="cuda")
    out2, idx2, gate2 = gpu_forward(D, w.K, workspace=junk, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(idx2, idx) and torch.equal(gate2, gate)


def test_sigmoid_bias_steers_selection_only():
    """On the GPU too: a bias that reorders the choice leaves the chosen
    experts' gates at their unbiased sigmoid scores."""
    w = wl.WORKLOADS["tiny"]
    x, C = wl.gen_x(w), wl.gen_centroids(w)
    rng = np.random.default_rng(3)
    b = rng.permutation(w.E).astype(np.float32)    # gaps of 1 > any spread of sigmoid scores
    D = upload({"x": x, "C": C, "bias": b})
    idx, gate = moe.route(D["x"], D["C"], K=w.K, bias=D["bias"], sigmoid=True)
    torch.cuda.synchronize()
    gi, gg = idx.cpu().numpy(), gate.cpu().numpy()
    want = np.argsort(-b.astype(np.float64), kind="stable")[: w.K]
    # every token picks the same K experts, in bias order
    assert all(row.tolist() == want.tolist() for row in gi)
    _, _, _, probs = oracle.route(x, C, b, w.K, return_probs=True, sigmoid=True)
    ref = probs[np.arange(w.T)[:, None], gi]
    assert np.allclose(gg, ref, rtol=1e-5, atol=1e-7)
