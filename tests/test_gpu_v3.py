"""Parity at the full DeepSeek-V3 layer shape (d=7168, 256 routed + 1 shared
experts of inter 2048, top-8), in the launch configuration the benchmark
times: the 256-token decode batch and the 16384-token prefill batch with its
Zipf(1.2) logit bias.  Routing is checked for every token.  The layer output
and its residual-free delta are checked on every token of the decode batch,
and on the prefill batches on tokens chosen so that every (group, 256-row
M-tile) of the GEMM work lists holds a checked row, each group's ragged last
tile included (its routed part alone is covered at the smaller shapes, where
it is cheap to run the layer without its shared expert)."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl

from helpers import (bf16_bits, check_close, check_part, check_rounding, check_routing,
                     out_f64, tile_cover_tokens, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import fine_grained_mixture_router_amd as moe  # noqa: E402


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def v3_layer():
    """Host and device copies of the V3-shape weights (shared by both batches)."""
    w = wl.WORKLOADS["v3_decode"]
    _log("[v3] generating the 22.6 GB layer")
    H = {"C": wl.gen_centroids(w)}
    H["w1"], H["w3"], H["w2"] = wl.gen_routed(w)
    H["ws1"], H["ws3"], H["ws2"] = wl.gen_shared(w)
    D = {k: to_dev(v) for k, v in H.items()}
    torch.cuda.synchronize()
    _log("[v3] uploaded")
    yield H, D
    del D
    torch.cuda.empty_cache()


# The last case is the prefill batch cut to 12 345 tokens: a ragged last
# token tile of the 256-token router tile, and ragged row tiles everywhere.
@pytest.mark.parametrize("name,T", [("v3_decode", None), ("v3_prefill", None),
                                    ("v3_prefill", 12345)])
def test_v3_parity(v3_layer, name, T):
    H, D = v3_layer
    w = wl.WORKLOADS[name]
    _log(f"[v3] {name} T={T or w.T}")
    x = wl.gen_x(w)
    if T is not None:
        x = np.ascontiguousarray(x[:T])
    bias = wl.gen_bias(w)
    xd, bd = to_dev(x), to_dev(bias)

    def run(**kw):
        return moe.forward(xd, D["C"], D["w1"], D["w3"], D["w2"], D["ws1"], D["ws3"], D["ws2"],
                           K=w.K, bias=bd, return_routing=True, **kw)

    out, idx, gate = run()
    torch.cuda.synchronize()
    gi_all, gg_all = idx.cpu().numpy(), gate.cpu().numpy()

    # routing of every token
    ri, rg, rm = oracle.route(x, H["C"], bias, w.K)
    exempt = check_routing(gi_all, gg_all, ri, rg, rm, w.K)
    _log(f"[v3] {name}: routing ok, {exempt} near-tie tokens exempt")
    nt = x.shape[0]
    assert exempt < 0.1 * nt

    if name == "v3_decode":
        tok = np.arange(nt)
    else:
        tok = tile_cover_tokens(gi_all, w.E, w.Ks, nt)
        _log(f"[v3] {name}: checking {tok.size} tokens, one per (group, M-tile)")
    ref = oracle.forward(x[tok], H["C"], bias, H["w1"], H["w3"], H["w2"], H["ws1"], H["ws3"],
                         H["ws2"], w.K)
    ob = bf16_bits(out)[tok]
    check_close(synth.bf16_to_f64(ob), ref["out"])
    check_rounding(ob, ref["out"], ref["shared"], ref["routed"], ref["margin"])

    dout, didx, _ = run(no_residual=True)
    torch.cuda.synchronize()
    assert torch.equal(didx, idx)
    dref = oracle.forward(x[tok], H["C"], bias, H["w1"], H["w3"], H["w2"], H["ws1"], H["ws3"],
                          H["ws2"], w.K, no_residual=True, forced_idx=gi_all[tok])
    check_part(out_f64(dout)[tok], dref["out"], "delta")

    # determinism at full size, the rerun in a workspace of 0xFF bytes
    shape = moe.make_shape(nt, w.d, w.E, w.I, w.K, w.Ks, w.Is)
    junk = torch.full((moe.workspace_size(shape),), 0xFF, dtype=torch.uint8, device="cuda")
    out2, idx2, _ = run(workspace=junk)
    del junk
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(idx2, idx)


@pytest.mark.parametrize("name", ["v3_decode", "v3_prefill"])
def test_v3_backward(v3_layer, name):
    """The backward at the full V3 shape, through moe_forward_train and
    moe_backward, against the fp64 backward oracle under the GPU's routing:
    decode — every token's input and gate gradients, the centroid gradient,
    the weight gradients of three experts and of the shared expert; prefill —
    input and gate gradients of tokens that put a checked row in every
    (group, M-tile) of the dH / dX work lists, and the weight gradients of a
    middling and the smallest touched expert (the busiest one holds every
    token: its fp64 reference would take minutes)."""
    from helpers import check_grad
    H, D = v3_layer
    w = wl.WORKLOADS[name]
    _log(f"[v3-bwd] {name}")
    x = wl.gen_x(w)
    bias = wl.gen_bias(w)
    dout = wl.gen_dout(w)
    xd, bd, dod = to_dev(x), to_dev(bias), to_dev(dout)
    args = (xd, D["C"], D["w1"], D["w3"], D["w2"], D["ws1"], D["ws3"], D["ws2"])
    out, st, idx = moe.forward_train(*args, K=w.K, bias=bd, return_routing=True)[:3]
    g = moe.backward(*args, dout=dod, state=st, return_dgate=True)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    counts = np.bincount(gi.ravel(), minlength=w.E)
    touched = np.nonzero(counts)[0]
    order = touched[np.argsort(-counts[touched], kind="stable")]
    if name == "v3_decode":
        tok = np.arange(w.T)
        experts = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
        want_shared = want_dC = True
    else:
        tok = tile_cover_tokens(gi, w.E, w.Ks, w.T)
        experts = sorted({int(order[len(order) // 2]), int(order[-1])})
        want_shared = want_dC = False
    _log(f"[v3-bwd] {name}: oracle on {tok.size} tokens, experts {experts} "
         f"({[int(counts[e]) for e in experts]} rows)")
    ref = oracle.backward(x, H["C"], bias, H["w1"], H["w3"], H["w2"], H["ws1"], H["ws3"],
                          H["ws2"], w.K, dout, tokens=tok, experts=experts,
                          want_shared=want_shared, want_dC=want_dC, forced_idx=gi)

    def f64(t):
        return out_f64(t) if t.dtype == torch.bfloat16 else t.double().cpu().numpy()

    msg = [f"dx {check_grad(f64(g['dx'])[tok], ref['dx'], 'dx'):.2e}",
           f"dgate {check_grad(f64(g['dgate'])[tok], ref['dgate'], 'dgate'):.2e}"]
    sel = torch.as_tensor(np.asarray(experts, dtype=np.int64), device="cuda")
    for nm in ("dw1", "dw3", "dw2"):
        msg.append(f"{nm} {check_grad(f64(g[nm][sel]), ref[nm], nm):.2e}")
    if want_shared:
        for nm in ("dws1", "dws3", "dws2"):
            msg.append(f"{nm} {check_grad(f64(g[nm]), ref[nm], nm):.2e}")
    if want_dC:
        msg.append(f"dC {check_grad(f64(g['dC']), ref['dC'], 'dC'):.2e}")
    _log(f"[v3-bwd] {name}: max|err|/max|ref| " + ", ".join(msg))
    # untouched experts get exact zeros
    untouched = np.nonzero(counts == 0)[0]
    if untouched.size:
        u = torch.as_tensor(untouched, device="cuda")
        for nm in ("dw1", "dw3", "dw2"):
            assert not bool((g[nm][u] != 0).any())
    # a rerun in a workspace of 0xFF bytes, into NaN-filled outputs, is
    # bit-identical: every gradient element of every expert is written and
    # nothing relies on a cleared workspace
    junk = torch.full((moe.backward_workspace_size(st.shape),), 0xFF, dtype=torch.uint8,
                      device="cuda")
    outs = {}
    for k, v in g.items():
        if v is not None:
            o = torch.empty_like(v)
            if o.dtype == torch.bfloat16:
                o.view(torch.int16).fill_(0x7FC0)
            else:
                o.fill_(float("nan"))
            outs[k] = o
    g2 = moe.backward(*args, dout=dod, state=st, workspace=junk, **outs)
    torch.cuda.synchronize()
    for k, v in g.items():
        if v is not None:
            bits = (lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32))
            assert torch.equal(bits(v), bits(g2[k])), k
    del g, g2, outs, junk, st
    torch.cuda.empty_cache()
