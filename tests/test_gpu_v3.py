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

    # determinism at full size
    out2, idx2, _ = run()
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(idx2, idx)
