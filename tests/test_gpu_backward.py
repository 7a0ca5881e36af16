"""The training side on the GPU against the fp64 backward oracle
(oracle.backward): moe_forward_train then moe_backward through the C ABI.

The oracle runs under the GPU's own routing (forced_idx), so near-tie
choices cannot make the two differ; everything else — gates, scores, the
balance statistics, every gradient — the oracle recomputes itself.  Each
gradient tensor is held to helpers.check_grad (max |err| <= 2e-2 max|ref|,
RMS(err) <= 1e-2 RMS), the bars a CPU emulation of the backward's bf16
rounding points pins (test_part_tolerance.py)."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl

from helpers import check_grad, out_f64, tile_cover_tokens, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import fine_grained_mixture_router_amd as moe  # noqa: E402


def _log(msg):
    print(msg, flush=True)


def _f64(t):
    return out_f64(t) if t.dtype == torch.bfloat16 else t.detach().double().cpu().numpy()


def _nan_like(t):
    o = torch.empty_like(t)
    if o.dtype == torch.bfloat16:
        o.view(torch.int16).fill_(0x7FC0)           # a bf16 NaN
    else:
        o.fill_(float("nan"))
    return o


def _run(L, K, alpha=0.0, **flags):
    D = {k: to_dev(v) for k, v in L.items() if v is not None}
    ws = (D["ws1"], D["ws3"], D["ws2"]) if L["ws1"] is not None and len(L["ws1"]) else (None,) * 3
    args = (D["x"], D.get("C"), D.get("w1"), D.get("w3"), D.get("w2")) + ws
    out, st, idx, gate, stats = moe.forward_train(*args, K=K, bias=D.get("bias"),
                                                  return_routing=True, return_stats=True, **flags)
    ref_out = moe.forward(*args, K=K, bias=D.get("bias"), **flags)
    g = moe.backward(*args, dout=D["dout"], state=st, alpha=alpha, return_dgate=K > 0)
    # the second backward starts from a training forward into a state buffer
    # of 0xFF bytes, works in a workspace of 0xFF bytes and writes into
    # outputs filled with NaN, so the bit-equality below also shows that
    # nothing relies on cleared state or workspace and that every element of
    # every output (each expert's weight gradients, computed or zero) is written
    junk_state = torch.full((moe.train_state_size(st.shape),), 0xFF, dtype=torch.uint8,
                            device="cuda")
    _, stj = moe.forward_train(*args, K=K, bias=D.get("bias"), state=junk_state, **flags)
    junk = torch.full((moe.backward_workspace_size(st.shape),), 0xFF, dtype=torch.uint8,
                      device="cuda")
    g2 = moe.backward(*args, dout=D["dout"], state=stj, alpha=alpha, return_dgate=K > 0,
                      workspace=junk, **{k: _nan_like(v) for k, v in g.items() if v is not None})
    torch.cuda.synchronize()
    # the training forward is the forward; the backward is deterministic
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    for k, v in g.items():
        if v is not None:
            assert torch.equal(v.view(torch.int32) if v.dtype == torch.float32 else v.view(torch.int16),
                               g2[k].view(torch.int32) if v.dtype == torch.float32
                               else g2[k].view(torch.int16)), k
    return out, idx, gate, stats, g


def _oracle(L, K, idx, alpha, tokens=None, experts=(), want_shared=True, want_dC=True, **flags):
    ws = (L["ws1"], L["ws3"], L["ws2"]) if L["ws1"] is not None and len(L["ws1"]) else (None,) * 3
    return oracle.backward(L["x"], L["C"], L.get("bias"), L["w1"], L["w3"], L["w2"], *ws, K,
                           L["dout"], alpha=alpha, tokens=tokens, experts=experts,
                           want_shared=want_shared, want_dC=want_dC, forced_idx=idx, **flags)


def _compare(g, ref, tok, experts, K, Ks, want_dC=True, what=""):
    r = check_grad(_f64(g["dx"])[tok], ref["dx"], what + "dx")
    msg = [f"dx {r:.2e}"]
    if K > 0:
        r = check_grad(_f64(g["dgate"])[tok], ref["dgate"], what + "dgate")
        msg.append(f"dgate {r:.2e}")
        for name in ("dw1", "dw3", "dw2"):
            if len(experts):
                sel = torch.as_tensor(np.asarray(experts, dtype=np.int64), device=g[name].device)
                got = _f64(g[name][sel])
                r = check_grad(got, ref[name], what + name)
                msg.append(f"{name} {r:.2e}")
        if want_dC:
            r = check_grad(_f64(g["dC"]), ref["dC"], what + "dC")
            msg.append(f"dC {r:.2e}")
    if Ks > 0 and ref["dws1"] is not None:
        for name in ("dws1", "dws3", "dws2"):
            r = check_grad(_f64(g[name]), ref[name], what + name)
            msg.append(f"{name} {r:.2e}")
    _log(f"[bwd] {what}max|err|/RMS: " + ", ".join(msg))


def _with_dout(L, w):
    L = dict(L)
    L["dout"] = wl.gen_dout(w, L["x"].shape[0])
    return L


VARIANTS = [("softmax", dict(), 0.0), ("renorm", dict(renorm=True), 0.0),
            ("sigmoid-renorm", dict(sigmoid=True, renorm=True), 0.0),
            ("softmax-balance", dict(), 0.01), ("no-residual", dict(no_residual=True), 0.0)]


@pytest.mark.parametrize("var", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_backward_tiny_every_output(var):
    """The tiny layer: every token, every expert, the shared expert and dC."""
    name, flags, alpha = var
    w = wl.WORKLOADS["tiny"]
    L = _with_dout(wl.gen_all(w), w)
    _log(f"[bwd] tiny {name}")
    out, idx, gate, stats, g = _run(L, w.K, alpha, **flags)
    gi = idx.cpu().numpy()
    ref = _oracle(L, w.K, gi, alpha, experts=range(w.E), **flags)
    _compare(g, ref, np.arange(w.T), list(range(w.E)), w.K, w.Ks)
    # balance statistics of the training forward
    f, P, Lb = (s.cpu().numpy() for s in stats)
    assert np.array_equal(np.round(f.astype(np.float64) * w.K * w.T / w.E), ref["counts"])
    assert np.allclose(P, ref["mean_score"], rtol=1e-5, atol=1e-7)
    assert abs(float(Lb) - ref["bal"]) <= 1e-5 * abs(ref["bal"])


@pytest.mark.parametrize("name,ntok,flags,want_dC", [("2b", 96, dict(), True),
                                                     ("16b_zipf", 64, dict(renorm=True), False),
                                                     ("16b", 64, dict(no_residual=True), False)])
def test_backward_mid_shapes(name, ntok, flags, want_dC):
    """The 2B and 16B layers (the latter with and without its Zipf load skew):
    dx and gate gradients of sampled tokens, dW of the busiest, a middling and
    the idlest touched experts, the shared experts and dC."""
    w = wl.WORKLOADS[name]
    L = _with_dout(wl.gen_all(w), w)
    _log(f"[bwd] {name}")
    out, idx, gate, stats, g = _run(L, w.K, 0.0, **flags)
    gi = idx.cpu().numpy()
    counts = np.bincount(gi.ravel(), minlength=w.E)
    touched = np.nonzero(counts)[0]
    order = touched[np.argsort(-counts[touched], kind="stable")]
    experts = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    untouched = np.nonzero(counts == 0)[0]
    rng = np.random.default_rng(w.T)
    tok = np.unique(np.r_[0, rng.choice(w.T, ntok, replace=False), w.T - 1])
    ref = _oracle(L, w.K, gi, 0.0, tokens=tok, experts=experts, want_dC=want_dC, **flags)
    _compare(g, ref, tok, experts, w.K, w.Ks, want_dC=want_dC, what=f"{name} ")
    if untouched.size:                        # experts no token chose get zero gradients
        for nm in ("dw1", "dw3", "dw2"):
            assert not bool(g[nm][torch.from_numpy(untouched).cuda()].float().abs().max() > 0)


def _rand_layer(seed, T, d, E, I, K, Ks, Is, sc=0.05, bias_scale=0.0):
    rng = np.random.default_rng(seed)

    def r(shape, s):
        return synth.f32_to_bf16_rne((rng.standard_normal(shape) * s).astype(np.float32))

    L = dict(x=r((T, d), 1.0), C=r((E, d), 0.05), w1=r((E, I, d), sc), w3=r((E, I, d), sc),
             w2=r((E, d, I), sc), ws1=r((Ks, Is, d), sc), ws3=r((Ks, Is, d), sc),
             ws2=r((Ks, d, Is), sc), dout=r((T, d), 1.0),
             bias=(rng.standard_normal(E) * bias_scale).astype(np.float32) if bias_scale else None)
    return L


EDGE = [
    # T, d, E, I, K, Ks, Is, bias — ragged N tiles (I = 192, Is = 320, d = 576),
    # expert counts not multiples of 64, one token, top-1, K = E
    (1, 64, 1, 64, 1, 0, 64, 0.0),
    (67, 576, 13, 192, 3, 2, 320, 0.5),
    (300, 256, 64, 128, 64, 1, 64, 0.0),
    (129, 320, 200, 64, 8, 0, 64, 0.5),
    (700, 512, 5, 512, 1, 3, 128, 0.5),
    # many rows per group, strongly skewed: ragged 256-row tiles of many sizes
    (2048, 256, 6, 128, 2, 2, 192, 1.5),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"T{c[0]}d{c[1]}E{c[2]}I{c[3]}K{c[4]}Ks{c[5]}Is{c[6]}"
                                            for c in EDGE])
def test_backward_edge_shapes(case):
    T, d, E, I, K, Ks, Is, bs = case
    _log(f"[bwd] edge {case}")
    L = _rand_layer(hash(case) % 1000, T, d, E, I, K, Ks, Is, bias_scale=bs)
    if Ks == 0:
        L["ws1"] = L["ws3"] = L["ws2"] = None
    out, idx, gate, stats, g = _run(L, K, 0.02)
    gi = idx.cpu().numpy()
    tok = np.arange(T) if T <= 300 else np.unique(np.r_[np.arange(0, T, 7), T - 1])
    experts = list(range(E)) if E <= 16 else [0, E // 2, E - 1]
    ref = _oracle(L, K, gi, 0.02, tokens=tok, experts=experts, want_shared=Ks > 0)
    _compare(g, ref, tok, experts, K, Ks, what="edge ")


def test_backward_shared_only():
    """K = 0: no router; dx = dout + the shared experts' input gradient."""
    T, d, I, Ks = 200, 256, 128, 2
    L = _rand_layer(5, T, d, 4, I, 0, Ks, I)
    D = {k: to_dev(v) for k, v in L.items() if v is not None}
    out, st = moe.forward_train(D["x"], None, None, None, None, D["ws1"], D["ws3"], D["ws2"], K=0)
    g = moe.backward(D["x"], None, None, None, None, D["ws1"], D["ws3"], D["ws2"], dout=D["dout"],
                     state=st)
    torch.cuda.synchronize()
    assert g["dw1"] is None and g["dC"] is None
    ref = oracle.backward(L["x"], L["C"][:1], None, L["w1"][:1], L["w3"][:1], L["w2"][:1],
                          L["ws1"], L["ws3"], L["ws2"], 0, L["dout"], want_shared=True)
    _compare(g, ref, np.arange(T), [], 0, Ks, what="shared-only ")
