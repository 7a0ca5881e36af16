"""The 8-bit routed-weight path (moe_forward_fp8) on the GPU.

Exact probes first: one-hot tokens, a SwiGLU whose gate saturates (silu(448)
= 448 in fp32) and power-of-two scales make every output an exact bf16
multiple of one decoded E4M3 code, so the GPU must reproduce the decode of
all 254 finite codes bit for bit, through the down weights and through the
up weights (and the gate weights to bf16 rounding).  Then parity against
the fp64 oracle's 8-bit path on seeded layers, at the V3 decode shape, on
edge shapes, and run-to-run identity."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl

from helpers import (bf16_bits, check_close, check_part, check_rounding, check_routing, out_f64,
                     tile_cover_tokens)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import fine_grained_mixture_router_amd as moe  # noqa: E402

E4M3 = np.array([oracle.e4m3(c) for c in range(256)])

CODE_1 = 0x38          # 1.0
CODE_448 = 0x7E        # 448, the largest finite value


def _log(msg):
    print(msg, flush=True)


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def _codes_under_test(rows):
    """codes[r, t] = r + 64 t for t < 4 (every code once), NaN codes -> 0."""
    c = (np.arange(rows)[:, None] + 64 * np.arange(4)[None, :]).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0
    return c


def _probe_inputs(d=64, I=64):
    T = 4
    x = np.zeros((T, d), np.float32)
    x[np.arange(T), np.arange(T)] = 1.0                  # token t = e_t
    return dict(x=synth.f32_to_bf16_rne(x), C=np.zeros((1, d), np.uint16))


def _run(P, q1, s1, q3, s3, q2, s2):
    out = moe.forward_fp8(dev(P["x"]), dev(P["C"]), dev(q1[None]), dev(s1[None]), dev(q3[None]),
                          dev(s3[None]), dev(q2[None]), dev(s2[None]), K=1, no_residual=True)
    torch.cuda.synchronize()
    return out_f64(out)


def test_down_weight_codes_decode_exactly():
    d = I = 64
    P = _probe_inputs(d, I)
    q1 = np.full((I, d), CODE_448, np.uint8)             # a_i = 448 -> silu = 448
    q3 = np.zeros((I, d), np.uint8)
    q3[np.arange(4), np.arange(4)] = CODE_1              # b_i = 2^-9 [i == t]
    s1 = np.ones(I, np.float32)
    s3 = np.full(I, 2.0 ** -9, np.float32)               # h = 0.875 e_t, exact in bf16
    q2 = np.zeros((d, I), np.uint8)
    codes = _codes_under_test(d)
    q2[:, :4] = codes                                    # y_o(t) = W2[o, t] * 0.875
    s2 = np.full(d, 2.0 ** -4, np.float32)
    got = _run(P, q1, s1, q3, s3, q2, s2)
    want = np.array([[oracle.e4m3(codes[o, t]) * 0.875 / 16 for o in range(d)] for t in range(4)])
    assert np.array_equal(got, want)


def test_up_weight_codes_decode_exactly():
    d = I = 64
    P = _probe_inputs(d, I)
    q1 = np.full((I, d), CODE_448, np.uint8)
    s1 = np.ones(I, np.float32)
    q3 = np.zeros((I, d), np.uint8)
    codes = _codes_under_test(I)
    q3[:, :4] = codes                                    # b_i(t) = W3[i, t]
    s3 = np.full(I, 2.0 ** -9, np.float32)               # h_i = 0.875 e4m3(code)
    q2 = np.zeros((d, I), np.uint8)
    q2[np.arange(I), np.arange(I)] = CODE_1              # W2 = identity
    s2 = np.ones(d, np.float32)
    got = _run(P, q1, s1, q3, s3, q2, s2)
    want = np.array([[oracle.e4m3(codes[o, t]) * 0.875 for o in range(d)] for t in range(4)])
    assert np.array_equal(got, want)


def test_gate_weight_codes_decode():
    d = I = 64
    P = _probe_inputs(d, I)
    q1 = np.zeros((I, d), np.uint8)
    codes = _codes_under_test(I)
    q1[:, :4] = codes                                    # a_i(t) = W1[i, t]
    s1 = np.ones(I, np.float32)
    q3 = np.full((I, d), CODE_1, np.uint8)               # b_i = 1
    s3 = np.ones(I, np.float32)
    q2 = np.zeros((d, I), np.uint8)
    q2[np.arange(I), np.arange(I)] = CODE_1
    s2 = np.ones(d, np.float32)
    got = _run(P, q1, s1, q3, s3, q2, s2)
    v = np.array([[oracle.e4m3(codes[o, t]) for o in range(d)] for t in range(4)])
    want = v / (1.0 + np.exp(-v))                        # silu, then bf16 H and out
    assert np.all(np.abs(got - want) <= 2.0 ** -7 * np.abs(want) + 1e-30)


def _fp8_layer(w):
    L = dict(x=wl.gen_x(w), C=wl.gen_centroids(w), bias=wl.gen_bias(w))
    L["ws1"], L["ws3"], L["ws2"] = wl.gen_shared(w)
    L["q1"], L["s1"], L["q3"], L["s3"], L["q2"], L["s2"] = wl.gen_routed_fp8(w)
    return L


def _upload(L):
    return {k: (None if v is None else dev(v)) for k, v in L.items()}


def _gpu(D, K, Ks=None, **kw):
    ws = (None, None, None) if Ks == 0 else (D["ws1"], D["ws3"], D["ws2"])
    return moe.forward_fp8(D["x"], D["C"], D["q1"], D["s1"], D["q3"], D["s3"], D["q2"], D["s2"],
                           *ws, K=K, bias=D.get("bias"), return_routing=True, **kw)


def _junk_ws(w, act8=False):
    """A workspace filled with 0xFF bytes: a rerun in it must match the first
    run bit for bit, so no kernel relies on a cleared workspace."""
    shape = moe.make_shape(w.T, w.d, w.E, w.I, w.K, w.Ks, w.Is, act8=act8)
    return torch.full((moe.workspace_size(shape),), 0xFF, dtype=torch.uint8, device="cuda")


def _rerun_in_junk(D, w, K, out, idx, act8=False, **kw):
    """The same call again in a workspace of 0xFF bytes, into a NaN-filled
    output: bit-identical."""
    shape = moe.make_shape(w.T, w.d, w.E, w.I, K, w.Ks, w.Is, act8=act8, **kw)
    ws = torch.full((moe.workspace_size(shape),), 0xFF, dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(out)
    o2.view(torch.int16).fill_(0x7FC0)
    out2, idx2, _ = _gpu(D, K, act8=act8, workspace=ws, out=o2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(idx2, idx)


def _ref(L, K, tok, Ks=None, **kw):
    ws = (L["ws1"][:0], L["ws3"][:0], L["ws2"][:0]) if Ks == 0 else (L["ws1"], L["ws3"], L["ws2"])
    return oracle.forward_fp8(L["x"][tok], L["C"], L["bias"], L["q1"], L["s1"], L["q3"], L["s3"],
                              L["q2"], L["s2"], *ws, K, **kw)


@pytest.mark.parametrize("name,nsample", [("tiny", 128), ("2b", 128), ("16b_zipf", 96)])
def test_fp8_layer_parity(name, nsample):
    w = wl.WORKLOADS[name]
    _log(f"[fp8] {name}")
    L = _fp8_layer(w)
    D = _upload(L)
    out, idx, gate = _gpu(D, w.K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.T + 7)
    tok = np.unique(np.r_[0, rng.choice(w.T, min(nsample, w.T), replace=False), w.T - 1])
    ref = _ref(L, w.K, tok)
    gi, gg = idx.cpu().numpy()[tok], gate.cpu().numpy()[tok]
    check_routing(gi, gg, ref["idx"], ref["gate"], ref["margin"], w.K)
    ob = bf16_bits(out)[tok]
    check_close(synth.bf16_to_f64(ob), ref["out"])
    check_rounding(ob, ref["out"], ref["shared"], ref["routed"], ref["margin"])

    dout, didx, _ = _gpu(D, w.K, no_residual=True)
    torch.cuda.synchronize()
    assert torch.equal(didx, idx)
    dref = _ref(L, w.K, tok, no_residual=True, forced_idx=gi)
    check_part(out_f64(dout)[tok], dref["out"], "delta")

    rout, ridx, _ = _gpu(D, w.K, Ks=0, no_residual=True)
    torch.cuda.synchronize()
    rref = _ref(L, w.K, tok, Ks=0, no_residual=True, forced_idx=ridx.cpu().numpy()[tok])
    check_part(out_f64(rout)[tok], rref["routed"], "routed")

    out2, idx2, gate2 = _gpu(D, w.K, workspace=_junk_ws(w))
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(idx2, idx) and torch.equal(gate2, gate)


@pytest.mark.parametrize("case", [
    (1, 64, 1, 64, 1, 0, 64, False),
    (67, 576, 13, 192, 3, 2, 320, True),
    (300, 256, 64, 128, 64, 1, 64, False),
    (700, 1024, 5, 512, 1, 3, 128, True),
], ids=lambda c: "T%dd%dE%dI%dK%dKs%dIs%d" % c[:7])
def test_fp8_edge_shapes(case):
    T, d, E, I, K, Ks, Is, bias = case
    _log(f"[fp8] edge {case}")
    w = wl.Workload("edge", T=T, d=d, E=E, I=I, K=K, Ks=Ks, Is=Is, wseed=T + d, xseed=T + E)
    L = _fp8_layer(w)
    if bias:
        L["bias"] = (np.random.default_rng(T).standard_normal(E) * 0.5).astype(np.float32)
    D = _upload(L)
    dout, idx, _ = _gpu(D, K, no_residual=True)
    torch.cuda.synchronize()
    tok = np.unique(np.r_[0, np.random.default_rng(d).choice(T, min(T, 48), replace=False), T - 1])
    ref = _ref(L, K, tok, no_residual=True, forced_idx=idx.cpu().numpy()[tok])
    check_part(out_f64(dout)[tok], ref["out"], "delta")
    _rerun_in_junk(D, w, K, dout, idx, no_residual=True)


def test_fp8_v3_decode_shape():
    """The DeepSeek-V3-shape layer (256 routed experts of 7168 x 2048) on the
    256-token decode batch, with 8-bit routed weights (11.3 GB of codes)."""
    w = wl.WORKLOADS["v3_decode"]
    _log("[fp8] v3_decode: generating 8-bit routed weights")
    L = _fp8_layer(w)
    D = _upload(L)
    _log("[fp8] v3_decode: uploaded")
    out, idx, gate = _gpu(D, w.K)
    torch.cuda.synchronize()
    ri, rg, rm = oracle.route(L["x"], L["C"], L["bias"], w.K)
    check_routing(idx.cpu().numpy(), gate.cpu().numpy(), ri, rg, rm, w.K)
    tok = np.arange(w.T)                      # every token: each expert's one tile
    ref = _ref(L, w.K, tok)
    ob = bf16_bits(out)[tok]
    check_close(synth.bf16_to_f64(ob), ref["out"])
    check_rounding(ob, ref["out"], ref["shared"], ref["routed"], ref["margin"])
    dout, _, _ = _gpu(D, w.K, no_residual=True)
    torch.cuda.synchronize()
    dref = _ref(L, w.K, tok, no_residual=True, forced_idx=idx.cpu().numpy()[tok])
    check_part(out_f64(dout)[tok], dref["out"], "delta")
    del D
    torch.cuda.empty_cache()


def test_fp8_v3_prefill_shape():
    """The V3-shape prefill batch (16384 tokens, Zipf(1.2) bias) with 8-bit
    routed weights: the 256 x 256 tiles of the 8-bit kernel, shared-expert
    tiles in bf16 within the same launch; routing of every token, the output
    and its delta on tokens that put a checked row in every (group, M-tile)
    of the work lists."""
    w = wl.WORKLOADS["v3_prefill"]
    _log("[fp8] v3_prefill: generating inputs")
    L = _fp8_layer(w)
    D = _upload(L)
    _log("[fp8] v3_prefill: uploaded")
    out, idx, gate = _gpu(D, w.K)
    torch.cuda.synchronize()
    ri, rg, rm = oracle.route(L["x"], L["C"], L["bias"], w.K)
    exempt = check_routing(idx.cpu().numpy(), gate.cpu().numpy(), ri, rg, rm, w.K)
    assert exempt < 0.1 * w.T
    tok = tile_cover_tokens(idx.cpu().numpy(), w.E, w.Ks, w.T)
    _log(f"[fp8] v3_prefill: checking {tok.size} tokens, one per (group, M-tile)")
    ref = _ref(L, w.K, tok)
    ob = bf16_bits(out)[tok]
    check_close(synth.bf16_to_f64(ob), ref["out"])
    check_rounding(ob, ref["out"], ref["shared"], ref["routed"], ref["margin"])
    dout, _, _ = _gpu(D, w.K, no_residual=True)
    torch.cuda.synchronize()
    dref = _ref(L, w.K, tok, no_residual=True, forced_idx=idx.cpu().numpy()[tok])
    check_part(out_f64(dout)[tok], dref["out"], "delta")
    out2, _, _ = _gpu(D, w.K)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    del D
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,nsample", [("tiny", 96), ("16b_zipf", 96)])
def test_fp8_v3_style_gate(name, nsample):
    """8-bit routed weights under the V3-style gate (sigmoid affinities, a
    selection-only bias, renormalised gates): the router is shared with the
    bf16 path, so this checks that the 8-bit GEMMs take its gates as given."""
    w = wl.WORKLOADS[name]
    kw = dict(renorm=True, sigmoid=True)
    _log(f"[fp8] {name} sigmoid+renorm")
    L = _fp8_layer(w)
    L["bias"] = (np.random.default_rng(w.T + 3).standard_normal(w.E) * 0.02).astype(np.float32)
    D = _upload(L)
    out, idx, gate = _gpu(D, w.K, **kw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.T + 11)
    tok = np.unique(np.r_[0, rng.choice(w.T, min(nsample, w.T), replace=False), w.T - 1])
    ref = _ref(L, w.K, tok, **kw)
    gi, gg = idx.cpu().numpy()[tok], gate.cpu().numpy()[tok]
    # selection keys of the sigmoid gate: score + bias
    _, _, _, probs = oracle.route(L["x"][tok], L["C"], L["bias"], w.K, return_probs=True, **kw)
    rows = np.arange(len(tok))[:, None]
    keys = probs[rows, ref["idx"]] + L["bias"].astype(np.float64)[ref["idx"]]
    check_routing(gi, gg, ref["idx"], ref["gate"], ref["margin"], w.K, ref_keys=keys)
    check_close(synth.bf16_to_f64(bf16_bits(out)[tok]), ref["out"])
    dout, didx, _ = _gpu(D, w.K, no_residual=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(didx, idx)
    dref = _ref(L, w.K, tok, no_residual=True, forced_idx=gi, **kw)
    check_part(out_f64(dout)[tok], dref["out"], "delta")


# ---------------------------------------------------------------------------
# 8-bit activations (MOE_FLAG_ACT8): the routed gate/up products on the FP8
# matrix cores (256-row tiles) or, for decode-size batches, on the bf16 tile
# fed the dequantised rows.
# ---------------------------------------------------------------------------

def _act8_codes(D, L, K, shape_kw):
    """Run the 8-bit forward with a workspace of our own and read back the
    activation codes and exponents it wrote."""
    T, d = L["x"].shape
    E, I = L["q1"].shape[0], L["q1"].shape[1]
    Ks = L["ws1"].shape[0]
    shape = moe.make_shape(T, d, E, I, K, Ks, L["ws1"].shape[1] if Ks else 0, act8=True, **shape_kw)
    lay = moe.workspace_layout(shape)
    ws = torch.empty(moe.workspace_size(shape), dtype=torch.uint8, device="cuda")
    out, idx, gate = _gpu(D, K, act8=True, workspace=ws, **shape_kw)
    torch.cuda.synchronize()
    codes = ws[lay["act8_codes"]:lay["act8_codes"] + T * d].cpu().numpy().reshape(T, d)
    exps = ws[lay["act8_exps"]:lay["act8_exps"] + 4 * T].view(torch.int32).cpu().numpy()
    return out, idx, gate, codes, exps


@pytest.mark.parametrize("name", ["tiny", "2b"])
def test_act8_codes_bit_exact(name):
    """Every activation code and exponent equals the oracle's (an integer
    decision: bit-exact), on rows of every magnitude, an all-zero row and
    a row of bf16 subnormals."""
    w = wl.WORKLOADS[name]
    _log(f"[fp8] act8 codes {name}")
    L = _fp8_layer(w)
    rng = np.random.default_rng(11)
    x = synth.bf16_to_f64(L["x"]) * np.exp(rng.uniform(-12, 12, (w.T, 1)))
    x[1] = 0.0
    x[2] = x[2] * 2.0 ** -130                       # subnormal row
    L["x"] = synth.f32_to_bf16_rne(x.astype(np.float32))
    D = _upload(L)
    _, _, _, codes, exps = _act8_codes(D, L, w.K, {})
    rc, re_ = oracle.quantize_act8(L["x"])
    assert np.array_equal(exps, re_)
    assert np.array_equal(codes, rc)


@pytest.mark.parametrize("name", ["tiny", "2b", "16b_zipf"])
def test_act8_h_codes(name):
    """The down projection's 8-bit input: on the FP8 down tiles (2B, 16B)
    every code and exponent of h's routed rows equals the oracle's
    quantisation of the bf16 h the call left in its workspace (bit-exact);
    on the decode-size tiles (tiny) h is replaced by its dequantised rows,
    which the quantisation maps back to themselves exactly."""
    w = wl.WORKLOADS[name]
    _log(f"[fp8] act8 h codes {name}")
    L = _fp8_layer(w)
    D = _upload(L)
    T, d, K, I = w.T, w.d, w.K, w.I
    shape = moe.make_shape(T, d, w.E, I, K, w.Ks, w.Is, act8=True)
    lay = moe.workspace_layout(shape)
    ws = torch.empty(moe.workspace_size(shape), dtype=torch.uint8, device="cuda")
    _gpu(D, K, act8=True, workspace=ws)
    torch.cuda.synchronize()
    h = ws[lay["h"]:lay["h"] + T * K * I * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(T * K, I)
    if lay["act8_h_codes"]:
        codes = ws[lay["act8_h_codes"]:lay["act8_h_codes"] + T * K * I].cpu().numpy().reshape(T * K, I)
        exps = ws[lay["act8_h_exps"]:lay["act8_h_exps"] + 4 * T * K].view(torch.int32).cpu().numpy()
        rc, re_ = oracle.quantize_act8(h)
        assert np.array_equal(exps, re_)
        assert np.array_equal(codes, rc)
        assert (exps != 0).any() and (codes != 0).any()
    else:
        assert name == "tiny"
        rc, re_ = oracle.quantize_act8(h)
        deq = E4M3[rc] * np.ldexp(1.0, re_)[:, None]
        assert np.array_equal(deq, synth.bf16_to_f64(h))


@pytest.mark.parametrize("name,nsample", [("tiny", 128), ("2b", 96), ("16b_zipf", 96)])
def test_act8_layer_parity(name, nsample):
    """The layer with 8-bit activations against the oracle's ACT8 layer:
    routing, output and the residual-free delta under the GPU's routing
    (tiny takes the decode-size tiles, 2B and 16B the FP8 256-row tiles)."""
    w = wl.WORKLOADS[name]
    _log(f"[fp8] act8 {name}")
    L = _fp8_layer(w)
    D = _upload(L)
    out, idx, gate = _gpu(D, w.K, act8=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.T + 9)
    tok = np.unique(np.r_[0, rng.choice(w.T, min(nsample, w.T), replace=False), w.T - 1])
    ref = _ref(L, w.K, tok, act8=True)
    gi, gg = idx.cpu().numpy()[tok], gate.cpu().numpy()[tok]
    check_routing(gi, gg, ref["idx"], ref["gate"], ref["margin"], w.K)
    ob = bf16_bits(out)[tok]
    check_close(synth.bf16_to_f64(ob), ref["out"])
    dout, didx, _ = _gpu(D, w.K, act8=True, no_residual=True)
    torch.cuda.synchronize()
    assert torch.equal(didx, idx)
    dref = _ref(L, w.K, tok, act8=True, no_residual=True, forced_idx=gi)
    check_part(out_f64(dout)[tok], dref["out"], "delta")
    rout, ridx, _ = _gpu(D, w.K, Ks=0, act8=True, no_residual=True)
    torch.cuda.synchronize()
    rref = _ref(L, w.K, tok, Ks=0, act8=True, no_residual=True, forced_idx=ridx.cpu().numpy()[tok])
    check_part(out_f64(rout)[tok], rref["routed"], "routed")
    out2, _, _ = _gpu(D, w.K, act8=True, workspace=_junk_ws(w, act8=True))
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny", "2b"])
def test_act8_v3_style_gate(name):
    """8-bit activations under the V3-style gate (sigmoid scores, the bias in
    the selection only, renormalised gates): routing, the residual-free
    delta under the GPU's routing, and the full output against the oracle."""
    w = wl.WORKLOADS[name]
    _log(f"[fp8] act8 sigmoid+renorm {name}")
    L = _fp8_layer(w)
    if L.get("bias") is None:
        L["bias"] = (np.random.default_rng(w.T).standard_normal(w.E) * 0.5).astype(np.float32)
    D = _upload(L)
    kw = dict(act8=True, sigmoid=True, renorm=True)
    out, idx, gate = _gpu(D, w.K, **kw)
    torch.cuda.synchronize()
    tok = np.unique(np.r_[0, np.random.default_rng(w.T + 3).choice(w.T, min(96, w.T), replace=False), w.T - 1])
    ref = _ref(L, w.K, tok, **kw)
    gi, gg = idx.cpu().numpy()[tok], gate.cpu().numpy()[tok]
    check_routing(gi, gg, ref["idx"], ref["gate"], ref["margin"], w.K)
    check_close(synth.bf16_to_f64(bf16_bits(out)[tok]), ref["out"])
    dout, _, _ = _gpu(D, w.K, no_residual=True, **kw)
    torch.cuda.synchronize()
    dref = _ref(L, w.K, tok, no_residual=True, forced_idx=gi, **kw)
    check_part(out_f64(dout)[tok], dref["out"], "delta")


@pytest.mark.parametrize("case", [
    (67, 576, 13, 192, 3, 2, 320),
    (700, 1024, 5, 512, 1, 3, 128),
    (2048, 256, 6, 128, 2, 1, 192),
    (2048, 320, 4, 192, 2, 1, 192),   # 256-row tiles with d, I not multiples of 128: dequantised rows
    (1, 128, 4, 128, 4, 1, 64),       # one token, every expert
], ids=lambda c: "T%dd%dE%dI%dK%dKs%dIs%d" % c)
def test_act8_edge_shapes(case):
    T, d, E, I, K, Ks, Is = case
    _log(f"[fp8] act8 edge {case}")
    w = wl.Workload("edge", T=T, d=d, E=E, I=I, K=K, Ks=Ks, Is=Is, wseed=T + d, xseed=T + E)
    L = _fp8_layer(w)
    D = _upload(L)
    dout, idx, _ = _gpu(D, K, act8=True, no_residual=True)
    torch.cuda.synchronize()
    tok = np.unique(np.r_[0, np.random.default_rng(d).choice(T, min(T, 64), replace=False), T - 1])
    ref = _ref(L, K, tok, act8=True, no_residual=True, forced_idx=idx.cpu().numpy()[tok])
    check_part(out_f64(dout)[tok], ref["out"], "delta")
    _rerun_in_junk(D, w, K, dout, idx, act8=True, no_residual=True)


def test_act8_v3_prefill_shape():
    """The V3-shape prefill batch with 8-bit weights and activations: routing
    of every token, and the output on tokens that put a checked row in every
    (group, 256-row tile) of the gate/up work list."""
    w = wl.WORKLOADS["v3_prefill"]
    _log("[fp8] act8 v3_prefill: generating inputs")
    L = _fp8_layer(w)
    D = _upload(L)
    out, idx, gate = _gpu(D, w.K, act8=True)
    torch.cuda.synchronize()
    ri, rg, rm = oracle.route(L["x"], L["C"], L["bias"], w.K)
    check_routing(idx.cpu().numpy(), gate.cpu().numpy(), ri, rg, rm, w.K)
    tok = tile_cover_tokens(idx.cpu().numpy(), w.E, w.Ks, w.T)
    _log(f"[fp8] act8 v3_prefill: checking {tok.size} tokens")
    dout, _, _ = _gpu(D, w.K, act8=True, no_residual=True)
    torch.cuda.synchronize()
    dref = _ref(L, w.K, tok, act8=True, no_residual=True, forced_idx=idx.cpu().numpy()[tok])
    check_part(out_f64(dout)[tok], dref["out"], "delta")
    ob = bf16_bits(out)[tok]
    check_close(synth.bf16_to_f64(ob), dref["out"] + synth.bf16_to_f64(L["x"][tok]))
    del D
    torch.cuda.empty_cache()
