"""The Python binding on the GPU: every malformed tensor is rejected before
anything is launched (the caller's output stays as it was), a forward on a
side stream is safe against allocations on the current stream, and exact
ties in the router resolve to the lower expert index on both router tiles."""
import numpy as np
import pytest

import synth

from helpers import bf16_bits, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import fine_grained_mixture_router_amd as moe  # noqa: E402


def _log(msg):
    print(msg, flush=True)


def _layer(T=96, d=128, E=8, I=64, Ks=1, seed=3):
    g = np.random.default_rng(seed)

    def r(shape, s):
        return to_dev(synth.f32_to_bf16_rne((g.standard_normal(shape) * s).astype(np.float32)))

    return dict(x=r((T, d), 1.0), C=r((E, d), 0.05), w1=r((E, I, d), 0.05),
                w3=r((E, I, d), 0.05), w2=r((E, d, I), 0.05), ws1=r((Ks, I, d), 0.05),
                ws3=r((Ks, I, d), 0.05), ws2=r((Ks, d, I), 0.05),
                bias=torch.zeros(E, dtype=torch.float32, device="cuda"))


def _args(D):
    return [D["x"], D["C"], D["w1"], D["w3"], D["w2"], D["ws1"], D["ws3"], D["ws2"]]


BAD = {
    "x dtype": lambda D: D.update(x=D["x"].float()),
    "x transposed view": lambda D: D.update(x=D["x"].t().contiguous().t()),
    "centroids rows": lambda D: D.update(C=D["C"][:-1].contiguous()),
    "centroids width": lambda D: D.update(C=torch.zeros(D["C"].shape[0], 64, dtype=torch.bfloat16,
                                                        device="cuda")),
    "w1 fewer experts": lambda D: D.update(w1=D["w1"][:-1].contiguous()),
    "w3 inter": lambda D: D.update(w3=D["w3"][:, :-64].contiguous() if D["w3"].shape[1] > 64
                                   else D["w3"][:, :, :64].contiguous()),
    "w2 transposed": lambda D: D.update(w2=D["w2"].transpose(1, 2)),
    "w2 on the host": lambda D: D.update(w2=D["w2"].cpu()),
    "ws2 shape": lambda D: D.update(ws2=D["ws2"][:, :-64].contiguous()),
    "bias length": lambda D: D.update(bias=D["bias"][:-1].contiguous()),
    "bias dtype": lambda D: D.update(bias=D["bias"].to(torch.bfloat16)),
}


@pytest.mark.parametrize("what", sorted(BAD))
def test_bad_tensor_is_rejected_before_launch(what):
    D = _layer()
    T, d = D["x"].shape
    out = torch.full((T, d), 7.0, dtype=torch.bfloat16, device="cuda")
    BAD[what](D)
    with pytest.raises(ValueError):
        moe.forward(*_args(D), K=2, bias=D["bias"], out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "output written despite the rejection"


def test_bad_outputs_are_rejected_before_launch():
    D = _layer()
    T, d = D["x"].shape
    for kw in (dict(out=torch.empty((T - 1, d), dtype=torch.bfloat16, device="cuda")),
               dict(topk_idx=torch.empty((T, 1), dtype=torch.int32, device="cuda")),
               dict(topk_gate=torch.empty((T, 2), dtype=torch.float64, device="cuda")),
               dict(workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))):
        with pytest.raises(ValueError):
            moe.forward(*_args(D), K=2, bias=D["bias"], **kw)
    with pytest.raises(ValueError):
        moe.route(D["x"], D["C"], K=2, topk_idx=torch.empty((T, 3), dtype=torch.int32,
                                                            device="cuda"))


def test_fp8_bad_scales_rejected():
    D = _layer()
    E, I, d = D["w1"].shape
    q = torch.zeros((E, I, d), dtype=torch.uint8, device="cuda")
    q2 = torch.zeros((E, d, I), dtype=torch.uint8, device="cuda")
    s = torch.ones((E, I), dtype=torch.float32, device="cuda")
    s2 = torch.ones((E, d), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        moe.forward_fp8(D["x"], D["C"], q, s[:, :-1].contiguous(), q, s, q2, s2, K=2)
    with pytest.raises(ValueError):
        moe.forward_fp8(D["x"], D["C"], q, s, q, s, q2, s, K=2)


def test_side_stream_forward_is_safe_against_current_stream_allocations():
    """forward(stream=side) allocates its workspace and outputs while another
    stream is current; allocations and writes on the current stream right
    after must not disturb it (the binding marks its allocations as used by
    the side stream).  The result must equal an ordinary run bit for bit."""
    D = _layer(T=4096, d=512, E=16, I=256)
    ref = moe.forward(*_args(D), K=4, bias=D["bias"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        out = moe.forward(*_args(D), K=4, bias=D["bias"], stream=side)
        outs.append(out)
        # churn the caching allocator on the current stream while side runs
        junk = [torch.full((1 << 22,), 1.0, device="cuda") for _ in range(8)]
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("T", [200, 8300], ids=["64-token tiles", "256-token tiles"])
def test_exact_ties_pick_lowest_ids(T):
    """Zero centroids make every score exactly 1/E: the top-K must be experts
    0..K-1 in order, each with gate 1/E (E a power of two, so exactly), for
    the default gate, and 1/K renormalised."""
    E, K, d = 64, 6, 256
    g = np.random.default_rng(1)
    x = to_dev(synth.f32_to_bf16_rne(g.standard_normal((T, d)).astype(np.float32)))
    C = torch.zeros((E, d), dtype=torch.bfloat16, device="cuda")
    _log(f"[ties] T={T}")
    idx, gate = moe.route(x, C, K=K)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), torch.arange(K, dtype=torch.int32).repeat(T, 1))
    assert bool((gate == 1.0 / E).all())
    idx, gate = moe.route(x, C, K=K, renorm=True)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), torch.arange(K, dtype=torch.int32).repeat(T, 1))
    assert torch.allclose(gate, torch.full_like(gate, 1.0 / K), rtol=1e-6, atol=0)
    # through the whole forward: zero centroids route every token to 0..K-1
    I = 64
    w = [to_dev(synth.f32_to_bf16_rne((g.standard_normal(s) * 0.05).astype(np.float32)))
         for s in ((E, I, d), (E, I, d), (E, d, I))]
    out, fidx, fgate = moe.forward(x, C, *w, K=K, return_routing=True)
    torch.cuda.synchronize()
    assert torch.equal(fidx.cpu(), torch.arange(K, dtype=torch.int32).repeat(T, 1))
    assert bool((fgate == 1.0 / E).all())
    assert np.isfinite(synth.bf16_to_f64(bf16_bits(out))).all()
