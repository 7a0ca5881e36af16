"""moe_forward_noalloc (the forward whose workspace is the library's static
scratch array) against moe_forward, through the C ABI: bit-identical
outputs and routing on two calls in a row, the second with a smaller batch
(the scratch keeps the first call's contents), no device allocation by the
call, and shapes beyond the scratch rejected before launch."""
import ctypes

import numpy as np
import pytest

import synth

from helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import fine_grained_mixture_router_amd as moe  # noqa: E402


def _layer(T, d, E, I, Ks, seed):
    g = np.random.default_rng(seed)

    def r(shape, s):
        return to_dev(synth.f32_to_bf16_rne((g.standard_normal(shape) * s).astype(np.float32)))

    return dict(x=r((T, d), 1.0), C=r((E, d), 0.05), w1=r((E, I, d), 0.03), w3=r((E, I, d), 0.03),
                w2=r((E, d, I), 0.03), ws1=r((Ks, I, d), 0.03), ws3=r((Ks, I, d), 0.03),
                ws2=r((Ks, d, I), 0.03),
                bias=to_dev((g.standard_normal(E) * 0.3).astype(np.float32)))


def _args(D):
    return [D["x"], D["C"], D["w1"], D["w3"], D["w2"], D["ws1"], D["ws3"], D["ws2"]]


# first a batch with many rows per expert (the 256 x 256 tiles), then a
# smaller one with few rows per expert (the 32-row tiles)
CASES = [(2048, 512, 16, 256, 4, 1), (100, 256, 24, 128, 6, 2)]


def test_noalloc_matches_forward_on_consecutive_calls():
    for i, (T, d, E, I, K, Ks) in enumerate(CASES):
        print(f"[noalloc] call {i}: T={T} d={d} E={E} I={I} K={K} Ks={Ks}", flush=True)
        D = _layer(T, d, E, I, Ks, seed=40 + i)
        shape = moe.make_shape(T, d, E, I, K, Ks, I)
        assert moe.workspace_size(shape) <= moe.noalloc_scratch_bytes()
        ref, ridx, rgate = moe.forward(*_args(D), K=K, bias=D["bias"], return_routing=True)
        out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        moe.forward_noalloc(*_args(D), K=K, bias=D["bias"], out=out, topk_idx=idx,
                            topk_gate=gate)
        assert torch.cuda.memory_allocated() == before
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(idx, ridx) and torch.equal(gate, rgate)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    D = _layer(64, 128, 8, 64, 1, seed=7)
    big = moe.make_shape(16384, 7168, 256, 2048, 8, 1, 2048)
    assert moe.workspace_size(big) > moe.noalloc_scratch_bytes()
    out = torch.full((64, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    vp = ctypes.c_void_p
    p = [vp(t.data_ptr()) for t in _args(D)]
    code = moe.lib().moe_forward_noalloc(ctypes.byref(big), p[0], p[1], None, p[2], p[3], p[4],
                                         p[5], p[6], p[7], vp(out.data_ptr()), None, None, None)
    assert code == 8 and moe.status_string(code).startswith("MOE_ERR_SCRATCH")
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
