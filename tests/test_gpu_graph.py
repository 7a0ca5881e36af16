"""The layer forward captured in a HIP graph (torch.cuda.CUDAGraph).

The forward launches only kernels on the caller's stream (no allocation, no
memset, no synchronisation), so it can be captured and replayed.  Each
replay must reproduce the eager result bit for bit; replays alternate with
eager work on the same buffers and with synchronisation, and an input
changed in place between replays is picked up by the next replay.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import fine_grained_mixture_router_amd as moe  # noqa: E402  (fails loudly if unbuilt)
from synth import workloads as wl  # noqa: E402

from helpers import upload  # noqa: E402


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


# the few-rows tile (tiny) and the many-rows ring tile (16b_zipf), with bf16
# or 8-bit routed weights, and with 8-bit activations (the quantisation
# kernels and, on 16b_zipf, the FP8 tiles)
@pytest.mark.parametrize("name,fp8,act8", [("tiny", False, False), ("16b_zipf", False, False),
                                           ("tiny", True, False), ("16b_zipf", True, False),
                                           ("tiny", True, True), ("16b_zipf", True, True)])
def test_graph_replay_matches_eager(name, fp8, act8):
    w = wl.WORKLOADS[name]
    print(f"[graph] {name} fp8={fp8} act8={act8}", flush=True)
    D = upload(wl.gen_all(w))
    if fp8:
        for k, a in zip(("q1", "s1", "q3", "s3", "q2", "s2"), wl.gen_routed_fp8(w)):
            D[k] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    shape = moe.make_shape(w.T, w.d, w.E, w.I, w.K, w.Ks, w.Is, act8=act8)
    ws = torch.empty(moe.workspace_size(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    gate = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")

    def fwd(**kw):
        if fp8:
            return moe.forward_fp8(D["x"], D["C"], D["q1"], D["s1"], D["q3"], D["s3"], D["q2"],
                                   D["s2"], D["ws1"], D["ws3"], D["ws2"], K=w.K, bias=D["bias"],
                                   act8=act8, **kw)
        return moe.forward(D["x"], D["C"], D["w1"], D["w3"], D["w2"], D["ws1"], D["ws3"], D["ws2"],
                           K=w.K, bias=D["bias"], **kw)

    def run():
        fwd(out=out, topk_idx=idx, topk_gate=gate, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = [out.clone(), idx.clone(), gate.clone()]

    side = torch.cuda.Stream()                       # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()

    for rep in range(3):
        out.zero_()                                  # eager work on the same buffers
        idx.fill_(-1)
        gate.zero_()
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, idx, gate), ref):
            assert torch.equal(_bits(got), _bits(want)), f"replay {rep}"

    # a new batch written into the captured input buffer
    D["x"].copy_(torch.roll(D["x"], shifts=1, dims=0))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    want, widx, wgate = fwd(return_routing=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(want))
    assert torch.equal(idx, widx) and torch.equal(gate, wgate)
    # the rolled batch is the old one with its rows moved by one
    assert torch.equal(_bits(out), _bits(torch.roll(ref[0], shifts=1, dims=0)))
