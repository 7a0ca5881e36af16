"""The token permutation on the GPU, checked directly: after a forward call,
the arrays moe_workspace_layout places in its workspace are read back and
compared, exactly, with what the routing the call returned implies.

The permutation gathers each expert's tokens after the top-K (eliteato.com
DeepSeek-V2 explainer, section 3.1); the checks:
  * goff: each routed expert's row count is its number of (token, choice)
    pairs, in expert order, then Ks groups of T rows;
  * tok_of / slot_of: a bijection between the T K (token, choice) pairs and
    the routed rows, each expert's rows holding its tokens in increasing
    order (so the row order does not depend on thread timing), and shared
    row goff[E + s] + t holding token t;
  * the two work lists: as sets, exactly one entry per (group with rows,
    tile of tile_rows rows, tile of tile_cols output columns), with the
    ragged row count of the group's last tile; nothing beyond ntiles is
    read, and ntiles stays within max_tiles.
Every case runs on both tile shapes the plan picks (32-row tiles for few rows
per expert, 256-row tiles otherwise) and on skewed loads."""
import numpy as np
import pytest

import synth
from synth import workloads as wl

from helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import fine_grained_mixture_router_amd as moe  # noqa: E402


def _log(msg):
    print(msg, flush=True)


def _rand_layer(seed, T, d, E, I, Ks, Is, bias_scale):
    rng = np.random.default_rng(seed)

    def r(shape, s):
        return synth.f32_to_bf16_rne((rng.standard_normal(shape) * s).astype(np.float32))

    L = dict(x=r((T, d), 1.0), C=r((E, d), 0.05), w1=r((E, I, d), 0.02), w3=r((E, I, d), 0.02),
             w2=r((E, d, I), 0.02), ws1=r((Ks, Is, d), 0.02), ws3=r((Ks, Is, d), 0.02),
             ws2=r((Ks, d, Is), 0.02),
             bias=(rng.standard_normal(E) * bias_scale).astype(np.float32))
    return L


def _read(ws, off, n, dtype):
    if n == 0:
        return np.zeros(0, dtype=np.int32)
    return ws[off:off + 4 * n].view(dtype).cpu().numpy()


def _expected_tiles(counts, Ks, T, bm, bn, ncols_r, ncols_s):
    out = set()
    for g, n in enumerate(list(counts) + [T] * Ks):
        ncols = ncols_r if g < len(counts) else ncols_s
        for m0 in range(0, n, bm):
            for n0 in range(0, ncols, bn):
                out.add((g, m0, n0, min(bm, n - m0)))
    return out


def _check(L, K, flags, what):
    T, d = L["x"].shape
    E, I = L["w1"].shape[0], L["w1"].shape[1]
    Ks = L["ws1"].shape[0]
    Is = L["ws1"].shape[1] if Ks else 0
    D = {k: to_dev(v) for k, v in L.items()}
    shape = moe.make_shape(T, d, E, I, K, Ks, Is, **flags)
    lay = moe.workspace_layout(shape)
    # filled with 0xFF bytes: every array read back below must have been written
    ws = torch.full((moe.workspace_size(shape),), 0xFF, dtype=torch.uint8, device="cuda")
    ws_args = (D["ws1"], D["ws3"], D["ws2"]) if Ks else (None, None, None)
    _, idx, _ = moe.forward(D["x"], D["C"], D["w1"], D["w3"], D["w2"], *ws_args, K=K,
                            bias=D["bias"], workspace=ws, return_routing=True, **flags)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    G = E + Ks
    rows = T * K + T * Ks
    assert lay["rows"] == rows

    # group offsets
    counts = np.bincount(idx.ravel(), minlength=E) if K else np.zeros(E, np.int64)
    goff = _read(ws, lay["goff"], G + 1, torch.int32)
    want = np.concatenate([[0], np.cumsum(np.r_[counts, np.full(Ks, T)])])
    assert np.array_equal(goff, want), f"{what}: goff"

    # tok_of / slot_of
    tok_of = _read(ws, lay["tok_of"], rows, torch.int32)
    slot_of = _read(ws, lay["slot_of"], T * K, torch.int32).reshape(T, K)
    if K:
        assert np.array_equal(np.sort(slot_of.ravel()), np.arange(T * K)), f"{what}: slot_of not a bijection"
        tt = np.repeat(np.arange(T), K).reshape(T, K)
        assert np.array_equal(tok_of[slot_of], tt), f"{what}: tok_of[slot_of] != token"
        grp = np.searchsorted(goff[:E + 1], slot_of, side="right") - 1
        assert np.array_equal(grp, idx), f"{what}: a row outside its expert's group"
        for e in np.nonzero(counts)[0]:
            toks = tok_of[goff[e]:goff[e + 1]]
            assert np.array_equal(toks, np.nonzero((idx == e).any(axis=1))[0]), \
                f"{what}: expert {e} rows not its tokens in increasing order"
    for s in range(Ks):
        assert np.array_equal(tok_of[goff[E + s]:goff[E + s + 1]], np.arange(T)), f"{what}: shared {s}"

    # work lists
    nt = _read(ws, lay["ntiles"], 2, torch.int32)
    for li, (key, bm, bn, ncr, ncs, mx) in enumerate([
            ("tiles_gate_up", lay["tile_rows_gate_up"], lay["tile_cols_gate_up"], I, Is,
             lay["max_tiles_gate_up"]),
            ("tiles_down", lay["tile_rows_down"], lay["tile_cols_down"], d, d, lay["max_tiles_down"])]):
        n = int(nt[li])
        assert 0 <= n <= mx, f"{what}: {key} count {n} beyond its bound {mx}"
        ent = _read(ws, lay[key], 4 * n, torch.int32).reshape(n, 4)
        got = [tuple(int(v) for v in r) for r in ent]
        exp = _expected_tiles(counts, Ks, T, bm, bn, ncr, ncs)
        assert len(got) == len(set(got)), f"{what}: {key} repeats an entry"
        assert set(got) == exp, f"{what}: {key} entries differ ({len(set(got) ^ exp)} of {len(exp)})"
    _log(f"[perm] {what}: T={T} E={E} K={K} Ks={Ks}, tiles {lay['tile_rows_gate_up']}-row, "
         f"lists {int(nt[0])} / {int(nt[1])}, max rows {counts.max() if K else 0}")


CASES = [
    # T, d, E, I, K, Ks, Is, bias scale (a large bias skews the load)
    (1, 64, 1, 64, 1, 0, 64, 0.0),
    (67, 576, 13, 192, 3, 2, 320, 0.5),
    (300, 256, 64, 128, 64, 1, 64, 0.0),          # K = E: every expert takes every token
    (129, 320, 200, 64, 8, 0, 64, 0.5),           # 200 experts (four 64-expert blocks)
    (700, 512, 5, 512, 1, 3, 128, 0.5),
    (2048, 256, 6, 128, 2, 2, 192, 1.5),          # 256-row tiles, strongly skewed, ragged
    (4100, 128, 16, 64, 4, 1, 64, 3.0),           # a ragged last chunk, few hot experts
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}E{c[2]}K{c[4]}Ks{c[5]}" for c in CASES])
@pytest.mark.parametrize("sigmoid", [False, True], ids=["softmax", "sigmoid"])
def test_permutation_edge_shapes(case, sigmoid):
    T, d, E, I, K, Ks, Is, bs = case
    L = _rand_layer(T + E, T, d, E, I, Ks, Is, bs)
    _check(L, K, dict(sigmoid=sigmoid, renorm=sigmoid), f"T{T} E{E} K{K}")


@pytest.mark.parametrize("name", ["tiny", "2b", "16b_zipf"])
def test_permutation_workloads(name):
    w = wl.WORKLOADS[name]
    L = wl.gen_all(w)
    if L.get("bias") is None:
        L["bias"] = np.zeros(w.E, np.float32)
    _check(L, w.K, {}, name)


def test_permutation_shared_only():
    """K = 0: no routed rows, the shared groups alone."""
    L = _rand_layer(9, 200, 128, 4, 64, 2, 64, 0.0)
    D = {k: to_dev(v) for k, v in L.items()}
    shape = moe.make_shape(200, 128, 1, 64, 0, 2, 64)   # the binding's shape without routed experts
    lay = moe.workspace_layout(shape)
    # filled with 0xFF bytes: every array read back below must have been written
    ws = torch.full((moe.workspace_size(shape),), 0xFF, dtype=torch.uint8, device="cuda")
    moe.forward(D["x"], None, None, None, None, D["ws1"], D["ws3"], D["ws2"], K=0, workspace=ws)
    torch.cuda.synchronize()
    goff = _read(ws, lay["goff"], 1 + 2 + 1, torch.int32)
    assert np.array_equal(goff, [0, 0, 200, 400])
    tok_of = _read(ws, lay["tok_of"], 400, torch.int32)
    assert np.array_equal(tok_of, np.r_[np.arange(200), np.arange(200)])
