"""Pins of the oracle's 8-bit routed-weight path: the OCP FP8 E4M3 decode
(the format's defining facts, monotonicity, sign symmetry, exactness in
bf16) and the whole layer with 8-bit routed weights against the bf16 layer
when the two hold the same real weights (power-of-two row scales make
decode(q) * scale exact in bf16, so both oracles see identical values and
must agree to the last bit)."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl

E4M3 = np.array([oracle.e4m3(c) for c in range(256)])


def test_format_facts():
    """OCP FP8 E4M3: exponent bias 7, three mantissa bits, no infinities,
    NaN only at S.1111.111, largest finite 448, smallest normal 2^-6,
    smallest subnormal 2^-9."""
    assert E4M3[0x00] == 0.0 and E4M3[0x80] == 0.0 and np.signbit(E4M3[0x80])
    assert E4M3[0x38] == 1.0                       # exponent field 7 = bias
    assert E4M3[0x7E] == 448.0 and E4M3[0xFE] == -448.0
    assert E4M3[0x08] == 2.0 ** -6                 # smallest normal
    assert E4M3[0x01] == 2.0 ** -9                 # smallest subnormal
    assert E4M3[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert np.isnan(E4M3[0x7F]) and np.isnan(E4M3[0xFF])
    assert np.isfinite(E4M3).sum() == 254
    assert E4M3[0x3C] == 1.5 and E4M3[0x30] == 0.5 and E4M3[0x40] == 2.0


def test_monotone_symmetric_and_evenly_spaced():
    pos = E4M3[:0x7F]
    assert np.all(np.diff(pos) > 0)                # codes 0x00..0x7E increase
    assert np.array_equal(E4M3[0x80:0xFF], -pos)   # sign bit negates
    for e in range(1, 16):                         # 8 evenly spaced values per binade
        vals = pos[e * 8: min(e * 8 + 8, 0x7F)]
        assert np.allclose(np.diff(vals), 2.0 ** (e - 10), rtol=0, atol=0)
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9, rtol=0, atol=0)   # subnormals and the first normal


def test_every_finite_value_is_exact_in_bf16():
    fin = E4M3[np.isfinite(E4M3)]
    back = synth.bf16_to_f64(synth.f32_to_bf16_rne(fin.astype(np.float32)))
    assert np.array_equal(back, fin)


def _layer(seed, T=24, d=128, E=8, I=64, Ks=1):
    w = wl.Workload("t", T=T, d=d, E=E, I=I, K=3, Ks=Ks, Is=I, wseed=seed, xseed=seed)
    rng = np.random.default_rng(seed)
    q1, _, q3, _, q2, _ = wl.gen_routed_fp8(w)
    # per-row power-of-two scales, different on every row
    pw = lambda *s: np.ldexp(1.0, -rng.integers(6, 14, size=s)).astype(np.float32)
    s1, s3, s2 = pw(E, I), pw(E, I), pw(E, d)
    L = dict(x=wl.gen_x(w), C=wl.gen_centroids(w), q1=q1, q3=q3, q2=q2, s1=s1, s3=s3, s2=s2)
    L["ws1"], L["ws3"], L["ws2"] = wl.gen_shared(w)
    L["bias"] = (rng.standard_normal(E) * 0.05).astype(np.float32)

    def real(q, sc):                               # decode(q) * scale, exactly, as bf16
        v = E4M3[q] * sc.astype(np.float64)[..., None]
        bits = synth.f32_to_bf16_rne(v.astype(np.float32))
        assert np.array_equal(synth.bf16_to_f64(bits), v)
        return bits
    L["w1"], L["w3"], L["w2"] = real(q1, s1), real(q3, s3), real(q2, s2)
    return w, L


@pytest.mark.parametrize("kw", [{}, dict(renorm=True), dict(sigmoid=True, renorm=True),
                                dict(no_residual=True)])
def test_fp8_layer_equals_bf16_layer_holding_the_same_weights(kw):
    w, L = _layer(21)
    a = oracle.forward(L["x"], L["C"], L["bias"], L["w1"], L["w3"], L["w2"], L["ws1"], L["ws3"],
                       L["ws2"], w.K, **kw)
    b = oracle.forward_fp8(L["x"], L["C"], L["bias"], L["q1"], L["s1"], L["q3"], L["s3"],
                           L["q2"], L["s2"], L["ws1"], L["ws3"], L["ws2"], w.K, **kw)
    for k in ("out", "routed", "shared", "gate", "margin"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["idx"], b["idx"])


def test_down_scale_acts_on_its_output_row():
    """Doubling the W2 scale of output row o of one expert doubles exactly that
    column of the expert's routed contribution and leaves the rest."""
    w, L = _layer(22, E=4, Ks=0)
    forced = np.tile(np.array([[2, 0, 1]], np.int32), (w.T, 1))
    base = oracle.forward_fp8(L["x"], L["C"], None, L["q1"], L["s1"], L["q3"], L["s3"], L["q2"],
                              L["s2"], None, None, None, 3, no_residual=True, forced_idx=forced)
    s2 = L["s2"].copy()
    o = 17
    s2[2, o] *= 2
    mod = oracle.forward_fp8(L["x"], L["C"], None, L["q1"], L["s1"], L["q3"], L["s3"], L["q2"], s2,
                             None, None, None, 3, no_residual=True, forced_idx=forced)
    diff = mod["routed"] - base["routed"]
    others = np.delete(np.arange(w.d), o)
    assert np.all(diff[:, others] == 0)
    assert np.any(diff[:, o] != 0)
