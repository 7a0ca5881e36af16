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


# ---------------------------------------------------------------------------
# 8-bit activations (ACT8): per-token power-of-two scale, nearest-even E4M3
# codes, used by the routed experts' gate/up products only.
# ---------------------------------------------------------------------------

def test_act8_exponent_is_the_smallest_fitting_power_of_two():
    """Q1: e is the smallest integer with amax <= 448 * 2^e: exact at
    448 * 2^k, one more just above it; a zero row takes e = 0."""
    for k in range(-20, 12):
        top = 448.0 * 2.0 ** k
        assert oracle.act8_exponent(top) == k
        assert oracle.act8_exponent(np.nextafter(top, np.inf)) == k + 1
        assert oracle.act8_exponent(np.nextafter(top, 0.0)) == k
        assert oracle.act8_exponent(224.0 * 2.0 ** k) == k - 1       # the binade below fits one lower
        assert oracle.act8_exponent(np.nextafter(224.0 * 2.0 ** k, np.inf)) == k
    assert oracle.act8_exponent(0.0) == 0
    rng = np.random.default_rng(3)
    for a in np.exp(rng.uniform(-30, 20, 500)):
        e = oracle.act8_exponent(a)
        assert a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1)


def test_e4m3_nearest_even():
    """Q2: every finite E4M3 value maps to its own code; midpoints between
    neighbours go to the even code, values beside them to the nearer one;
    the sign bit follows the sign (also of zero)."""
    pos = E4M3[:0x7F]
    for q in range(0x7F):
        assert oracle.e4m3_nearest(pos[q]) == q
        assert oracle.e4m3_nearest(-pos[q]) == q | 0x80
    for q in range(0x7E):
        mid = 0.5 * (pos[q] + pos[q + 1])
        even = q if q % 2 == 0 else q + 1
        assert oracle.e4m3_nearest(mid) == even
        assert oracle.e4m3_nearest(np.nextafter(mid, 0.0)) == q
        assert oracle.e4m3_nearest(np.nextafter(mid, np.inf)) == q + 1
    assert oracle.e4m3_nearest(0.0) == 0x00 and oracle.e4m3_nearest(-0.0) == 0x80
    assert oracle.e4m3_nearest(448.0) == 0x7E


def test_act8_rows_error_bound_and_top_binade():
    """Q3: every dequantised value is within half a code step of the input
    (the step of E4M3 at that magnitude times 2^e), each row's largest
    magnitude, scaled, lies in (224, 448] and so codes to a value in [224,
    448] (e is not larger than needed), and a row of already representable
    values comes back exactly."""
    rng = np.random.default_rng(5)
    x = synth.f32_to_bf16_rne((rng.standard_normal((16, 512)) * np.exp(rng.uniform(-8, 8, (16, 1))))
                              .astype(np.float32))
    codes, exps = oracle.quantize_act8(x)
    xv = synth.bf16_to_f64(x)
    deq = E4M3[codes] * np.ldexp(1.0, exps)[:, None]
    y = np.abs(xv) * np.ldexp(1.0, -exps)[:, None]
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
    assert np.all(np.abs(deq - xv) <= 0.5 * step * np.ldexp(1.0, exps)[:, None])
    top = np.abs(E4M3[codes]).max(axis=1)
    assert np.all((top >= 224.0) & (top <= 448.0))
    assert np.all(np.abs(xv).max(axis=1) * np.ldexp(1.0, -exps) > 224.0)
    # representable rows: codes times a power of two, the row max at 448 * 2^e
    q = rng.integers(0, 0x7E, size=(4, 64)).astype(np.uint8)
    q[:, 0] = 0x7E
    for t, e in enumerate([-3, 0, 5, -12]):
        row = E4M3[q[t]] * 2.0 ** e
        bits = synth.f32_to_bf16_rne(row.astype(np.float32))
        c2, e2 = oracle.quantize_act8(bits[None, :])
        assert e2[0] == e and np.array_equal(c2[0], q[t])


def _fp8(w, L, **kw):
    return oracle.forward_fp8(L["x"], L["C"], L["bias"], L["q1"], L["s1"], L["q3"], L["s3"],
                              L["q2"], L["s2"], L["ws1"], L["ws3"], L["ws2"], w.K, **kw)


def test_bf16_nearest():
    """Q6: h is rounded to bf16 before its codes are taken.  Every finite
    bf16 value maps to its own bits (both zeros, subnormals, the largest
    finite), the midpoint of two neighbours to the one with the even
    significand, values just beside a midpoint to the nearer neighbour."""
    bits = np.arange(0x8000, dtype=np.uint32)
    bits = bits[(bits & 0x7F80) != 0x7F80].astype(np.uint16)          # finite, non-negative
    val = synth.bf16_to_f64(bits)
    for b, v in zip(bits[::7], val[::7]):
        assert oracle.bf16_nearest(v) == b
        assert oracle.bf16_nearest(-v) == b | 0x8000
    for b in list(range(0, 40)) + list(range(0x3F70, 0x3F90)) + list(range(0x7F00, 0x7F7F)):
        lo, hi = val[b], val[b + 1]
        mid = 0.5 * (lo + hi)                      # exact in double
        assert oracle.bf16_nearest(mid) == (b if b % 2 == 0 else b + 1)
        assert oracle.bf16_nearest(np.nextafter(mid, 0.0)) == b
        assert oracle.bf16_nearest(np.nextafter(mid, np.inf)) == b + 1
        assert oracle.bf16_nearest(-mid) == (b if b % 2 == 0 else b + 1) | 0x8000


def test_act8_down_input_is_the_quantised_bf16_h():
    """Q4: the routed experts' down projection takes 8-bit activations made
    from h rounded to bf16.  With rows already on the 8-bit grid (so the x
    quantisation changes nothing), one expert per token with gate 1
    (renormalised K = 1) and W2 the identity (d = I), the 8-bit-weight
    layer's routed part is h itself, and the ACT8 layer's must be exactly
    e4m3(codes) * 2^e of quantize_act8(bf16(h)) row by row.  The instance
    is one where skipping the bf16 rounding would change some codes."""
    T, d, E = 16, 128, 6
    w = wl.Workload("t", T=T, d=d, E=E, I=d, K=1, Ks=1, Is=64, wseed=41, xseed=41)
    rng = np.random.default_rng(41)
    q1, _, q3, _, _, _ = wl.gen_routed_fp8(w)
    pw = lambda *s: np.ldexp(1.0, -rng.integers(3, 6, size=s)).astype(np.float32)
    q2 = np.zeros((E, d, d), np.uint8)
    q2[:, np.arange(d), np.arange(d)] = 0x38                           # e4m3 1.0 on the diagonal
    L = dict(C=wl.gen_centroids(w), q1=q1, q3=q3, q2=q2, s1=pw(E, d), s3=pw(E, d),
             s2=np.ones((E, d), np.float32), bias=np.zeros(E, np.float32))
    L["ws1"], L["ws3"], L["ws2"] = wl.gen_shared(w)
    q = rng.integers(0, 0x7E, size=(T, d)).astype(np.uint8)
    q[:, 5] = 0x7E
    sign = np.where(rng.random((T, d)) < 0.5, -1.0, 1.0)
    L["x"] = synth.f32_to_bf16_rne((sign * E4M3[q] * np.ldexp(1.0, rng.integers(-4, 0, size=(T, 1))))
                                   .astype(np.float32))
    a = _fp8(w, L, renorm=True)
    b = _fp8(w, L, renorm=True, act8=True)
    assert np.all(a["gate"] == 1.0)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["shared"], b["shared"])
    h = a["routed"]
    hb = np.array([[oracle.bf16_nearest(v) for v in row] for row in h], np.uint16)
    codes, exps = oracle.quantize_act8(hb)
    want = E4M3[codes] * np.ldexp(1.0, exps)[:, None]
    assert np.array_equal(b["routed"], want)
    direct = np.array([[oracle.e4m3_nearest(v * 2.0 ** -e) for v in row] for row, e in zip(h, exps)])
    assert (direct != codes).any()                 # the bf16 step matters here


def test_act8_touches_only_the_routed_experts():
    """Q5: on ordinary rows, ACT8 leaves the routing and the shared experts'
    part unchanged to the last bit and moves the routed part by about the
    size of the activation rounding (and no more)."""
    w, L = _layer(32, T=16, d=128)
    a, b = _fp8(w, L), _fp8(w, L, act8=True)
    for k in ("shared", "gate", "margin"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["idx"], b["idx"])
    d = b["routed"] - a["routed"]
    rel = np.sqrt((d ** 2).mean()) / np.sqrt((a["routed"] ** 2).mean())
    assert 1e-4 < rel < 0.1
