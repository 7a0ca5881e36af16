"""The seeded input generator: determinism, slice regeneration, bf16 rounding,
and the shape of its draws."""
from fractions import Fraction
import math

import numpy as np
import pytest

import synth
from synth import workloads as wl


def test_deterministic_and_sliceable():
    a = synth.normal_bf16(7, 3, (1000,), 0.006)
    b = synth.normal_bf16(7, 3, (1000,), 0.006)
    assert np.array_equal(a, b)
    # any slice, odd or even offset, regenerates the same elements
    for off, n in ((0, 10), (1, 7), (333, 100), (998, 2)):
        s = synth.normal_bf16(7, 3, (n,), 0.006, offset=off)
        assert np.array_equal(s, a[off:off + n])
    # different streams / seeds differ
    assert not np.array_equal(a, synth.normal_bf16(7, 4, (1000,), 0.006))
    assert not np.array_equal(a, synth.normal_bf16(8, 3, (1000,), 0.006))


def test_thread_count_independent(monkeypatch):
    a = synth.normal_bf16(11, 0, (4097,), 1.0)
    # the per-element result depends only on the counter, so it equals the
    # unrounded draw rounded once
    z = synth.normal_f64(11, 0, 4097)
    ref = np.array([synth.bf16_from_double(v) for v in z], dtype=np.uint16)
    assert np.array_equal(a, ref)


def _exact_bf16_rne(v: float) -> int:
    """Nearest-even bf16 of a finite double, by exact rational arithmetic."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    q = Fraction(abs(v))
    e = math.floor(math.log2(abs(v)))
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)                         # subnormal range uses the min exponent
    ulp = Fraction(2) ** (e - 7)
    m = q / ulp
    lo = math.floor(m)
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    val = lo * ulp
    # re-encode val as bf16 bits through float32 (exact: val has <= 8 significant bits)
    f = np.array([float(val)], dtype=np.float32).view(np.uint32)[0]
    return sign | int(f >> 16)


@pytest.mark.parametrize("v", [
    1.0, -1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -60, 1.01171875,
    1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40, 1.0 + 2 ** -8 - 2 ** -40,
    0.006, -0.006, 3.14159265358979, 65504.0, 2 ** -130, 1.5 * 2 ** -133,
    0.1, -2.5e-3, 123456.789,
])
def test_bf16_rounding_exact(v):
    assert synth.bf16_from_double(v) == _exact_bf16_rne(v)


def test_bf16_rounding_random():
    rng = np.random.default_rng(0)
    vals = rng.standard_normal(2000) * np.exp(rng.uniform(-20, 20, 2000))
    for v in vals:
        assert synth.bf16_from_double(float(v)) == _exact_bf16_rne(float(v))


def test_normal_moments():
    z = synth.normal_f64(5, 1, 200_000)
    assert abs(z.mean()) < 0.01
    assert abs(z.std() - 1.0) < 0.01
    # fourth moment of a normal is 3
    assert abs((z ** 4).mean() - 3.0) < 0.1
    w = synth.bf16_to_f64(synth.normal_bf16(5, 1, (200_000,), 0.006))
    assert abs(w.std() / 0.006 - 1.0) < 0.01


def test_permutation_and_zipf_bias():
    p = synth.permutation(3, 2, 256)
    assert sorted(p.tolist()) == list(range(1, 257))
    assert np.array_equal(p, synth.permutation(3, 2, 256))
    b = synth.zipf_bias(3, 256, 1.2)
    assert b.dtype == np.float32
    # exp(b) proportional to rank^-s: the rank-1 expert has bias 0, the rest below
    assert b.max() == 0.0 and int(np.argmax(b)) == int(np.where(p == 1)[0][0])
    np.testing.assert_allclose(np.exp(b.astype(np.float64)), p.astype(np.float64) ** -1.2, rtol=1e-6)


def test_workload_slices_match_full():
    w = wl.WORKLOADS["tiny"]
    full = wl.gen_all(w)
    for e in (0, 5, w.E - 1):
        w1, w3, w2 = wl.gen_expert(w, e)
        assert np.array_equal(w1, full["w1"][e])
        assert np.array_equal(w3, full["w3"][e])
        assert np.array_equal(w2, full["w2"][e])
    rows = wl.gen_x_rows(w, [0, 17, 127])
    assert np.array_equal(rows, full["x"][[0, 17, 127]])
    assert full["bias"] is None
    assert wl.gen_bias(wl.WORKLOADS["16b_zipf"]).shape == (64,)


def test_workload_table():
    # fine-grained shapes: E = N*m routed experts of inter I_std/m
    t = wl.WORKLOADS
    assert (t["tiny"].E, t["tiny"].I, t["tiny"].K, t["tiny"].Ks) == (16, 256, 4, 1)
    assert t["v3_decode"].rows == 256 * 9
    assert t["v3_prefill"].rows == 16384 * 9
    assert t["v3_prefill"].wseed == t["v3_decode"].wseed
