"""The C-ABI library on a host without a GPU: it loads, exports every entry
point include/moe.h declares, sizes workspaces, and rejects bad arguments
before touching the device (nothing is ever launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("fine_grained_mixture_router_amd")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS)
    for n in names:
        assert hasattr(moe.lib(), n), n
    # no other moe_* symbols leak from the library
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(names)


def test_status_strings():
    for code, name in moe.STATUS.items():
        assert moe.status_string(code).startswith(name)
    assert "unknown" in moe.status_string(99)


def S(**kw):
    base = dict(T=128, d=512, E=16, I=256, K=4, Ks=1, Is=256)
    base.update(kw)
    return moe.make_shape(**base)


def test_workspace_size():
    n = moe.workspace_size(S())
    assert n > 0 and n % 256 == 0
    # grows with T and holds at least H and Y
    big = moe.workspace_size(S(T=4096))
    assert big > n
    T, d, K, Ks, I = 4096, 512, 4, 1, 256
    assert big >= (T * K * I + T * Ks * I) * 2 + T * (K + Ks) * d * 2
    # the V3-shape prefill layer
    v3 = moe.workspace_size(moe.make_shape(16384, 7168, 256, 2048, 8, 1, 2048))
    assert 2.5e9 < v3 < 3.2e9


@pytest.mark.parametrize("kw", [
    dict(T=0), dict(d=100), dict(d=32), dict(E=0), dict(E=257), dict(K=17), dict(K=-1),
    dict(I=100), dict(Ks=-1), dict(Ks=17), dict(Ks=1, Is=96), dict(T=(1 << 24) + 1),
])
def test_bad_shapes(kw):
    s = S(**kw)
    assert moe.lib().moe_workspace_size(ctypes.byref(s)) == 0
    code = moe.lib().moe_forward(ctypes.byref(s), *([ctypes.c_void_p(4096)] * 13),
                                 ctypes.c_size_t(1 << 40), None)
    assert code == 2


def test_bad_flags():
    s = S()
    for f in (8, 16, 1 << 31):
        s.flags = f
        assert moe.lib().moe_workspace_size(ctypes.byref(s)) == 0
    for f in (0, 1, 2, 4, 7):                    # NO_RESIDUAL, RENORM, SIGMOID and combinations
        s.flags = f
        assert moe.lib().moe_workspace_size(ctypes.byref(s)) > 0


def _fwd(shape, ws_bytes=1 << 40, **over):
    ptrs = dict(x=4096, C=4096, bias=None, w1=4096, w3=4096, w2=4096, ws1=4096, ws3=4096,
                ws2=4096, out=4096, idx=None, gate=None, ws=4096)
    ptrs.update(over)
    args = [ptrs[k] for k in ("x", "C", "bias", "w1", "w3", "w2", "ws1", "ws3", "ws2", "out",
                              "idx", "gate", "ws")]
    return moe.lib().moe_forward(ctypes.byref(shape),
                                 *[None if a is None else ctypes.c_void_p(a) for a in args],
                                 ctypes.c_size_t(ws_bytes), None)


def test_null_and_alignment():
    s = S()
    assert moe.lib().moe_forward(None, *([None] * 13), ctypes.c_size_t(0), None) == 1
    assert _fwd(s, x=None) == 1
    assert _fwd(s, out=None) == 1
    assert _fwd(s, w2=None) == 1
    assert _fwd(s, ws1=None) == 1
    assert _fwd(s, ws=None) == 1
    assert _fwd(s, C=None) == 1
    assert _fwd(s, x=4096 + 8) == 3
    assert _fwd(s, w1=4096 + 2) == 3
    assert _fwd(s, ws=4096 + 16) == 3
    assert _fwd(s, idx=4096 + 2) == 3
    # K = 0 needs no centroids or routed weights; Ks = 0 no shared weights
    s0 = S(K=0)
    assert _fwd(s0, C=None, w1=None, w3=None, w2=None, ws_bytes=1) == 4
    s1 = S(Ks=0)
    assert _fwd(s1, ws1=None, ws3=None, ws2=None, ws_bytes=1) == 4


def test_workspace_too_small():
    s = S()
    n = moe.workspace_size(s)
    assert _fwd(s, ws_bytes=n - 1) == 4


def test_no_device_reported_cleanly():
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this checks the no-device path only")
    s = S()
    assert _fwd(s, ws_bytes=moe.workspace_size(s)) == 5
    code = moe.lib().moe_route(ctypes.byref(s), ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                               None, ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                               ctypes.c_void_p(4096), ctypes.c_size_t(moe.workspace_size(s)), None)
    assert code == 5


def test_route_validation():
    s = S()
    n = moe.workspace_size(s)
    f = moe.lib().moe_route
    assert f(ctypes.byref(s), ctypes.c_void_p(4096), ctypes.c_void_p(4096), None, None,
             ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_size_t(n), None) == 1
    s0 = S(K=0)
    assert f(ctypes.byref(s0), ctypes.c_void_p(4096), ctypes.c_void_p(4096), None,
             ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096),
             ctypes.c_size_t(n), None) == 2


def test_profile_validation():
    f = moe.lib()
    assert f.moe_profile_begin(0) == 2
    assert f.moe_profile_end(None, None, 7) == 1          # nothing recording
    assert f.moe_profile_slot_name(4) == b"gemm_gate_up"
    assert f.moe_profile_slot_name(7) == b""
    assert f.moe_profile_begin_slots(1, 0) == 2           # empty slot mask
    assert f.moe_profile_begin_slots(1, 1 << 7) == 2      # past the last slot
    assert f.moe_profile_begin_slots(0, 1 << 4) == 2


def test_segment_helper():
    # N=16 experts of inter 4096 split m=4 -> 64 experts of inter 1024
    g = moe.segment(16, 4, 4096, K=8, Ks=1)
    assert (g["E"], g["I"], g["K"], g["Ks"]) == (64, 1024, 8, 1)
    with pytest.raises(ValueError):
        moe.segment(4, 3, 1000, K=2)


def test_stream_read_validation():
    f = moe.lib().moe_profile_stream_read
    assert f(None, ctypes.c_size_t(32768), None) == 1
    assert f(ctypes.c_void_p(4096), ctypes.c_size_t(0), None) == 2
    assert f(ctypes.c_void_p(4096), ctypes.c_size_t(32768 + 16), None) == 2
    assert f(ctypes.c_void_p(4096 + 8), ctypes.c_size_t(32768), None) == 3
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() == 0:
        assert f(ctypes.c_void_p(4096), ctypes.c_size_t(32768), None) == 5


def _fwd8(shape, ws_bytes=1 << 40, **over):
    ptrs = dict(x=4096, C=4096, bias=None, q1=4096, s1=4096, q3=4096, s3=4096, q2=4096, s2=4096,
                ws1=4096, ws3=4096, ws2=4096, out=4096, idx=None, gate=None, ws=4096)
    ptrs.update(over)
    keys = ("x", "C", "bias", "q1", "s1", "q3", "s3", "q2", "s2", "ws1", "ws3", "ws2", "out",
            "idx", "gate", "ws")
    return moe.lib().moe_forward_fp8(ctypes.byref(shape),
                                     *[None if ptrs[k] is None else ctypes.c_void_p(ptrs[k])
                                       for k in keys],
                                     ctypes.c_size_t(ws_bytes), None)


def test_fp8_entry_validation():
    s = S()
    assert moe.lib().moe_forward_fp8(None, *([None] * 16), ctypes.c_size_t(0), None) == 1
    for k in ("q1", "s1", "q3", "s3", "q2", "s2", "out", "ws1"):
        assert _fwd8(s, **{k: None}) == 1, k
    assert _fwd8(s, q2=4096 + 8) == 3
    assert _fwd8(s, s3=4096 + 2) == 3
    assert _fwd8(s, ws_bytes=moe.workspace_size(s) - 1) == 4
    # K = 0: no routed weights or centroids needed
    s0 = S(K=0)
    assert _fwd8(s0, C=None, q1=None, s1=None, q3=None, s3=None, q2=None, s2=None, ws_bytes=1) == 4
    bad = S(d=100)
    assert _fwd8(bad) == 2


def test_workspace_covers_both_weight_forms():
    # a prefill-sized batch: the 8-bit form plans thin tiles, whose work list
    # is longer; the one workspace size serves both entry points
    s = moe.make_shape(16384, 7168, 256, 2048, 8, 1, 2048)
    assert moe.workspace_size(s) >= 2.5e9
