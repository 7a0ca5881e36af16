"""MI355X (gfx950) DeepSeekMoE layer forward: Python binding of libmoe.so.

The layer: softmax top-K routing over E = N*m fine-grained experts, K_s
always-on shared experts, SwiGLU experts, out = x + shared + sum gate*expert
("DeepSeekMoE 深度解读报告" sections 2.2, 2.3 and 3.1; the Expert module of the
youleyou page).  Every step runs in the HIP kernels of libmoe.so; this module
only marshals arguments: torch provides device memory and the current stream.
There is no CPU fallback: if libmoe.so is missing or was not built, import
fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

NO_RESIDUAL = 1
RENORM = 2       # MOE_FLAG_RENORM
SIGMOID = 4      # MOE_FLAG_SIGMOID

STATUS = {
    0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN",
    4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_NO_DEVICE", 6: "MOE_ERR_DEVICE_ARCH", 7: "MOE_ERR_HIP",
}


class MoEError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (status {code})")
        self.code = code


class Shape(ctypes.Structure):
    """moe_shape_t."""
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("I", ctypes.c_int32), ("K", ctypes.c_int32), ("Ks", ctypes.c_int32),
                ("Is", ctypes.c_int32), ("flags", ctypes.c_uint32)]

    def as_tuple(self):
        return (self.T, self.d, self.E, self.I, self.K, self.Ks, self.Is, self.flags)


# torch is loaded first so that libmoe.so binds to the HIP runtime torch
# already carries (both name it libamdhip64.so.7): a second copy of the
# runtime in the same process would not share its devices, streams or
# allocations.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python fine_grained_mixture_router_amd/build.py` "
        "(there is no fallback implementation)")

_lib = ctypes.CDLL(LIB_PATH)
_vp = ctypes.c_void_p
_lib.moe_workspace_size.restype = ctypes.c_size_t
_lib.moe_workspace_size.argtypes = [ctypes.POINTER(Shape)]
_lib.moe_status_string.restype = ctypes.c_char_p
_lib.moe_status_string.argtypes = [ctypes.c_int]
_lib.moe_forward.restype = ctypes.c_int
_lib.moe_forward.argtypes = [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.moe_route.restype = ctypes.c_int
_lib.moe_route.argtypes = [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                           _vp]

_lib.moe_profile_begin.restype = ctypes.c_int
_lib.moe_profile_begin.argtypes = [ctypes.c_int32]
_lib.moe_profile_begin_slots.restype = ctypes.c_int
_lib.moe_profile_begin_slots.argtypes = [ctypes.c_int32, ctypes.c_uint32]
_lib.moe_profile_end.restype = ctypes.c_int
_lib.moe_profile_end.argtypes = [_vp, _vp, ctypes.c_int32]
_lib.moe_profile_slot_name.restype = ctypes.c_char_p
_lib.moe_profile_slot_name.argtypes = [ctypes.c_int32]
_lib.moe_forward_fp8.restype = ctypes.c_int
_lib.moe_forward_fp8.argtypes = [ctypes.POINTER(Shape)] + [_vp] * 16 + [ctypes.c_size_t, _vp]
_lib.moe_profile_stream_read.restype = ctypes.c_int
_lib.moe_profile_stream_read.argtypes = [_vp, ctypes.c_size_t, _vp]

EXPORTS = ("moe_workspace_size", "moe_forward", "moe_forward_fp8", "moe_route", "moe_status_string",
           "moe_profile_begin", "moe_profile_begin_slots", "moe_profile_end", "moe_profile_slot_name",
           "moe_profile_stream_read")
N_SLOTS = 7


def lib():
    return _lib


def status_string(code: int) -> str:
    return _lib.moe_status_string(int(code)).decode()


def _check(code: int):
    if code != 0:
        raise MoEError(code, status_string(code))


def make_shape(T, d, E, I, K, Ks=0, Is=0, no_residual=False, renorm=False,
               sigmoid=False) -> Shape:
    flags = ((NO_RESIDUAL if no_residual else 0) | (RENORM if renorm else 0)
             | (SIGMOID if sigmoid else 0))
    return Shape(T, d, E, I, K, Ks, Is if Ks else 0, flags)


def segment(N: int, m: int, I_std: int, K: int, Ks: int = 0) -> dict:
    """Fine-grained segmentation of N standard experts of inter-dim I_std into
    E = N*m experts of inter-dim I_std/m ("DeepSeekMoE 深度解读报告" section
    2.2).  K (routed experts per token) and Ks are passed through."""
    if I_std % m:
        raise ValueError("I_std must be divisible by m")
    return dict(E=N * m, I=I_std // m, K=K, Ks=Ks, Is=I_std // m)


def workspace_size(shape: Shape) -> int:
    n = _lib.moe_workspace_size(ctypes.byref(shape))
    if n == 0:
        raise MoEError(2, status_string(2))
    return int(n)


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _stream(device, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return _vp(s.cuda_stream)


def _shape_of(x, centroids, w1, ws1, K, no_residual, renorm=False, sigmoid=False):
    T, d = x.shape
    E = centroids.shape[0] if centroids is not None else (w1.shape[0] if w1 is not None else 1)
    I = w1.shape[1] if w1 is not None else 64
    Ks = ws1.shape[0] if ws1 is not None else 0
    Is = ws1.shape[1] if ws1 is not None and Ks else 0
    return make_shape(T, d, E, I, K, Ks, Is, no_residual, renorm, sigmoid)


def forward(x, centroids, w1, w3, w2, ws1=None, ws3=None, ws2=None, *, K: int, bias=None,
            no_residual: bool = False, renorm: bool = False, sigmoid: bool = False, out=None,
            topk_idx=None, topk_gate=None, workspace=None, stream=None,
            return_routing: bool = False):
    """Layer forward on the GPU.  Tensors are CUDA (HIP) tensors: x [T,d],
    centroids [E,d], w1/w3 [E,I,d], w2 [E,d,I], ws1/ws3 [Ks,Is,d], ws2
    [Ks,d,Is] in bfloat16; bias float32 [E] or None.  renorm / sigmoid select
    the gating variant (MOE_FLAG_RENORM / MOE_FLAG_SIGMOID).  Returns out
    [T,d] bfloat16 (and (idx, gate) when return_routing)."""
    import torch
    shape = _shape_of(x, centroids, w1, ws1, K, no_residual, renorm, sigmoid)
    dev = x.device
    if out is None:
        out = torch.empty((shape.T, shape.d), dtype=torch.bfloat16, device=dev)
    if return_routing and K > 0:
        if topk_idx is None:
            topk_idx = torch.empty((shape.T, K), dtype=torch.int32, device=dev)
        if topk_gate is None:
            topk_gate = torch.empty((shape.T, K), dtype=torch.float32, device=dev)
    nbytes = workspace_size(shape)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    code = _lib.moe_forward(ctypes.byref(shape), _ptr(x), _ptr(centroids), _ptr(bias), _ptr(w1),
                            _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(out),
                            _ptr(topk_idx), _ptr(topk_gate), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _check(code)
    if return_routing:
        return out, topk_idx, topk_gate
    return out


def forward_fp8(x, centroids, w1q, w1s, w3q, w3s, w2q, w2s, ws1=None, ws3=None, ws2=None, *,
                K: int, bias=None, no_residual: bool = False, renorm: bool = False,
                sigmoid: bool = False, out=None, topk_idx=None, topk_gate=None, workspace=None,
                stream=None, return_routing: bool = False):
    """Layer forward with 8-bit routed weights: w1q/w3q uint8 [E,I,d], w2q
    [E,d,I] (OCP E4M3 codes) with float32 per-row scales w1s/w3s [E,I], w2s
    [E,d]; shared experts ws* in bfloat16; the rest as forward()."""
    import torch
    T, d = x.shape
    E = centroids.shape[0] if centroids is not None else (w1q.shape[0] if w1q is not None else 1)
    I = w1q.shape[1] if w1q is not None else 64
    Ks = ws1.shape[0] if ws1 is not None else 0
    Is = ws1.shape[1] if ws1 is not None and Ks else 0
    shape = make_shape(T, d, E, I, K, Ks, Is, no_residual, renorm, sigmoid)
    dev = x.device
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    if return_routing and K > 0:
        if topk_idx is None:
            topk_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        if topk_gate is None:
            topk_gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    nbytes = workspace_size(shape)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    code = _lib.moe_forward_fp8(ctypes.byref(shape), _ptr(x), _ptr(centroids), _ptr(bias),
                                _ptr(w1q), _ptr(w1s), _ptr(w3q), _ptr(w3s), _ptr(w2q), _ptr(w2s),
                                _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(out), _ptr(topk_idx),
                                _ptr(topk_gate), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _check(code)
    if return_routing:
        return out, topk_idx, topk_gate
    return out


def route(x, centroids, *, K: int, bias=None, renorm: bool = False, sigmoid: bool = False,
          topk_idx=None, topk_gate=None, workspace=None, I: int = 64, stream=None):
    """Routing only: returns (idx int32 [T,K], gate float32 [T,K])."""
    import torch
    T, d = x.shape
    shape = make_shape(T, d, centroids.shape[0], I, K, renorm=renorm, sigmoid=sigmoid)
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    nbytes = workspace_size(shape)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    code = _lib.moe_route(ctypes.byref(shape), _ptr(x), _ptr(centroids), _ptr(bias),
                          _ptr(topk_idx), _ptr(topk_gate), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _check(code)
    return topk_idx, topk_gate


def profile_begin(max_calls: int, kernels=None):
    """Record HIP events around every kernel of the next max_calls forwards,
    or only around the kernels named in `kernels` (slot names)."""
    if kernels is None:
        _check(_lib.moe_profile_begin(int(max_calls)))
        return
    names = [_lib.moe_profile_slot_name(k).decode() for k in range(N_SLOTS)]
    mask = 0
    for name in kernels:
        mask |= 1 << names.index(name)
    _check(_lib.moe_profile_begin_slots(int(max_calls), mask))


def profile_end() -> dict:
    """{kernel name: (summed ms, launches)} of the recorded forwards."""
    ms = (ctypes.c_float * N_SLOTS)()
    n = (ctypes.c_int32 * N_SLOTS)()
    _check(_lib.moe_profile_end(ctypes.cast(ms, _vp), ctypes.cast(n, _vp), N_SLOTS))
    return {_lib.moe_profile_slot_name(k).decode(): (float(ms[k]), int(n[k]))
            for k in range(N_SLOTS)}


def stream_read(buf, stream=None):
    """Enqueue one pass of 16-byte loads over the device tensor `buf` (its
    size a multiple of 32768 bytes): time it to get the practical HBM read
    rate."""
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    _check(_lib.moe_profile_stream_read(ctypes.c_void_p(buf.data_ptr()),
                                        buf.numel() * buf.element_size(),
                                        ctypes.c_void_p(s.cuda_stream)))
