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
ACT8 = 8         # MOE_FLAG_ACT8 (moe_forward_fp8 only)

STATUS = {
    0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN",
    4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_NO_DEVICE", 6: "MOE_ERR_DEVICE_ARCH", 7: "MOE_ERR_HIP",
    8: "MOE_ERR_SCRATCH",
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
class Layout(ctypes.Structure):
    """moe_layout_t: where the forward leaves its token permutation."""
    _fields_ = [(n, ctypes.c_size_t) for n in ("idx", "gate", "goff", "tok_of", "slot_of",
                                               "tiles_gate_up", "tiles_down", "ntiles",
                                               "act8_codes", "act8_exps", "h",
                                               "act8_h_codes", "act8_h_exps")] + \
               [(n, ctypes.c_int32) for n in ("rows", "max_tiles_gate_up", "max_tiles_down",
                                              "tile_rows_gate_up", "tile_cols_gate_up",
                                              "tile_rows_down", "tile_cols_down")]


_lib.moe_workspace_layout.restype = ctypes.c_int
_lib.moe_workspace_layout.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Layout)]
_lib.moe_route_workspace_size.restype = ctypes.c_size_t
_lib.moe_route_workspace_size.argtypes = [ctypes.POINTER(Shape)]
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
_lib.moe_train_state_size.restype = ctypes.c_size_t
_lib.moe_train_state_size.argtypes = [ctypes.POINTER(Shape)]
_lib.moe_backward_workspace_size.restype = ctypes.c_size_t
_lib.moe_backward_workspace_size.argtypes = [ctypes.POINTER(Shape)]
_lib.moe_forward_train.restype = ctypes.c_int
_lib.moe_forward_train.argtypes = [ctypes.POINTER(Shape)] + [_vp] * 14 + [ctypes.c_size_t, _vp]
_lib.moe_backward.restype = ctypes.c_int
_lib.moe_backward.argtypes = ([ctypes.POINTER(Shape)] + [_vp] * 9 + [ctypes.c_float, _vp,
                              ctypes.c_size_t] + [_vp] * 10 + [ctypes.c_size_t, _vp])
_lib.moe_forward_noalloc.restype = ctypes.c_int
_lib.moe_forward_noalloc.argtypes = [ctypes.POINTER(Shape)] + [_vp] * 13
_lib.moe_noalloc_scratch_bytes.restype = ctypes.c_size_t
_lib.moe_noalloc_scratch_bytes.argtypes = []
_lib.moe_profile_stream_read.restype = ctypes.c_int
_lib.moe_profile_stream_read.argtypes = [_vp, ctypes.c_size_t, _vp]

EXPORTS = ("moe_workspace_size", "moe_workspace_layout", "moe_route_workspace_size", "moe_forward", "moe_forward_fp8", "moe_route", "moe_status_string",
           "moe_profile_begin", "moe_profile_begin_slots", "moe_profile_end", "moe_profile_slot_name",
           "moe_profile_stream_read", "moe_forward_noalloc", "moe_noalloc_scratch_bytes",
           "moe_train_state_size", "moe_backward_workspace_size", "moe_forward_train",
           "moe_backward")
N_SLOTS = 18


def lib():
    return _lib


def status_string(code: int) -> str:
    return _lib.moe_status_string(int(code)).decode()


def _check(code: int):
    if code != 0:
        raise MoEError(code, status_string(code))


def make_shape(T, d, E, I, K, Ks=0, Is=0, no_residual=False, renorm=False,
               sigmoid=False, act8=False) -> Shape:
    flags = ((NO_RESIDUAL if no_residual else 0) | (RENORM if renorm else 0)
             | (SIGMOID if sigmoid else 0) | (ACT8 if act8 else 0))
    return Shape(T, d, E, I, K, Ks, Is if Ks else 0, flags)


def segment(N: int, m: int, I_std: int, K_std: int, Ks: int = 0,
            isolate_from_pool: bool = True) -> dict:
    """Layer shape of DeepSeekMoE's fine-grained segmentation and shared-expert
    isolation ("DeepSeekMoE 深度解读报告", sections 2.2 and 2.3).

    N standard experts of inter-dim I_std, K_std of them active per token,
    are each split m ways along the intermediate dimension: N*m experts of
    inter-dim I_std/m, with m*K_std of them active, so the parameters and the
    per-token compute stay those of the unsegmented layer (section 2.2).  Ks
    of the fine-grained experts are then isolated as shared experts that
    every token uses (section 2.3): with isolate_from_pool they come out of
    the N*m pool and the routed active count drops by Ks, which keeps both
    totals fixed (E = N*m - Ks routed, K = m*K_std - Ks); without it the Ks
    shared experts are added on top (E = N*m, K = m*K_std).  The 2B
    validation layer is segment(16, 4, 3584, 2, Ks=1): 63 routed experts of
    inter 896, top-7, plus one shared."""
    if m < 1 or N < 1 or K_std < 0 or Ks < 0:
        raise ValueError("N, m >= 1 and K_std, Ks >= 0")
    if I_std % m:
        raise ValueError("I_std must be divisible by m")
    E, K = N * m, m * K_std
    if isolate_from_pool:
        E, K = E - Ks, K - Ks
        if E < 1 or K < 0:
            raise ValueError("more shared experts than the segmented pool or active count holds")
    return dict(E=E, I=I_std // m, K=K, Ks=Ks, Is=I_std // m)


def workspace_size(shape: Shape) -> int:
    n = _lib.moe_workspace_size(ctypes.byref(shape))
    if n == 0:
        raise MoEError(2, status_string(2))
    return int(n)


def workspace_layout(shape: Shape) -> dict:
    """moe_workspace_layout as a dict: byte offsets of the permutation arrays
    in a forward call's workspace, and the work lists' sizes and tile shapes."""
    lay = Layout()
    _check(_lib.moe_workspace_layout(ctypes.byref(shape), ctypes.byref(lay)))
    return {n: getattr(lay, n) for n, _ in Layout._fields_}


def route_workspace_size(shape: Shape) -> int:
    n = _lib.moe_route_workspace_size(ctypes.byref(shape))
    if n == 0:
        raise MoEError(2, status_string(2))
    return int(n)


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _resolve_stream(device, stream):
    """(stream object, whether it differs from the device's current stream)."""
    cur = torch.cuda.current_stream(device)
    if stream is None:
        return cur, False
    return stream, stream.cuda_stream != cur.cuda_stream


def _need(t, name, dtype, shape, device):
    """Validate a tensor argument before its pointer crosses the ABI: on
    `device`, of `dtype`, exactly `shape`, contiguous.  A mismatch raises
    ValueError and nothing is launched."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _absent(t, name):
    if t is not None:
        raise ValueError(f"{name} must be None here")


class _Alloc:
    """Allocations made on behalf of the caller.  With an explicit stream
    other than the current one, every such tensor is marked as used by that
    stream (record_stream), so torch's caching allocator does not hand its
    memory to other work before the enqueued kernels are done with it."""

    def __init__(self, device, stream):
        self.device = device
        self.stream, self.side = _resolve_stream(device, stream)

    def empty(self, shape, dtype):
        t = torch.empty(shape, dtype=dtype, device=self.device)
        if self.side:
            t.record_stream(self.stream)
        return t

    def handle(self):
        return _vp(self.stream.cuda_stream)


def _x_of(x):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [T, d]")
    if not x.is_cuda:
        raise ValueError("x must be a device (HIP) tensor")
    return x.shape[0], x.shape[1], x.device


def _check_routing_args(T, d, E, K, centroids, bias, dev):
    if K > 0:
        _need(centroids, "centroids", torch.bfloat16, (E, d), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,), dev)


def _check_shared(ws1, ws3, ws2, d, dev):
    if ws1 is None and ws3 is None and ws2 is None:
        return 0, 0
    if ws1 is None or ws1.dim() != 3:
        raise ValueError("ws1 must be [Ks, Is, d] (or all of ws1/ws3/ws2 None)")
    Ks, Is = ws1.shape[0], ws1.shape[1]
    _need(ws1, "ws1", torch.bfloat16, (Ks, Is, d), dev)
    _need(ws3, "ws3", torch.bfloat16, (Ks, Is, d), dev)
    _need(ws2, "ws2", torch.bfloat16, (Ks, d, Is), dev)
    return Ks, (Is if Ks else 0)


def _routing_outputs(al, T, K, topk_idx, topk_gate, want):
    if K > 0:
        if topk_idx is not None:
            _need(topk_idx, "topk_idx", torch.int32, (T, K), al.device)
        elif want:
            topk_idx = al.empty((T, K), torch.int32)
        if topk_gate is not None:
            _need(topk_gate, "topk_gate", torch.float32, (T, K), al.device)
        elif want:
            topk_gate = al.empty((T, K), torch.float32)
    else:
        _absent(topk_idx, "topk_idx (K == 0)")
        _absent(topk_gate, "topk_gate (K == 0)")
    return topk_idx, topk_gate


def _outputs(al, T, d, K, out, topk_idx, topk_gate, return_routing):
    if out is None:
        out = al.empty((T, d), torch.bfloat16)
    else:
        _need(out, "out", torch.bfloat16, (T, d), al.device)
    return (out,) + _routing_outputs(al, T, K, topk_idx, topk_gate, return_routing)


def _workspace(al, shape, workspace, size_fn=workspace_size):
    nbytes = size_fn(shape)
    if workspace is None:
        return al.empty((nbytes,), torch.uint8)
    if workspace.device != al.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on x's device")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"needs {nbytes}")
    return workspace


def forward(x, centroids, w1, w3, w2, ws1=None, ws3=None, ws2=None, *, K: int, bias=None,
            no_residual: bool = False, renorm: bool = False, sigmoid: bool = False, out=None,
            topk_idx=None, topk_gate=None, workspace=None, stream=None,
            return_routing: bool = False):
    """Layer forward on the GPU.  Tensors are CUDA (HIP) tensors: x [T,d],
    centroids [E,d], w1/w3 [E,I,d], w2 [E,d,I], ws1/ws3 [Ks,Is,d], ws2
    [Ks,d,Is] in bfloat16; bias float32 [E] or None.  renorm / sigmoid select
    the gating variant (MOE_FLAG_RENORM / MOE_FLAG_SIGMOID).  Every tensor is
    checked (device, dtype, shape, contiguity) before anything is launched.
    Returns out [T,d] bfloat16 (and (idx, gate) when return_routing)."""
    T, d, dev = _x_of(x)
    _need(x, "x", torch.bfloat16, (T, d), dev)
    if K > 0:
        if w1 is None or w1.dim() != 3:
            raise ValueError("w1 must be [E, I, d] when K > 0")
        E, I = w1.shape[0], w1.shape[1]
        _need(w1, "w1", torch.bfloat16, (E, I, d), dev)
        _need(w3, "w3", torch.bfloat16, (E, I, d), dev)
        _need(w2, "w2", torch.bfloat16, (E, d, I), dev)
    else:
        E = centroids.shape[0] if centroids is not None else (w1.shape[0] if w1 is not None else 1)
        I = w1.shape[1] if w1 is not None else 64
    _check_routing_args(T, d, E, K, centroids, bias, dev)
    Ks, Is = _check_shared(ws1, ws3, ws2, d, dev)
    shape = make_shape(T, d, E, I, K, Ks, Is, no_residual, renorm, sigmoid)
    al = _Alloc(dev, stream)
    out, topk_idx, topk_gate = _outputs(al, T, d, K, out, topk_idx, topk_gate, return_routing)
    workspace = _workspace(al, shape, workspace)
    code = _lib.moe_forward(ctypes.byref(shape), _ptr(x), _ptr(centroids), _ptr(bias), _ptr(w1),
                            _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(out),
                            _ptr(topk_idx), _ptr(topk_gate), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), al.handle())
    _check(code)
    if return_routing:
        return out, topk_idx, topk_gate
    return out


def noalloc_scratch_bytes() -> int:
    return int(_lib.moe_noalloc_scratch_bytes())


def forward_noalloc(x, centroids, w1, w3, w2, ws1=None, ws3=None, ws2=None, *, K: int,
                    bias=None, out, topk_idx=None, topk_gate=None, no_residual: bool = False,
                    renorm: bool = False, sigmoid: bool = False, stream=None):
    """moe_forward_noalloc: the layer forward with the library's static scratch
    array as workspace.  Allocates nothing: the caller passes out (and the
    optional topk_idx / topk_gate).  Calls that overlap on one GPU race on the
    shared scratch.  Shapes too large for it raise MoEError (MOE_ERR_SCRATCH)."""
    T, d, dev = _x_of(x)
    _need(x, "x", torch.bfloat16, (T, d), dev)
    if K > 0:
        if w1 is None or w1.dim() != 3:
            raise ValueError("w1 must be [E, I, d] when K > 0")
        E, I = w1.shape[0], w1.shape[1]
        _need(w1, "w1", torch.bfloat16, (E, I, d), dev)
        _need(w3, "w3", torch.bfloat16, (E, I, d), dev)
        _need(w2, "w2", torch.bfloat16, (E, d, I), dev)
    else:
        E = centroids.shape[0] if centroids is not None else (w1.shape[0] if w1 is not None else 1)
        I = w1.shape[1] if w1 is not None else 64
    _check_routing_args(T, d, E, K, centroids, bias, dev)
    Ks, Is = _check_shared(ws1, ws3, ws2, d, dev)
    _need(out, "out", torch.bfloat16, (T, d), dev)
    shape = make_shape(T, d, E, I, K, Ks, Is, no_residual, renorm, sigmoid)
    al = _Alloc(dev, stream)
    topk_idx, topk_gate = _routing_outputs(al, T, K, topk_idx, topk_gate, False)
    code = _lib.moe_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(centroids), _ptr(bias),
                                    _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2),
                                    _ptr(out), _ptr(topk_idx), _ptr(topk_gate), al.handle())
    _check(code)
    return out


def train_state_size(shape: Shape) -> int:
    n = _lib.moe_train_state_size(ctypes.byref(shape))
    if n == 0:
        raise MoEError(2, status_string(2))
    return int(n)


def backward_workspace_size(shape: Shape) -> int:
    n = _lib.moe_backward_workspace_size(ctypes.byref(shape))
    if n == 0:
        raise MoEError(2, status_string(2))
    return int(n)


class TrainState:
    """What moe_forward_train saved for moe_backward: the shape and the state
    buffer (a uint8 device tensor the caller keeps until the backward)."""

    def __init__(self, shape: Shape, buf):
        self.shape = shape
        self.buf = buf


def _expert_args(x, centroids, w1, w3, w2, ws1, ws3, ws2, K, bias):
    T, d, dev = _x_of(x)
    _need(x, "x", torch.bfloat16, (T, d), dev)
    if K > 0:
        if w1 is None or w1.dim() != 3:
            raise ValueError("w1 must be [E, I, d] when K > 0")
        E, I = w1.shape[0], w1.shape[1]
        _need(w1, "w1", torch.bfloat16, (E, I, d), dev)
        _need(w3, "w3", torch.bfloat16, (E, I, d), dev)
        _need(w2, "w2", torch.bfloat16, (E, d, I), dev)
    else:
        E = centroids.shape[0] if centroids is not None else (w1.shape[0] if w1 is not None else 1)
        I = w1.shape[1] if w1 is not None else 64
    _check_routing_args(T, d, E, K, centroids, bias, dev)
    Ks, Is = _check_shared(ws1, ws3, ws2, d, dev)
    return T, d, E, I, Ks, Is, dev


def forward_train(x, centroids, w1, w3, w2, ws1=None, ws3=None, ws2=None, *, K: int, bias=None,
                  no_residual: bool = False, renorm: bool = False, sigmoid: bool = False,
                  out=None, topk_idx=None, topk_gate=None, state=None, stream=None,
                  return_routing: bool = False, return_stats: bool = False):
    """moe_forward_train: the forward (same results as forward()) that also
    writes the training state the backward reads.  Returns (out, TrainState)
    plus (idx, gate) with return_routing and the balance statistics
    (f [E], P [E], L_bal) with return_stats."""
    T, d, E, I, Ks, Is, dev = _expert_args(x, centroids, w1, w3, w2, ws1, ws3, ws2, K, bias)
    shape = make_shape(T, d, E, I, K, Ks, Is, no_residual, renorm, sigmoid)
    al = _Alloc(dev, stream)
    out, topk_idx, topk_gate = _outputs(al, T, d, K, out, topk_idx, topk_gate, return_routing)
    stats = al.empty((2 * E + 1,), torch.float32) if (return_stats and K > 0) else None
    state = _workspace(al, shape, state, train_state_size)
    code = _lib.moe_forward_train(ctypes.byref(shape), _ptr(x), _ptr(centroids), _ptr(bias),
                                  _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2),
                                  _ptr(out), _ptr(topk_idx), _ptr(topk_gate), _ptr(stats),
                                  _ptr(state), state.numel() * state.element_size(), al.handle())
    _check(code)
    res = (out, TrainState(shape, state))
    if return_routing:
        res += (topk_idx, topk_gate)
    if return_stats:
        res += ((stats[:E], stats[E:2 * E], stats[2 * E]) if stats is not None else None,)
    return res


def backward(x, centroids, w1, w3, w2, ws1=None, ws3=None, ws2=None, *, dout, state: TrainState,
             alpha: float = 0.0, dx=None, dw1=None, dw3=None, dw2=None, dws1=None, dws3=None,
             dws2=None, dC=None, dgate=None, workspace=None, stream=None,
             return_dgate: bool = False):
    """moe_backward: gradients of sum(dout * out) + alpha * L_bal for the
    forward that produced `state` (same inputs).  Returns a dict with dx
    [T,d], dw1/dw3 [E,I,d], dw2 [E,d,I] (bf16; None without a router),
    dws1/dws3/dws2 (bf16; None without shared experts), dC [E,d] (fp32) and,
    with return_dgate, dgate [T,K] (fp32)."""
    shape = state.shape
    K = shape.K
    T, d, E, I, Ks, Is, dev = _expert_args(x, centroids, w1, w3, w2, ws1, ws3, ws2, K, None)
    if (T, d, E, I, Ks, Is) != (shape.T, shape.d, shape.E, shape.I, shape.Ks, shape.Is):
        raise ValueError("the tensors do not match the shape of the training forward")
    _need(dout, "dout", torch.bfloat16, (T, d), dev)
    if state.buf.device != dev:
        raise ValueError("state is on another device")
    al = _Alloc(dev, stream)

    def out_t(t, name, dtype, shp, want):
        if not want:
            _absent(t, name)
            return None
        if t is None:
            return al.empty(shp, dtype)
        return _need(t, name, dtype, shp, dev)

    dx = out_t(dx, "dx", torch.bfloat16, (T, d), True)
    dw1 = out_t(dw1, "dw1", torch.bfloat16, (E, I, d), K > 0)
    dw3 = out_t(dw3, "dw3", torch.bfloat16, (E, I, d), K > 0)
    dw2 = out_t(dw2, "dw2", torch.bfloat16, (E, d, I), K > 0)
    dws1 = out_t(dws1, "dws1", torch.bfloat16, (Ks, Is, d), Ks > 0)
    dws3 = out_t(dws3, "dws3", torch.bfloat16, (Ks, Is, d), Ks > 0)
    dws2 = out_t(dws2, "dws2", torch.bfloat16, (Ks, d, Is), Ks > 0)
    dC = out_t(dC, "dC", torch.float32, (E, d), K > 0)
    dgate = out_t(dgate, "dgate", torch.float32, (T, K), K > 0 and (return_dgate or dgate is not None))
    workspace = _workspace(al, shape, workspace, backward_workspace_size)
    code = _lib.moe_backward(ctypes.byref(shape), _ptr(x), _ptr(centroids), _ptr(w1), _ptr(w3),
                             _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(dout),
                             ctypes.c_float(float(alpha)), _ptr(state.buf),
                             state.buf.numel() * state.buf.element_size(), _ptr(dx), _ptr(dw1),
                             _ptr(dw3), _ptr(dw2), _ptr(dws1), _ptr(dws3), _ptr(dws2), _ptr(dC),
                             _ptr(dgate), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), al.handle())
    _check(code)
    return dict(dx=dx, dw1=dw1, dw3=dw3, dw2=dw2, dws1=dws1, dws3=dws3, dws2=dws2, dC=dC,
                dgate=dgate)


def forward_fp8(x, centroids, w1q, w1s, w3q, w3s, w2q, w2s, ws1=None, ws3=None, ws2=None, *,
                K: int, bias=None, no_residual: bool = False, renorm: bool = False,
                sigmoid: bool = False, act8: bool = False, out=None, topk_idx=None, topk_gate=None,
                workspace=None, stream=None, return_routing: bool = False):
    """Layer forward with 8-bit routed weights: w1q/w3q uint8 [E,I,d], w2q
    [E,d,I] (OCP E4M3 codes) with float32 per-row scales w1s/w3s [E,I], w2s
    [E,d]; shared experts ws* in bfloat16; the rest as forward().  act8
    (MOE_FLAG_ACT8): the routed gate/up products take 8-bit activations
    (per-token power-of-two scale, nearest-even E4M3 codes) on the FP8
    matrix cores."""
    T, d, dev = _x_of(x)
    _need(x, "x", torch.bfloat16, (T, d), dev)
    if K > 0:
        if w1q is None or w1q.dim() != 3:
            raise ValueError("w1q must be [E, I, d] when K > 0")
        E, I = w1q.shape[0], w1q.shape[1]
        _need(w1q, "w1q", torch.uint8, (E, I, d), dev)
        _need(w3q, "w3q", torch.uint8, (E, I, d), dev)
        _need(w2q, "w2q", torch.uint8, (E, d, I), dev)
        _need(w1s, "w1s", torch.float32, (E, I), dev)
        _need(w3s, "w3s", torch.float32, (E, I), dev)
        _need(w2s, "w2s", torch.float32, (E, d), dev)
    else:
        E = centroids.shape[0] if centroids is not None else (w1q.shape[0] if w1q is not None else 1)
        I = w1q.shape[1] if w1q is not None else 64
    _check_routing_args(T, d, E, K, centroids, bias, dev)
    Ks, Is = _check_shared(ws1, ws3, ws2, d, dev)
    shape = make_shape(T, d, E, I, K, Ks, Is, no_residual, renorm, sigmoid, act8)
    al = _Alloc(dev, stream)
    out, topk_idx, topk_gate = _outputs(al, T, d, K, out, topk_idx, topk_gate, return_routing)
    workspace = _workspace(al, shape, workspace)
    code = _lib.moe_forward_fp8(ctypes.byref(shape), _ptr(x), _ptr(centroids), _ptr(bias),
                                _ptr(w1q), _ptr(w1s), _ptr(w3q), _ptr(w3s), _ptr(w2q), _ptr(w2s),
                                _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(out), _ptr(topk_idx),
                                _ptr(topk_gate), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), al.handle())
    _check(code)
    if return_routing:
        return out, topk_idx, topk_gate
    return out


def route(x, centroids, *, K: int, bias=None, renorm: bool = False, sigmoid: bool = False,
          topk_idx=None, topk_gate=None, workspace=None, stream=None):
    """Routing only: returns (idx int32 [T,K], gate float32 [T,K]).  Needs
    only the routing scratch (moe_route_workspace_size)."""
    T, d, dev = _x_of(x)
    _need(x, "x", torch.bfloat16, (T, d), dev)
    if centroids is None or centroids.dim() != 2:
        raise ValueError("centroids must be [E, d]")
    E = centroids.shape[0]
    if K < 1:
        raise ValueError("route needs K >= 1")
    _check_routing_args(T, d, E, K, centroids, bias, dev)
    shape = make_shape(T, d, E, 64, K, renorm=renorm, sigmoid=sigmoid)
    al = _Alloc(dev, stream)
    topk_idx, topk_gate = _routing_outputs(al, T, K, topk_idx, topk_gate, True)
    workspace = _workspace(al, shape, workspace, route_workspace_size)
    code = _lib.moe_route(ctypes.byref(shape), _ptr(x), _ptr(centroids), _ptr(bias),
                          _ptr(topk_idx), _ptr(topk_gate), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), al.handle())
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
