"""Seeded synthetic inputs for the MoE layer (host side, numpy).

This module only draws numbers; it holds no step of the layer's arithmetic.
Both the oracle and the HIP path consume the bytes it produces.  Draws are
counter-based (SplitMix64 as a hash of (seed, stream, index), then
Box-Muller, then one round-to-nearest-even to bfloat16), so one expert's
weights or one token's row can be regenerated without the rest.

Stream ids per tensor: x 0, centroids 1, bias permutation 2, W1 3, W3 4,
W2 5, shared W1 6, shared W3 7, shared W2 8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")

STREAM_X, STREAM_C, STREAM_BIAS, STREAM_W1, STREAM_W3, STREAM_W2 = 0, 1, 2, 3, 4, 5
STREAM_WS1, STREAM_WS3, STREAM_WS2 = 6, 7, 8
STREAM_Q1, STREAM_Q3, STREAM_Q2 = 9, 10, 11            # 8-bit routed weight codes
STREAM_S1, STREAM_S3, STREAM_S2 = 12, 13, 14           # their per-row scales
STREAM_DOUT = 15                                         # upstream gradient of a backward


def build(force: bool = True) -> str:
    """Compile gen.c into libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, i32, dbl = ctypes.c_uint64, ctypes.c_int32, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_word.restype = u64
        L.synth_word.argtypes = [u64, u64, u64]
        L.synth_bf16_from_double.restype = ctypes.c_uint16
        L.synth_bf16_from_double.argtypes = [dbl]
        L.synth_normal_bf16.restype = None
        L.synth_normal_bf16.argtypes = [u64, u64, u64, u64, dbl, vp]
        L.synth_normal_f64.restype = None
        L.synth_normal_f64.argtypes = [u64, u64, u64, u64, vp]
        L.synth_permutation.restype = None
        L.synth_permutation.argtypes = [u64, u64, i32, vp]
        L.synth_fp8_codes.restype = None
        L.synth_fp8_codes.argtypes = [u64, u64, u64, u64, vp]
        L.synth_uniform_f32.restype = None
        L.synth_uniform_f32.argtypes = [u64, u64, u64, u64, ctypes.c_float, ctypes.c_float, vp]
        _lib = L
    return _lib


def normal_bf16(seed: int, stream: int, shape, sigma: float, offset: int = 0,
                out: np.ndarray | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of sigma * N(0,1) draws number
    offset .. offset+prod(shape)-1 of stream (seed, stream)."""
    n = int(np.prod(shape)) if len(shape) else 1
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    if n:
        lib().synth_normal_bf16(seed, stream, offset, n, float(sigma),
                                out.ctypes.data_as(ctypes.c_void_p))
    return out


def normal_f64(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        lib().synth_normal_f64(seed, stream, offset, n, out.ctypes.data_as(ctypes.c_void_p))
    return out


def fp8_codes(seed: int, stream: int, shape, offset: int = 0,
              out: np.ndarray | None = None) -> np.ndarray:
    """uint8 codes number offset .. offset+prod(shape)-1 of an 8-bit weight
    stream (E4M3 bit layout; see gen.c for the draw)."""
    n = int(np.prod(shape)) if len(shape) else 1
    if out is None:
        out = np.empty(shape, dtype=np.uint8)
    assert out.dtype == np.uint8 and out.flags.c_contiguous and out.size == n
    if n:
        lib().synth_fp8_codes(seed, stream, offset, n, out.ctypes.data_as(ctypes.c_void_p))
    return out


def uniform_f32(seed: int, stream: int, n: int, lo: float, hi: float, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        lib().synth_uniform_f32(seed, stream, offset, n, lo, hi, out.ctypes.data_as(ctypes.c_void_p))
    return out


def bf16_from_double(v: float) -> int:
    return int(lib().synth_bf16_from_double(float(v)))


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """A seeded permutation of 1..n (int32)."""
    out = np.empty(n, dtype=np.int32)
    lib().synth_permutation(seed, stream, n, out.ctypes.data_as(ctypes.c_void_p))
    return out


def zipf_bias(seed: int, E: int, s: float) -> np.ndarray:
    """Fixed per-expert logit bias b_e = -s * ln(r_e), r a seeded permutation
    of the ranks 1..E, so exp(b_e) is proportional to the Zipf(s) weight
    r_e^-s.  Returned as float32 (the precision the layer takes it in)."""
    r = permutation(seed, STREAM_BIAS, E).astype(np.float64)
    return (-s * np.log(r)).astype(np.float32)


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns, nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)
