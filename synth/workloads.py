"""The six layer shapes the build is measured and tested on, and their seeded
inputs.

Shapes follow the DeepSeekMoE configurations: the fine-grained expert count
E = N*m with inter-dim I = I_std/m ("DeepSeekMoE 深度解读报告", section 2.2),
K_s always-on shared experts (same page, section 2.3) and SwiGLU experts of
the DeepSeek-V3 shape d=7168, inter=2048 (the youleyou page's Expert module).
Weights and centroids are N(0, 0.006) (the 0.006 initialisation std of the
same report, section 3.3); activations x are N(0, 1).

Seeds: every workload names a weight seed (centroids and expert weights), an
activation seed (x) and, when it carries a Zipf bias, a bias seed.  The two
DeepSeek-V3-shape workloads (decode and prefill) share one weight set: they
are the same layer fed different batches.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import (STREAM_C, STREAM_DOUT, STREAM_Q1, STREAM_Q2, STREAM_Q3, STREAM_S1, STREAM_S2, STREAM_S3,
               STREAM_W1, STREAM_W2, STREAM_W3, STREAM_WS1, STREAM_WS2, STREAM_WS3, STREAM_X,
               fp8_codes, normal_bf16, uniform_f32, zipf_bias)

SIGMA_W = 0.006
SIGMA_X = 1.0
# 8-bit routed weights: the drawn E4M3 codes have an RMS value of about 134,
# so per-row scales of FP8_SCALE * U(0.5, 1.5) give weights of about the same
# size as the bf16 ones.
FP8_SCALE = SIGMA_W / 134.0


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    I: int
    K: int
    Ks: int
    Is: int
    wseed: int
    xseed: int
    zipf_s: float = 0.0
    bseed: int = 0
    note: str = ""

    @property
    def rows(self) -> int:
        return self.T * (self.K + self.Ks)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", T=128, d=512, E=16, I=256, K=4, Ks=1, Is=256,
                     wseed=1000, xseed=1000,
                     note="N=4 standard experts split m=4, top-4, 1 shared"),
    "2b": Workload("2b", T=2048, d=1280, E=63, I=896, K=7, Ks=1, Is=896,
                   wseed=1001, xseed=1001,
                   note="2B validation scale: 1 shared + 63 routed (m=4), top-7"),
    "16b": Workload("16b", T=4096, d=2048, E=64, I=1408, K=6, Ks=2, Is=1408,
                    wseed=1002, xseed=1002,
                    note="16B scale: 2 shared + 64 routed, top-6"),
    "16b_zipf": Workload("16b_zipf", T=4096, d=2048, E=64, I=1408, K=6, Ks=2, Is=1408,
                         wseed=1002, xseed=1002, zipf_s=1.1, bseed=1012,
                         note="16B scale with a fixed Zipf(1.1) per-expert logit bias"),
    "v3_decode": Workload("v3_decode", T=256, d=7168, E=256, I=2048, K=8, Ks=1, Is=2048,
                          wseed=1003, xseed=1003,
                          note="DeepSeek-V3 shape, 256-token decode batch (HBM-bound)"),
    "v3_prefill": Workload("v3_prefill", T=16384, d=7168, E=256, I=2048, K=8, Ks=1, Is=2048,
                           wseed=1003, xseed=1004, zipf_s=1.2, bseed=1004,
                           note="DeepSeek-V3 shape prefill with a Zipf(1.2) logit bias (MFMA-bound)"),
}


def gen_x(w: Workload) -> np.ndarray:
    return normal_bf16(w.xseed, STREAM_X, (w.T, w.d), SIGMA_X)


def gen_x_rows(w: Workload, tokens) -> np.ndarray:
    """Rows of x for the given token ids only (regenerated from the counter)."""
    out = np.empty((len(tokens), w.d), dtype=np.uint16)
    for i, t in enumerate(tokens):
        normal_bf16(w.xseed, STREAM_X, (w.d,), SIGMA_X, offset=int(t) * w.d, out=out[i])
    return out


def gen_dout(w: Workload, T: int | None = None) -> np.ndarray:
    """Upstream gradient dLoss/dout for a backward, N(0, 1) bf16 [T, d], from
    the activation seed on its own stream."""
    T = w.T if T is None else T
    return normal_bf16(w.xseed, STREAM_DOUT, (T, w.d), 1.0)


def gen_centroids(w: Workload) -> np.ndarray:
    return normal_bf16(w.wseed, STREAM_C, (w.E, w.d), SIGMA_W)


def gen_bias(w: Workload):
    return zipf_bias(w.bseed, w.E, w.zipf_s) if w.zipf_s else None


def gen_expert(w: Workload, e: int):
    """(w1[e], w3[e], w2[e]) of routed expert e, regenerated on its own."""
    n = w.I * w.d
    w1 = normal_bf16(w.wseed, STREAM_W1, (w.I, w.d), SIGMA_W, offset=e * n)
    w3 = normal_bf16(w.wseed, STREAM_W3, (w.I, w.d), SIGMA_W, offset=e * n)
    w2 = normal_bf16(w.wseed, STREAM_W2, (w.d, w.I), SIGMA_W, offset=e * n)
    return w1, w3, w2


def gen_routed(w: Workload):
    n = (w.E, w.I, w.d)
    w1 = normal_bf16(w.wseed, STREAM_W1, n, SIGMA_W)
    w3 = normal_bf16(w.wseed, STREAM_W3, n, SIGMA_W)
    w2 = normal_bf16(w.wseed, STREAM_W2, (w.E, w.d, w.I), SIGMA_W)
    return w1, w3, w2


def gen_shared(w: Workload):
    n = (w.Ks, w.Is, w.d)
    ws1 = normal_bf16(w.wseed, STREAM_WS1, n, SIGMA_W)
    ws3 = normal_bf16(w.wseed, STREAM_WS3, n, SIGMA_W)
    ws2 = normal_bf16(w.wseed, STREAM_WS2, (w.Ks, w.d, w.Is), SIGMA_W)
    return ws1, ws3, ws2


def gen_routed_fp8(w: Workload):
    """Routed weights as 8-bit E4M3 codes with one float32 scale per output
    row: (q1, s1, q3, s3, q2, s2), q1/q3 uint8 [E, I, d], s1/s3 [E, I], q2
    [E, d, I], s2 [E, d].  The weight is decode(q) * scale of its row."""
    q1 = fp8_codes(w.wseed, STREAM_Q1, (w.E, w.I, w.d))
    q3 = fp8_codes(w.wseed, STREAM_Q3, (w.E, w.I, w.d))
    q2 = fp8_codes(w.wseed, STREAM_Q2, (w.E, w.d, w.I))
    s1 = (uniform_f32(w.wseed, STREAM_S1, w.E * w.I, 0.5, 1.5) * np.float32(FP8_SCALE)).reshape(w.E, w.I)
    s3 = (uniform_f32(w.wseed, STREAM_S3, w.E * w.I, 0.5, 1.5) * np.float32(FP8_SCALE)).reshape(w.E, w.I)
    s2 = (uniform_f32(w.wseed, STREAM_S2, w.E * w.d, 0.5, 1.5) * np.float32(FP8_SCALE)).reshape(w.E, w.d)
    return q1, s1, q3, s3, q2, s2


def gen_all(w: Workload) -> dict:
    """Every input of the layer as host arrays (bf16 as uint16 bit patterns)."""
    w1, w3, w2 = gen_routed(w)
    ws1, ws3, ws2 = gen_shared(w)
    return dict(x=gen_x(w), C=gen_centroids(w), bias=gen_bias(w),
                w1=w1, w3=w3, w2=w2, ws1=ws1, ws3=ws3, ws2=ws2)
