"""The oracle's pins catch plausible mistakes.  Each case plants one mistake
in a scratch copy of oracle.c (CPU only), rebuilds that copy, and runs the pin
suites against it: at least one pin must fail.  The real oracle is never
modified."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_oracle_gating.py", "tests/test_oracle_fp8.py"]

MUTATIONS = [
    ("sigmoid gate includes the bias", "        gate[k] = probs[best];\n", "        gate[k] = key[best];\n"),
    ("sigmoid selection ignores the bias", "            key[e] = probs[e] + b;", "            key[e] = probs[e];"),
    ("sigmoid sign flipped", "probs[e] = 1.0 / (1.0 + exp(-acc));", "probs[e] = 1.0 / (1.0 + exp(acc));"),
    ("renormalisation skipped",
     "        for (int k = 0; k < K; ++k) gate[k] /= z;\n    }\n    if (K == 0",
     "        (void)z;\n    }\n    if (K == 0"),
    ("forced-routing renormalisation skipped",
     "                if (s->flags & ORACLE_RENORM)\n                    for (int k = 0; k < K; ++k) gate[k] /= z;",
     "                (void)z;"),
    ("softmax bias dropped", "            probs[e] = acc + b;", "            probs[e] = acc;"),
    ("ties to the higher index", "(best < 0 || key[e] > key[best])", "(best < 0 || key[e] >= key[best])"),
    ("margin from scores, not keys", "*margin = key[idx[K - 1]] - key[next];",
     "*margin = probs[idx[K - 1]] - probs[next];"),
    ("silu sign flipped", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("residual dropped", "res * xt[j] + sh[j] + ro[j]", "sh[j] + ro[j]"),
    ("up projection reads W1", "b += wat(w3, i, d, j) * x_t[j];", "b += wat(w1, i, d, j) * x_t[j];"),
    ("softmax denominator skips the last expert", "            z += probs[e];\n", "            z += e + 1 < E ? probs[e] : 0.0;\n"),
    ("shared experts skipped", "for (int si = 0; si < s->Ks; ++si) {", "for (int si = 0; si < 0; ++si) {"),
    ("gate taken from the next expert", "        gate[k] = probs[best];\n", "        gate[k] = probs[(best + 1) % E];\n"),
    ("e4m3 exponent bias 8", "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3 subnormals one binade low", "v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    ("e4m3 mantissa reversed", "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)(7 - m) / 8.0, e - 7);"),
    ("8-bit row scale from the neighbouring row", "e4m3_value[w->q[i]] * (double)w->scale[row]",
     "e4m3_value[w->q[i]] * (double)w->scale[row ^ 1]"),
    ("8-bit activation ties away from zero", "if (dd < bd || (dd == bd && (q & 1) == 0)) {",
     "if (dd < bd || dd == bd) {"),
    ("8-bit activation scale one binade high", "    while (ldexp(448.0, e - 1) >= amax) --e;\n    return e;",
     "    while (ldexp(448.0, e - 1) >= amax) --e;\n    return e + 1;"),
    ("8-bit activation scale not applied", "for (int j = 0; j < d; ++j) xr[j] = ldexp(oracle_e4m3(q[j]), e);",
     "for (int j = 0; j < d; ++j) xr[j] = oracle_e4m3(q[j]) + 0 * e;"),
    ("8-bit activations into W2 skipped", "        oracle_quantize_act8(hq, 1, inter, q, &e);\n        for (int i = 0; i < inter; ++i) h[i] = ldexp(oracle_e4m3(q[i]), e);",
     "        (void)e;"),
    ("h truncated to bf16 before its codes", "hq[i] = oracle_bf16_nearest(h[i]);",
     "{ const float f = (float)h[i]; uint32_t u; memcpy(&u, &f, 4); hq[i] = (uint16_t)(u >> 16); }"),
    ("bf16 rounding ties away from zero", "r = ldexp(nearbyint(ldexp(f, 8)), e2 - 8);", "r = ldexp(round(ldexp(f, 8)), e2 - 8);"),
    ("h of the shared experts quantised too", "&sw2[si], xt, h, y, NULL, NULL);", "&sw2[si], xt, h, y, hq, q);"),
    ("8-bit activations also fed to the shared experts",
     "expert_ffn(d, s->Is, &sw1[si], &sw3[si], &sw2[si], xt, h, y, NULL, NULL);",
     "expert_ffn(d, s->Is, &sw1[si], &sw3[si], &sw2[si], xr, h, y, NULL, NULL);"),
]


# Mistakes in the backward (oracle_backward); its pins are in their own file.
BWD_MUTATIONS = [
    ("silu derivative without the z (1 - sig) term",
     "const double dsilu = sg * (1.0 + a[i] * (1.0 - sg));", "const double dsilu = sg;"),
    ("up-projection gradient uses W3 x instead of silu(W1 x)",
     "const double db = dh[i] * (a[i] * sg);", "const double db = dh[i] * b[i];"),
    ("dh not scaled by the gate", "    for (int i = 0; i < inter; ++i) dh[i] *= g;\n", "\n"),
    ("W2^T pairs the wrong output row", "dh[i] += w * dO[o];", "dh[i] += w * dO[(o + 1) % d];"),
    ("renormalised gate backward drops the common term",
     "ds[idx[k]] += (dg[k] - sg) / z;", "ds[idx[k]] += dg[k] / z;"),
    ("softmax backward drops the mean term", "dl[e] = pr[e] * (ds[e] - m);", "dl[e] = pr[e] * ds[e];"),
    ("sigmoid derivative missing (1 - s)", "dl[e] = pr[e] * (1.0 - pr[e]) * ds[e];",
     "dl[e] = pr[e] * ds[e];"),
    ("balance gradient weighted by mean score instead of hit rate",
     "ds[e] = K > 0 ? alpha * fe[e] / (double)T : 0.0;",
     "ds[e] = K > 0 ? alpha * mean_score[e] / (double)T : 0.0;"),
    ("dW2 without the gate", "            for (int i = 0; i < inter; ++i) h[i] *= gs[t];\n", "\n"),
    ("dW1 from the up-projection gradient", "r1[j] += da * xt[j];", "r1[j] += db * xt[j];"),
    ("residual gradient dropped", "acc[j] = (s->flags & ORACLE_NO_RESIDUAL) ? 0.0 : dO[j];",
     "acc[j] = 0.0;"),
    ("hit rate not divided by K",
     "fe[e] = K > 0 ? (double)E * (double)counts[e] / ((double)K * (double)T) : 0.0;",
     "fe[e] = K > 0 ? (double)E * (double)counts[e] / (double)T : 0.0;"),
    ("centroid gradient from the next token's affinity gradient",
     "const double g = dl_all[(size_t)t * E + e];",
     "const double g = dl_all[(size_t)((t + 1) % T) * E + e];"),
]


def _plant(tmp_path, name, old, new, pin_files):
    for sub in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.o"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    src = tmp_path / "oracle" / "oracle.c"
    code = src.read_text()
    assert old in code, f"mutation site not found: {name}"
    src.write_text(code.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *pin_files], cwd=tmp_path, capture_output=True, text=True,
                       env=dict(os.environ, PYTHONPATH=str(tmp_path)), timeout=600)
    assert r.returncode == 1, f"no pin caught '{name}':\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name,old,new", BWD_MUTATIONS, ids=[m[0] for m in BWD_MUTATIONS])
def test_planted_backward_mistake_fails_a_pin(tmp_path, name, old, new):
    _plant(tmp_path, name, old, new, ["tests/test_oracle_backward.py"])


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    _plant(tmp_path, name, old, new, PIN_FILES)
