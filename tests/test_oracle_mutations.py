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
    ("8-bit row scale from the neighbouring row", "oracle_e4m3(w->q[i]) * (double)w->scale[row]",
     "oracle_e4m3(w->q[i]) * (double)w->scale[row ^ 1]"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    for sub in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.o"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    src = tmp_path / "oracle" / "oracle.c"
    code = src.read_text()
    assert old in code, f"mutation site not found: {name}"
    src.write_text(code.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=tmp_path, capture_output=True, text=True,
                       env=dict(os.environ, PYTHONPATH=str(tmp_path)), timeout=600)
    assert r.returncode == 1, f"no pin caught '{name}':\n{r.stdout[-2000:]}"
