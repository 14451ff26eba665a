"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle into a temporary tree, plants one mistake in the C
source (a wrong tie rule, bit order, scale, dropped term, transposed operand,
missing clip, signed absmax; for the threshold quantizer a non-strict
comparison, a dropped factor or sign, the mean over the kept weights only),
rebuilds it with gcc and runs every oracle pin file against that copy in a
subprocess; at least one pin must fail.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("float r = rintf(t);", "float r = roundf(t);"),                       # ties away from zero
    ("byte |= code << (2 * i);", "byte |= code << (6 - 2 * i);"),          # MSB-first packing
    ("float inv = 127.0f / st;", "float inv = 128.0f / st;"),              # wrong int8 range
    ("h[i] = (gp * gp) * u[i];", "h[i] = gp * u[i];"),                     # ReLU not squared
    ("float c = (s[t] / 127.0f) * gamma;", "float c = s[t] * gamma;"),     # missing 1/127
    ("row += fabs((double)w[r * k + c]);", "row += (double)w[r * k + c];"),  # mean W, not mean|W|
    ("if (r < -1.0f) r = -1.0f;", ""),                                     # one-sided clip
    ("(int32_t)wt[r * k + c]", "(int32_t)wt[c * n + r]"),                  # transposed weights
    ("if (a > amax) amax = a;", "if (row[c] > amax) amax = row[c];"),      # max x, not max|x|
    ("(packed[r * kb + c / 4] >> (2 * (c % 4)))", "(packed[r * kb + c / 4] >> (6 - 2 * (c % 4)))"),  # K-major field order
    # 4-bit activations
    ("fabsf(row[c]) >= tau ?", "fabsf(row[c]) > tau ?"),                    # ties at the top-K threshold dropped
    ("if (a <= 0.25f) c = 0;", "if (a < 0.25f) c = 0;"),                   # E2M1 tie away from even
    ("const float inv = 6.0f / st;", "const float inv = 7.0f / st;"),      # wrong FP4 range
    ("const float tau = mag[keep - 1];", "const float tau = mag[keep > 1 ? keep - 2 : 0];"),  # off-by-one top-K
    # threshold quantizer
    ("if (a > delta) {", "if (a >= delta) {"),                              # >= instead of strict >
    ("const float delta = factor * mean;", "const float delta = mean;"),    # factor dropped
    ("(int8_t)((v > 0.0f) - (v < 0.0f))", "(int8_t)1"),                    # sign dropped
    ("row += (double)a;", "row += (double)a; kept += 1.0;"),                # alpha over the kept count
]
# the kept-count mutant also needs its counter declared and used
EXTRA = {
    "row += (double)a; kept += 1.0;": [("double total = 0.0;\n    for (int64_t r = 0; r < n; ++r) {\n        double row = 0.0;\n        for (int64_t c = 0; c < k; ++c) {\n            const float v",
                                        "double total = 0.0, kept = 0.0;\n    for (int64_t r = 0; r < n; ++r) {\n        double row = 0.0;\n        for (int64_t c = 0; c < k; ++c) {\n            const float v"),
                                       ("const double kept_mean = total / ((double)n * (double)k);",
                                        "const double kept_mean = kept > 0.0 ? total / kept : 0.0;")],
}


# mistakes planted in the Python part of the oracle (the RMS norm)
PY_MUTANTS = [
    ("ms = np.float32(s_sum / k)", "ms = np.float32(s_sum / (k - 1))"),              # biased mean
    ("d = np.float32(ms + NORM_EPS)", "d = np.float32(ms)"),                           # epsilon dropped
    ("r = np.float32(np.float32(1.0) / np.sqrt(d))", "r = np.float32(np.float32(1.0) / d)"),  # no square root
    ("            row = row * g", "            row = row"),                           # gain dropped
    ("rescale_q(acc, s, gamma, 12.0)", "rescale_q(acc, s, gamma, 6.0)"),                  # A4 step not doubled
]


@pytest.mark.parametrize("old,new,lang", [(o, n, "c") for o, n in MUTANTS] + [(o, n, "py") for o, n in PY_MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, old, new, lang):
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "test_oracle_mutants.py"))
    src = tmp_path / "oracle" / ("bitlinear_oracle.c" if lang == "c" else "__init__.py")
    text = src.read_text()
    assert text.count(old) == 1, old
    text = text.replace(old, new)
    for a, b in EXTRA.get(new, []):
        assert text.count(a) == 1, a
        text = text.replace(a, b)
    src.write_text(text)
    subprocess.run([sys.executable, str(tmp_path / "oracle" / "build.py")], check=True,
                   stdout=subprocess.DEVNULL)
    pins = sorted(f"tests/{f}" for f in os.listdir(tmp_path / "tests")
                  if f.startswith("test_oracle_pins") and f.endswith(".py"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *pins],
                       cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "planted mistake went unnoticed:\n" + r.stdout[-2000:]
