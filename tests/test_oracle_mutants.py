"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle into a temporary tree, plants one mistake in the C
source (a wrong tie rule, bit order, scale, dropped term, transposed operand,
missing clip, signed absmax), rebuilds it with gcc and runs the pin tests
against that copy in a subprocess; at least one pin must fail.
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
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_pins_catch_planted_mistake(tmp_path, old, new):
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "test_oracle_mutants.py"))
    src = tmp_path / "oracle" / "bitlinear_oracle.c"
    text = src.read_text()
    assert old in text
    src.write_text(text.replace(old, new))
    subprocess.run([sys.executable, str(tmp_path / "oracle" / "build.py")], check=True,
                   stdout=subprocess.DEVNULL)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode != 0, "planted mistake went unnoticed:\n" + r.stdout[-2000:]
