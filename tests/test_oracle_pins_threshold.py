"""Pins for the oracle's threshold weight quantizer ("BitNet 三元权重阈值优化工程实践",
section on the core principle of ternary threshold optimization): delta =
factor * mean|W|, w~ = sign(w) where |w| > delta, alpha = mean(|W| * mask).

* hand-worked cases (tests/golden/hand_worked.json), including a weight exactly
  at delta (the strict > decides) and the fp32 rounding of 0.7 * mean;
* exact rational re-derivation of mean, delta, mask and alpha;
* the Gaussian closed forms: zero fraction erf(0.7 / sqrt(pi)) and
  alpha / sigma = 2 phi(0.7 sqrt(2 / pi));
* special cases: factor 0 reduces to the sign quantizer with alpha = mean|W|
  (the absmean gamma), a factor above max|w| / mean keeps nothing; invariants
  under W -> 2^e W and W -> -W.
"""
from fractions import Fraction
from math import erf, exp, pi, sqrt

import numpy as np
import pytest

import oracle
import synth


def f32(x):
    return np.asarray(x, dtype=np.float32)


def _round_f32(q: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational (ties to even)."""
    cand = np.float32(float(q))
    opts = (cand, np.nextafter(cand, np.float32(np.inf)), np.nextafter(cand, np.float32(-np.inf)))
    return np.float32(min(opts, key=lambda c: (abs(Fraction(float(c)) - q), int(np.float32(c).view(np.uint32)) & 1)))


def test_hand_worked_threshold(golden):
    for c in golden["threshold_cases"]:
        w = f32(c["w"])
        packed, alpha, wt, delta = oracle.pack_weights_threshold(w, c["factor"])
        assert delta == np.float32(c["delta"]), c["name"]
        assert alpha == np.float32(c["alpha"]), c["name"]
        np.testing.assert_array_equal(wt, c["wt"], err_msg=c["name"])
        np.testing.assert_array_equal(packed, np.array(c["packed"], np.uint8), err_msg=c["name"])
        if "x_f32" in c:
            r = oracle.forward(f32(c["x_f32"]), packed, alpha, c["k"], "f32")
            np.testing.assert_array_equal(r["q"], c["q"])
            np.testing.assert_array_equal(r["acc"], c["acc"])
            np.testing.assert_array_equal(r["y"], f32(c["y"]))


@pytest.mark.parametrize("seed,n,k,factor", [(1, 8, 16, 0.7), (2, 33, 20, 0.7), (3, 16, 64, 0.6),
                                             (4, 4, 256, 0.75)])
def test_threshold_matches_exact_rationals(seed, n, k, factor):
    w = synth.weights(700 + seed, "W", n, k)
    wt, alpha, delta = oracle.threshold_ternarize(w, factor)
    mean = _round_f32(sum((abs(Fraction(float(v))) for v in w.ravel()), Fraction(0)) / w.size)
    want_delta = np.float32(np.float32(factor) * mean)      # one correctly rounded fp32 product
    assert delta == want_delta
    mask = np.abs(w) > want_delta
    np.testing.assert_array_equal(wt, (np.sign(w) * mask).astype(np.int8))
    kept = sum((abs(Fraction(float(v))) for v in w[mask]), Fraction(0))
    assert alpha == _round_f32(kept / w.size)


def test_threshold_gaussian_closed_forms():
    # N(0, sigma^2): mean|W| -> sigma sqrt(2/pi), t = 0.7 sqrt(2/pi) in units of sigma;
    # zero iff |z| <= t: P = erf(t / sqrt 2) = erf(0.7 / sqrt(pi)) = 0.4235;
    # alpha / sigma = E|z| 1(|z| > t) = 2 phi(t).
    t = 0.7 * sqrt(2.0 / pi)
    p0 = erf(t / sqrt(2.0))
    a_sigma = 2.0 * exp(-t * t / 2.0) / sqrt(2.0 * pi)
    assert abs(p0 - 0.42350) < 1e-4 and abs(a_sigma - 0.68266) < 1e-4
    w = synth.weights(1, "W", 256, 256)
    wt, alpha, _ = oracle.threshold_ternarize(w, 0.7)
    frac = float(np.mean(wt == 0))
    assert abs(frac - p0) < 4 * sqrt(p0 * (1 - p0) / wt.size)
    assert abs(float(alpha) / 0.02 - a_sigma) < 0.01
    assert abs(float(np.mean(wt == 1)) - float(np.mean(wt == -1))) < 0.02


def test_threshold_special_cases():
    w = synth.weights(710, "W", 12, 40)
    w[0, :5] = 0.0
    wt, alpha, delta = oracle.threshold_ternarize(w, 0.0)        # keep every non-zero weight
    assert delta == 0.0
    np.testing.assert_array_equal(wt, np.sign(w).astype(np.int8))
    assert alpha == oracle.absmean(w)
    big = float(np.abs(w).max() / oracle.absmean(w)) * 1.01     # delta above max|w|
    wt, alpha, _ = oracle.threshold_ternarize(w, big)
    assert np.all(wt == 0) and alpha == 0.0
    wt, alpha, delta = oracle.threshold_ternarize(np.zeros((3, 8), np.float32), 0.7)
    assert np.all(wt == 0) and alpha == 0.0 and delta == 0.0


def test_threshold_invariants():
    w = synth.weights(711, "W", 16, 64)
    p, a, wt, d = oracle.pack_weights_threshold(w, 0.7)
    p2, a2, wt2, d2 = oracle.pack_weights_threshold(w * np.float32(0.25), 0.7)
    np.testing.assert_array_equal(p, p2)
    assert a2 == a * np.float32(0.25) and d2 == d * np.float32(0.25)
    p3, a3, wt3, d3 = oracle.pack_weights_threshold(-w, 0.7)
    np.testing.assert_array_equal(wt3, -wt)
    np.testing.assert_array_equal(p3.astype(np.int32), 0xAA - p.astype(np.int32))
    assert a3 == a and d3 == d
    np.testing.assert_array_equal(oracle.unpack(p, 64), wt)      # same 2-bit layout as absmean
