"""Pins for the oracle's RMS normalization before the activation quantization
(subln: "穿越1比特的奇幻旅程", section 架构创新; layer normalization with epsilon
1e-5: "BitNet 中使用直通估计器工程化三元权重训练", section 工程化训练流程与参数配置).

* hand-worked cases (tests/golden/hand_worked.json): an exactly representable
  root, the gain, a rounding tie after the gain, an all-zero token;
* an exact-rational re-derivation of S, ms and r;
* the float64 brute force x / sqrt(mean x^2 + 1e-5) * g, including rows small
  enough that epsilon matters;
* scale invariance of absmax quantization: without a gain, the codes of the
  normalized row differ from those of the raw row by at most one.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def f32(x):
    return np.asarray(x, dtype=np.float32)


def test_hand_worked_norm(golden):
    for c in golden["norm_cases"]:
        x = f32(c["x_f32"])
        gain = f32(c["gain"]) if "gain" in c else None
        xn = oracle.rms_norm(x, "f32", gain)
        if "xn_bits" in c:
            np.testing.assert_array_equal(xn.view(np.uint32), np.array(c["xn_bits"], np.uint32))
        if "xn" in c:
            np.testing.assert_array_equal(xn, f32(c["xn"]))
        q, s = oracle.quant_act_norm(x, "f32", gain)
        np.testing.assert_array_equal(q, c["q"], err_msg=c["name"])
        np.testing.assert_array_equal(s, f32(c["s"]), err_msg=c["name"])


def _fp32_round(q: Fraction) -> np.float32:
    cand = np.float32(float(q))
    opts = (cand, np.nextafter(cand, np.float32(np.inf)), np.nextafter(cand, np.float32(-np.inf)))
    return np.float32(min(opts, key=lambda c: (abs(Fraction(float(c)) - q), int(np.float32(c).view(np.uint32)) & 1)))


@pytest.mark.parametrize("seed,k", [(1, 16), (2, 100), (3, 260)])
def test_norm_scale_from_exact_rationals(seed, k):
    x = synth.activations(800 + seed, 3, k, dtype="f32", outlier_channels=2, outlier_scale=30.0)
    xn = oracle.rms_norm(x)
    for t in range(3):
        exact = sum((Fraction(float(v)) ** 2 for v in x[t]), Fraction(0))
        s64 = float(exact)                          # correctly rounded to fp64
        ms = np.float32(s64 / k)
        r = np.float32(np.float32(1.0) / np.sqrt(np.float32(ms + np.float32(1e-5))))
        np.testing.assert_array_equal(xn[t], x[t] * r)
        assert ms == _fp32_round(Fraction(s64) / k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 1e-3, 30.0])
def test_norm_against_float64(dtype, scale):
    x = synth.activations(810, 8, 512, dtype="f32", outlier_channels=4, outlier_scale=20.0) * np.float32(scale)
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    gain = (1.0 + 0.5 * synth.normal(811, 512)).astype(np.float32)
    xn = oracle.rms_norm(x, dtype, gain)
    xf = (synth.bf16_bits_to_f32(x) if dtype == "bf16" else x).astype(np.float64)
    ref = xf / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + 1e-5) * gain.astype(np.float64)
    np.testing.assert_allclose(xn, ref, rtol=2e-6, atol=0)


def test_norm_zero_token_and_codes():
    x = np.zeros((2, 64), np.float32)
    x[1, 3] = 5.0
    xn = oracle.rms_norm(x)
    assert np.all(xn[0] == 0) and np.isfinite(xn).all()
    q, s = oracle.quant_act_norm(x)
    assert np.all(q[0] == 0) and s[0] == np.float32(1e-5)
    assert q[1, 3] == 127 and np.count_nonzero(q[1]) == 1


def test_norm_leaves_codes_within_one():
    x = synth.activations(812, 16, 1024, dtype="bf16", outlier_channels=10, outlier_scale=30.0)
    q0, _ = oracle.quant_act(x, "bf16")
    q1, _ = oracle.quant_act_norm(x, "bf16")
    assert np.max(np.abs(q0.astype(np.int32) - q1.astype(np.int32))) <= 1
    assert np.mean(q0 != q1) < 0.01


def test_forward_norm_matches_dequantized_float64():
    m, k, n = 4, 320, 40
    x = synth.activations(813, m, k, dtype="bf16", outlier_channels=3, outlier_scale=20.0)
    gain = (1.0 + 0.25 * synth.normal(814, k)).astype(np.float32)
    p, g, wt = oracle.pack_weights(synth.weights(813, "W", n, k))
    r = oracle.forward_norm(x, p, g, k, "bf16", gain)
    deq = r["q"].astype(np.float64) * (r["s"].astype(np.float64) / 127.0)[:, None]
    y64 = deq @ (wt.astype(np.float64) * float(g)).T
    np.testing.assert_allclose(r["y"], y64, rtol=1e-5, atol=1e-30)
    np.testing.assert_array_equal(r["q"], oracle.quant_act(r["xn"], "f32")[0])
