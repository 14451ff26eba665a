"""Pins for the CPU oracle: each check ties it to something other than itself.

* hand-worked cases (tests/golden/hand_worked.json), computed by hand from the
  definitions, including round-half-even ties and the bit order of the packing;
* exact rational arithmetic (fractions) for the absmean scale;
* float64 re-derivations away from rounding ties for both quantizers;
* numpy integer matmul for the contraction; float64 brute force of the
  dequantized operands for the rescale and for the FFN composition;
* closed-form invariants (scale, sign, identity weights, one-hot tokens) and
  degenerate cases (zero weights, zero tokens), and the Gaussian zero fraction.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def f32(x):
    return np.asarray(x, dtype=np.float32)


# ------------------------------------------------------------ hand-worked

def test_hand_worked_linear(golden):
    c = golden["linear_cases"][0]
    w = f32(c["w"])
    packed, gamma, wt = oracle.pack_weights(w)
    assert gamma == np.float32(c["gamma"])
    np.testing.assert_array_equal(wt, c["wt"])
    np.testing.assert_array_equal(packed, np.array(c["packed"], dtype=np.uint8))
    r = oracle.forward(f32(c["x_f32"]), packed, gamma, c["k"], "f32")
    np.testing.assert_array_equal(r["q"], c["q"])
    np.testing.assert_array_equal(r["s"], f32(c["s"]))
    np.testing.assert_array_equal(r["acc"], c["acc"])
    np.testing.assert_array_equal(r["y"], f32(c["y"]))


def test_hand_worked_scale_and_zero_token(golden):
    c = golden["linear_cases"][1]
    packed, gamma, _ = oracle.pack_weights(f32(c["w"]))
    assert gamma == np.float32(c["gamma"])
    r = oracle.forward(f32(c["x_f32"]), packed, gamma, c["k"], "f32")
    np.testing.assert_array_equal(r["q"], c["q"])
    np.testing.assert_array_equal(r["s"], f32(c["s"]))
    np.testing.assert_array_equal(r["acc"], c["acc"])
    np.testing.assert_allclose(r["y"], np.array(c["y_real"]), rtol=1e-6, atol=0)


def test_hand_worked_ffn(golden):
    c = golden["ffn_case"]
    pg, gg, _ = oracle.pack_weights(f32(c["w_gate"]))
    pu, gu, _ = oracle.pack_weights(f32(c["w_up"]))
    pd, gd, _ = oracle.pack_weights(f32(c["w_down"]))
    assert (gg, gu, gd) == (np.float32(c["gamma_gate"]), np.float32(c["gamma_up"]),
                            np.float32(c["gamma_down"]))
    np.testing.assert_array_equal(pg, np.array(c["packed_gate"], np.uint8))
    np.testing.assert_array_equal(pu, np.array(c["packed_up"], np.uint8))
    np.testing.assert_array_equal(pd, np.array(c["packed_down"], np.uint8))
    xb = synth.f32_to_bf16_bits(f32(c["x_f32"]))
    assert np.array_equal(synth.bf16_bits_to_f32(xb), f32(c["x_f32"]))  # bf16-exact input
    r = oracle.ffn(xb, (pg, gg), (pu, gu), (pd, gd), c["hidden"], c["ffn"], "bf16")
    for key in ("q", "qh", "acc_down"):
        np.testing.assert_array_equal(r[key], c[key])
    for key in ("s", "g", "u", "h", "sh", "y"):
        np.testing.assert_array_equal(r[key], f32(c[key]), err_msg=key)


# ------------------------------------------------------------ weight scale

def _exact_mean_f32(w):
    tot = sum((abs(Fraction(float(v))) for v in w.ravel()), Fraction(0))
    mean = tot / w.size
    # correctly rounded fp32 of the exact rational: round the double nearest to it,
    # then check the neighbours for the fp32 nearest.
    cand = np.float32(float(mean))
    best = min((cand, np.nextafter(cand, np.float32(np.inf)), np.nextafter(cand, np.float32(-np.inf))),
               key=lambda c: (abs(Fraction(float(c)) - mean), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


@pytest.mark.parametrize("seed,n,k", [(11, 8, 16), (12, 33, 20), (13, 64, 64), (14, 1, 256)])
def test_absmean_matches_exact_rational_mean(seed, n, k):
    w = synth.weights(100 + seed, "W", n, k)
    assert oracle.absmean(w) == _exact_mean_f32(w)


def test_absmean_dyadic_closed_form():
    # |w| = j / 64 for j = 0..255 laid out as 16x16: sum = 255*256/2/64 = 510, mean = 510/256.
    w = (np.arange(256, dtype=np.float32) / 64.0).reshape(16, 16)
    w[::2] *= -1.0
    assert oracle.absmean(w) == np.float32(510.0 / 256.0)


# ------------------------------------------------------------ quantizers

def _near_half(t, tol):
    frac = np.abs(t - np.floor(t) - 0.5)
    return frac < tol


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_ternarize_is_nearest_clipped_integer(seed):
    w = synth.weights(200 + seed, "W", 64, 128)
    g = oracle.absmean(w)
    wt = oracle.ternarize(w, g)
    t = w.astype(np.float64) / np.float64(g)
    ok = ~_near_half(t, 1e-6)
    ref = np.clip(np.rint(t), -1, 1)
    np.testing.assert_array_equal(wt[ok], ref[ok])
    assert set(np.unique(wt)).issubset({-1, 0, 1})


def test_gaussian_zero_fraction():
    # absmean on N(0, sigma^2): zero iff |w| < gamma/2 with gamma -> sigma*sqrt(2/pi);
    # P(|Z| < sqrt(2/pi)/2) = erf(sqrt(1/pi)/2)*... = 0.31006 (closed form below).
    from math import erf, pi, sqrt
    p0 = erf(sqrt(2.0 / pi) / 2.0 / sqrt(2.0))
    w = synth.weights(1, "W", 256, 256)
    _, g, wt = oracle.pack_weights(w)
    frac = float(np.mean(wt == 0))
    sd = sqrt(p0 * (1 - p0) / wt.size)
    assert abs(p0 - 0.31006) < 1e-4
    assert abs(frac - p0) < 4 * sd
    assert abs(float(g) / 0.02 - sqrt(2.0 / pi)) < 0.01


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_act_against_float64(dtype):
    x = synth.activations(300, 16, 512, dtype=dtype, outlier_channels=5, outlier_scale=30.0)
    q, s = oracle.quant_act(x, dtype)
    xf = synth.bf16_bits_to_f32(x) if dtype == "bf16" else x
    amax = np.max(np.abs(xf), axis=1)
    np.testing.assert_array_equal(s, np.maximum(amax, np.float32(1e-5)))
    t = xf.astype(np.float64) * 127.0 / s[:, None].astype(np.float64)
    ok = ~_near_half(t, 1e-4)
    np.testing.assert_array_equal(q[ok], np.clip(np.rint(t), -127, 127)[ok])
    # the absmax element of every non-zero token maps to +-127
    np.testing.assert_array_equal(np.max(np.abs(q.astype(np.int32)), axis=1), 127)


def test_quant_act_invariants():
    x = synth.activations(301, 8, 256, dtype="f32")
    q, s = oracle.quant_act(x)
    q2, s2 = oracle.quant_act(x * np.float32(8.0))      # power-of-two scale
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s * np.float32(8.0), s2)
    q3, s3 = oracle.quant_act(-x)                          # sign symmetry
    np.testing.assert_array_equal(q3, -q)
    np.testing.assert_array_equal(s3, s)


def test_zero_token_uses_epsilon():
    q, s = oracle.quant_act(np.zeros((2, 8), np.float32))
    assert np.all(q == 0)
    np.testing.assert_array_equal(s, np.float32(1e-5))


# ------------------------------------------------------------ packing

def test_pack_roundtrip_and_no_code_three():
    w = synth.weights(400, "W", 37, 260)
    packed, g, wt = oracle.pack_weights(w)
    assert packed.shape == (37, 65)
    b = packed.astype(np.uint32)
    assert np.all((b & (b >> 1) & 0x55) == 0)
    np.testing.assert_array_equal(oracle.unpack(packed, 260), wt)


def test_pack_kmajor_hand_worked_and_round_trip(golden):
    c = golden["ffn_case"]
    pd = np.array(c["packed_down"], np.uint8)
    np.testing.assert_array_equal(oracle.pack_kmajor(pd, c["ffn"]), np.array(c["packed_down_kmajor"], np.uint8))
    w = synth.weights(404, "W", 36, 52)
    p, _, wt = oracle.pack_weights(w)
    pt = oracle.pack_kmajor(p, 52)
    assert pt.shape == (52, 9)
    np.testing.assert_array_equal(oracle.unpack(pt, 36), wt.T)
    np.testing.assert_array_equal(oracle.pack_kmajor(pt, 36), p)   # transposing twice is the identity


def test_unpack_rejects_code_three():
    with pytest.raises(ValueError):
        oracle.unpack(np.array([[0x55, 0xC0]], np.uint8), 8)


def test_zero_weights():
    packed, g, wt = oracle.pack_weights(np.zeros((4, 8), np.float32))
    assert g == 0.0
    assert np.all(packed == 0x55) and np.all(wt == 0)
    r = oracle.forward(np.ones((2, 8), np.float32), packed, g, 8)
    assert np.all(r["acc"] == 0) and np.all(r["y"] == 0)


def test_weight_invariants():
    w = synth.weights(401, "W", 16, 64)
    p, g, wt = oracle.pack_weights(w)
    p2, g2, wt2 = oracle.pack_weights(w * np.float32(4.0))
    np.testing.assert_array_equal(p, p2)
    assert g2 == g * np.float32(4.0)
    p3, g3, wt3 = oracle.pack_weights(-w)
    np.testing.assert_array_equal(wt3, -wt)
    # code -> 2 - code, i.e. byte -> 0xAA - byte (no borrows since codes <= 2)
    np.testing.assert_array_equal(p3.astype(np.int32), 0xAA - p.astype(np.int32))


def test_identity_weights_pin_rescale():
    k = 64
    w = np.eye(k, dtype=np.float32)
    p, g, wt = oracle.pack_weights(w)
    assert g == np.float32(1.0 / k)
    np.testing.assert_array_equal(wt, np.eye(k, dtype=np.int8))
    x = synth.activations(402, 3, k, dtype="f32")
    r = oracle.forward(x, p, g, k)
    np.testing.assert_array_equal(r["acc"], r["q"].astype(np.int32))
    want = r["q"].astype(np.float64) * r["s"][:, None].astype(np.float64) / 127.0 / k
    np.testing.assert_allclose(r["y"], want, rtol=1e-6, atol=0)


def test_one_hot_token_reads_a_weight_column():
    w = synth.weights(403, "W", 24, 32)
    p, g, wt = oracle.pack_weights(w)
    for k0 in (0, 1, 2, 3, 5, 31):
        x = np.zeros((1, 32), np.float32)
        x[0, k0] = 3.0
        r = oracle.forward(x, p, g, 32)
        np.testing.assert_array_equal(r["acc"][0], 127 * wt[:, k0].astype(np.int32))


# ------------------------------------------------------------ contraction and rescale

@pytest.mark.parametrize("m,k,n", [(1, 4, 1), (3, 260, 7), (17, 256, 33)])
def test_matmul_equals_numpy_int64(m, k, n):
    rng = np.random.default_rng(m * 1000 + n)
    q = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    wt = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    ref = q.astype(np.int64) @ wt.astype(np.int64).T
    np.testing.assert_array_equal(oracle.matmul_i32(q, wt), ref)


def test_extreme_accumulator():
    k = 14336
    q = np.full((1, k), -127, np.int8)
    wt = np.ones((2, k), np.int8)
    wt[1] = -1
    acc = oracle.matmul_i32(q, wt)
    assert acc[0, 0] == -127 * k and acc[0, 1] == 127 * k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_matches_dequantized_float64(dtype):
    m, k, n = 5, 320, 48
    x = synth.activations(500, m, k, dtype=dtype, outlier_channels=3, outlier_scale=20.0)
    w = synth.weights(500, "W", n, k)
    p, g, wt = oracle.pack_weights(w)
    r = oracle.forward(x, p, g, k, dtype)
    deq_x = r["q"].astype(np.float64) * (r["s"].astype(np.float64) / 127.0)[:, None]
    deq_w = wt.astype(np.float64) * np.float64(g)
    y64 = deq_x @ deq_w.T
    np.testing.assert_allclose(r["y"], y64, rtol=1e-5, atol=1e-30)


def test_sqrelu_gate_against_float64():
    rng = np.random.default_rng(7)
    g = rng.standard_normal(1000).astype(np.float32) * 3
    u = rng.standard_normal(1000).astype(np.float32) * 3
    h = oracle.sqrelu_gate(g, u)
    ref = np.maximum(g.astype(np.float64), 0) ** 2 * u.astype(np.float64)
    np.testing.assert_allclose(h, ref, rtol=1e-6, atol=0)
    assert np.all(h[g <= 0] == 0)


def test_ffn_matches_float64_composition():
    hid, ffn_dim, m = 64, 128, 3
    x = synth.activations(600, m, hid, dtype="bf16")
    pg, gg, wg = oracle.pack_weights(synth.weights(600, "gate", ffn_dim, hid))
    pu, gu, wu = oracle.pack_weights(synth.weights(600, "up", ffn_dim, hid))
    pd, gd, wd = oracle.pack_weights(synth.weights(600, "down", hid, ffn_dim))
    r = oracle.ffn(x, (pg, gg), (pu, gu), (pd, gd), hid, ffn_dim, "bf16")
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    s = np.maximum(np.abs(xf).max(1), 1e-5)
    q = np.clip(np.rint(xf * 127.0 / s[:, None]), -127, 127)
    deq = q * (s / 127.0)[:, None]
    g64 = deq @ (wg.astype(np.float64) * float(gg)).T
    u64 = deq @ (wu.astype(np.float64) * float(gu)).T
    h64 = np.maximum(g64, 0) ** 2 * u64
    np.testing.assert_allclose(r["h"], h64, rtol=1e-5, atol=1e-12)
    sh = np.abs(h64).max(1)
    qh = np.rint(h64 * 127.0 / sh[:, None])
    assert np.max(np.abs(r["qh"].astype(np.int32) - qh)) <= 1
    y64 = (qh * (sh / 127.0)[:, None]) @ (wd.astype(np.float64) * float(gd)).T
    # y differs from y64 only through the rare +-1 flips of q_h near rounding ties
    scale = np.abs(y64).max()
    assert np.max(np.abs(r["y"] - y64)) <= 2e-2 * scale
