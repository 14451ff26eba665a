"""Pins for the oracle's 4-bit activations (W1.58A4: "BitNet 1-bit LLM 的混合精度
微调技术", paragraph on progressive quantization: MinMax FP4 with E2M1 bits,
top-K sparsification of 50 %).

* hand-worked cases (tests/golden/hand_worked.json): the top-K threshold and
  its ties, every E2M1 midpoint, a zero token, and a forward with its output;
* the E2M1 rounding against a brute-force nearest-value search on the grid;
* a numpy re-derivation of the whole quantizer (sort for the threshold, grid
  search for the rounding) on random tokens;
* invariants: power-of-two scaling, sign symmetry, keep = k drops nothing,
  keep = 1 keeps only the largest magnitude;
* the forward against float64 brute force of the dequantized operands.
"""
import numpy as np
import pytest

import oracle
import synth

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
EVEN = np.array([True, False, True, False, True, False, True, False])  # mantissa bit 0


def f32(x):
    return np.asarray(x, dtype=np.float32)


def _nearest_doubled(v):
    a = abs(float(v))
    d = np.abs(GRID - a)
    best = np.flatnonzero(d == d.min())
    i = best[0] if len(best) == 1 else [j for j in best if EVEN[j]][0]
    c = int(round(2 * GRID[i]))
    return -c if v < 0 else c


def test_hand_worked_a4(golden):
    for c in golden["a4_cases"]:
        q, s = oracle.quant_act_a4(f32(c["x_f32"]), "f32", c["keep"])
        np.testing.assert_array_equal(q, c["q"], err_msg=c["name"])
        np.testing.assert_array_equal(s, f32(c["s"]), err_msg=c["name"])
        if "w" in c:
            p, g, _ = oracle.pack_weights(f32(c["w"]))
            r = oracle.forward_a4(f32(c["x_f32"]), p, g, c["k"], "f32", c["keep"])
            np.testing.assert_array_equal(r["acc"], c["acc"])
            np.testing.assert_array_equal(r["y"], f32(c["y"]))


def test_e2m1_rounding_brute_force():
    vals = list(GRID) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 100.0]
    rng = np.random.default_rng(3)
    vals += list(rng.uniform(0, 6.5, 2000).astype(np.float32))
    for v in vals:
        for sv in (v, -v):
            assert oracle.e2m1_doubled(sv) == _nearest_doubled(np.float32(sv)), sv


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("keep_frac", [0.5, 0.25, 1.0])
def test_a4_against_numpy(dtype, keep_frac):
    x = synth.activations(900, 6, 200, dtype=dtype, outlier_channels=3, outlier_scale=20.0)
    xf = synth.bf16_bits_to_f32(x) if dtype == "bf16" else x
    keep = max(1, int(np.ceil(keep_frac * 200)))
    q, s = oracle.quant_act_a4(x, dtype, keep)
    for t in range(6):
        mag = np.abs(xf[t])
        tau = np.sort(mag)[::-1][keep - 1]
        st = np.float32(max(mag.max(), np.float32(1e-5)))
        inv = np.float32(np.float32(6.0) / st)
        want = [(_nearest_doubled(np.float32(v * inv)) if a >= tau else 0) for v, a in zip(xf[t], mag)]
        np.testing.assert_array_equal(q[t], want)
        assert s[t] == st
        assert np.count_nonzero(mag >= tau) >= keep


def test_a4_invariants():
    x = synth.activations(901, 8, 256, dtype="f32")
    q, s = oracle.quant_act_a4(x)
    q2, s2 = oracle.quant_act_a4(x * np.float32(4.0))
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s2, s * np.float32(4.0))
    q3, s3 = oracle.quant_act_a4(-x)
    np.testing.assert_array_equal(q3, -q)
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 12)        # the max maps to +-6
    assert np.all(np.count_nonzero(q, axis=1) <= 128)                      # at most half survive (no ties)
    qa, _ = oracle.quant_act_a4(x, keep=256)
    assert np.count_nonzero(qa) > np.count_nonzero(q)
    q1, _ = oracle.quant_act_a4(x, keep=1)
    assert np.all(np.count_nonzero(q1, axis=1) == 1)
    assert set(np.unique(q)).issubset({-12, -8, -6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6, 8, 12})


def test_forward_a4_matches_dequantized_float64():
    m, k, n = 5, 320, 48
    x = synth.activations(902, m, k, dtype="bf16", outlier_channels=3, outlier_scale=20.0)
    p, g, wt = oracle.pack_weights(synth.weights(902, "W", n, k))
    r = oracle.forward_a4(x, p, g, k, "bf16")
    deq = r["q"].astype(np.float64) * (r["s"].astype(np.float64) / 12.0)[:, None]
    y64 = deq @ (wt.astype(np.float64) * float(g)).T
    np.testing.assert_allclose(r["y"], y64, rtol=1e-5, atol=1e-30)
    np.testing.assert_array_equal(r["acc"], r["q"].astype(np.int64) @ wt.astype(np.int64).T)
