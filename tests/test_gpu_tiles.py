"""GPU parity of every tile shape of the MFMA GEMM (m > 64 tokens), single
matrix and gate/up pair, against the CPU oracle on full tensors.

The GEMM picks a tile of 128*FM tokens x 32*FN features per problem. For each
shape the host can pick, these tests use the smallest token and feature counts
(neither a multiple of the tile) that select it, with k = 704 or 644 inputs:
eleven 64-input steps, more than the direct-load ring depth, so the ring runs
in its steady state and ends on an odd step; 644 also takes the padded-weight
path (k not a multiple of 64). With an even step count (k = 1536) the
128-token tiles load and synchronize once per pair of steps. Checked: int32 accumulators bit-exact, fp32
outputs within 1e-5 relative, FFN requantized h bit-exact.
"""
import math

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests.gpu_util import assert_y_close, host, make_linear, to_dev  # noqa: E402


def pick_tile(m, n, na):
    """Mirror of the host-side tile choice: least rounds over 256 CUs times the
    per-tile cost (MFMA blocks, their weight expansion, a fixed per-step term),
    among shapes with at most 14 (one matrix) accumulator blocks, or for the
    gate/up pair 12 on 128-token tiles or the 256x128 and 256x64 tiles."""
    best, best_cost = (1, 4), math.inf
    for fm in (2, 1):
        for fn in range(8, 1, -1):
            if na == 2 and not ((fm == 1 and 4 <= fn <= 6) or (fm == 2 and fn in (2, 4))):
                continue
            if na == 1 and (fn < 4 or fm * fn > 14):
                continue
            tiles = math.ceil(n / (32 * fn)) * math.ceil(m / (128 * fm))
            cost = math.ceil(tiles / 256) * (fm * fn * na * (1.0 + 0.2 / fm) + 3.0)
            if cost < best_cost:
                best_cost, best = cost, (fm, fn)
    return best


def ragged_shape(fm, fn, na):
    """Smallest (m, n) that selects tile (fm, fn), with m and n both ragged.
    For the gate/up pair n is the FFN width, which the down projection takes
    as its input count, so it stays a multiple of 4."""
    best = None
    for m in (65, 200, 300, 520, 1000, 1500, 2100, 3000, 4100, 6000, 8200):
        for n in (range(33, 16000, 7) if na == 1 else range(36, 16000, 4)):
            if pick_tile(m, n, na) != (fm, fn) or m % (128 * fm) == 0 or n % (32 * fn) == 0:
                continue
            if best is None or m * n < best[0]:
                best = (m * n, m, n)
    assert best is not None, (fm, fn, na)
    return best[1], best[2]


SINGLE = [(2, 4), (2, 5), (2, 6), (2, 7), (1, 4), (1, 5), (1, 6), (1, 7), (1, 8)]
PAIR = [(1, 4), (1, 5), (1, 6), (2, 4), (2, 2)]


@pytest.fixture(scope="module")
def bl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_ternary_weight_bitlinear_amd as m
    m.load_library()
    return m


CASES = [(fm, fn, 704 if fm == 2 else 644) for fm, fn in SINGLE] + [(1, fn, 1536) for fm, fn in SINGLE if fm == 1]


@pytest.mark.parametrize("fm,fn,k", CASES)
def test_gemm_tile_shapes(bl, fm, fn, k):
    """k = 1536 (24 steps, even): 128-token tiles take two steps per ring stage."""
    m, n = ragged_shape(fm, fn, 1)
    print(f"tile {128 * fm}x{32 * fn}: m={m} n={n} k={k}", flush=True)
    w, p_ref, g_ref, _ = make_linear(97, fm * 10 + fn, n, k)
    x = synth.activations(97, m, k, dtype="bf16", heavy_channels=max(1, k // 100))
    packed, gamma = bl.pack_weights(to_dev(w))
    y, acc = bl.forward(to_dev(x, "bf16"), packed, gamma, return_acc=True)
    r = oracle.forward(x, p_ref, g_ref, k, "bf16")
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


@pytest.mark.parametrize("fm,fn", [(2, 7), (1, 5)])
def test_gemm_i32_tile_shapes(bl, fm, fn):
    """The integer-only entry point (int8 q in, int32 out) on the same tiles."""
    m, n = ragged_shape(fm, fn, 1)
    k = 644
    w, p_ref, g_ref, _ = make_linear(98, fm * 10 + fn, n, k)
    x = synth.activations(98, m, k, dtype="f32")
    q, _ = oracle.quant_act(x, "f32")
    packed, _ = bl.pack_weights(to_dev(w))
    acc = bl.gemm_i32(to_dev(q), packed)
    r = oracle.forward(x, p_ref, g_ref, k, "f32")
    np.testing.assert_array_equal(host(acc), r["acc"])


@pytest.mark.parametrize("fm,fn", PAIR)
def test_ffn_pair_tile_shapes(bl, fm, fn):
    """Gate/up pair on one activation ring (h = relu(g)^2 * u in the epilogue),
    then the requantized h through the down projection (k = ffn, ragged)."""
    m, f = ragged_shape(fm, fn, 2)
    hid = 704
    x = synth.activations(99, m, hid, dtype="bf16")
    dev_w, ref_w = {}, {}
    for tid, (name, shape) in enumerate((("gate", (f, hid)), ("up", (f, hid)), ("down", (hid, f)))):
        w, p_ref, g_ref, _ = make_linear(99, 16 * fn + tid, *shape)
        dev_w[name] = bl.pack_weights(to_dev(w))
        ref_w[name] = (p_ref, g_ref)
    y, hq, hs = bl.ffn(to_dev(x, "bf16"), dev_w["gate"], dev_w["up"], dev_w["down"], return_hq=True)
    r = oracle.ffn(x, ref_w["gate"], ref_w["up"], ref_w["down"], hid, f, "bf16")
    np.testing.assert_array_equal(host(hq), r["qh"])
    np.testing.assert_array_equal(host(hs).view(np.uint32), r["sh"].view(np.uint32))
    assert_y_close(host(y), r["y"])
