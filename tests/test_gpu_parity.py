"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: packed bytes, gamma bits, int8 codes, per-token scales and int32
accumulators bit-exact; fp32 outputs within 1e-5 relative (they are expected to
be bit-exact too, since both sides use the same fp32 operation order).
Shapes span several tiles and ragged tails (k = 260, n = 7, m = 3, 17, 65) on
both the v_dot4 decode path (m <= 4) and the MFMA path (m > 4), and the full
workload sizes in the launch configuration the benchmark times, compared on
whole tensors (the oracle's OpenMP int32 product takes seconds to about a
minute at 2048 tokens). The accumulator extreme |acc| = 127 k is reached on
every contraction path.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests.gpu_util import assert_y_close, host, make_linear, to_dev  # noqa: E402


@pytest.fixture(scope="module")
def bl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_ternary_weight_bitlinear_amd as m
    m.load_library()
    return m


# ------------------------------------------------------------------ pack

@pytest.mark.parametrize("n,k", [(1, 4), (7, 260), (256, 256), (300, 2560), (2560, 6912), (6912, 2560),
                                 (14336, 4096)])
def test_pack_bit_exact(bl, n, k):
    w, p_ref, g_ref, _ = make_linear(90, 1, n, k)
    packed, gamma = bl.pack_weights(to_dev(w))
    assert host(gamma)[0].view(np.uint32) == np.float32(g_ref).view(np.uint32)
    np.testing.assert_array_equal(host(packed), p_ref)


def test_pack_zero_weights(bl):
    packed, gamma = bl.pack_weights(to_dev(np.zeros((5, 64), np.float32)))
    assert host(gamma)[0] == 0.0
    assert np.all(host(packed) == 0x55)


def test_pack_hand_worked(bl, golden):
    c = golden["linear_cases"][0]
    packed, gamma = bl.pack_weights(to_dev(np.array(c["w"], np.float32)))
    assert host(gamma)[0] == np.float32(c["gamma"])
    np.testing.assert_array_equal(host(packed), np.array(c["packed"], np.uint8))


# ------------------------------------------------------------------ act-quant

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m,k", [(1, 4), (3, 20), (4, 256), (5, 260), (2, 2560), (3, 6912), (2, 14336),
                                 (1, 16388), (64, 4096),
                                 (1030, 260), (1024, 8192), (1027, 8196)])  # many tokens, ragged and whole rows
def test_quant_act_bit_exact(bl, dtype, m, k):
    x = synth.activations(91, m, k, dtype=dtype, outlier_channels=min(3, k), outlier_scale=30.0)
    q, s = bl.quant_act(to_dev(x, dtype))
    q_ref, s_ref = oracle.quant_act(x, dtype)
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))


def test_quant_act_zero_token(bl):
    x = np.zeros((2, 64), np.float32)
    x[1, 5] = -2.5
    q, s = bl.quant_act(to_dev(x))
    q_ref, s_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(s), s_ref)


# ------------------------------------------------------------------ forward (small / ragged)

FWD_SHAPES = [
    (1, 4, 1), (1, 256, 256), (2, 260, 7), (3, 2560, 300), (4, 1024, 129),      # decode path
    (1, 2560, 6913), (3, 512, 1031), (1, 16384, 300), (2, 20000, 64),            # decode: ragged blocks, long k
    (6, 2560, 6913), (7, 6912, 2561), (8, 260, 33), (8, 20000, 64), (8, 16384, 300),  # decode, 5..8 tokens
    (9, 644, 40), (12, 4100, 77), (13, 2052, 45), (16, 6912, 2561), (16, 8192, 100),  # 9..16 tokens
    (8, 6912, 100), (16, 2560, 300),                                             # one-launch path, layer shapes
    (5, 256, 256), (17, 260, 33), (33, 512, 257), (64, 2560, 512), (65, 256, 300),  # MFMA paths
    (130, 640, 200), (300, 256, 130),
    (1, 256, 40000), (2, 512, 20000),  # decode: more than 64 rows per workgroup, one 8-chunk block per row
    (12, 1024, 4000), (16, 2048, 300),   # 5..16 tokens, quantized inside the launch (k >= 1024, m*k <= 32768)
    (20, 1000, 3000), (24, 2560, 700), (32, 4096, 300),  # 17..32 tokens: two token blocks, quantized rows
    (40, 2560, 700), (48, 1024, 1000), (64, 6912, 300), (50, 8192, 33),  # 33..64: several token passes
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m,k,n", FWD_SHAPES)
def test_forward_small(bl, dtype, m, k, n):
    w, p_ref, g_ref, _ = make_linear(92, 1, n, k)
    x = synth.activations(92, m, k, dtype=dtype, outlier_channels=2, outlier_scale=20.0)
    packed, gamma = bl.pack_weights(to_dev(w))
    y, acc = bl.forward(to_dev(x, dtype), packed, gamma, return_acc=True)
    r = oracle.forward(x, p_ref, g_ref, k, dtype)
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


def test_forward_hand_worked(bl, golden):
    for c in golden["linear_cases"]:
        packed, gamma = bl.pack_weights(to_dev(np.array(c["w"], np.float32)))
        y, acc = bl.forward(to_dev(np.array(c["x_f32"], np.float32)), packed, gamma, return_acc=True)
        np.testing.assert_array_equal(host(acc), c["acc"])
        want = np.array(c["y"] if "y" in c else c["y_real"], np.float64)
        np.testing.assert_allclose(host(y), want, rtol=1e-6, atol=0)


def test_forward_zero_weights_and_tokens(bl):
    for m in (1, 8):
        packed, gamma = bl.pack_weights(to_dev(np.zeros((16, 64), np.float32)))
        x = synth.activations(93, m, 64, dtype="f32")
        x[0] = 0.0
        y, acc = bl.forward(to_dev(x), packed, gamma, return_acc=True)
        assert np.all(host(acc) == 0) and np.all(host(y) == 0)


def test_gemm_i32_bit_exact(bl):
    rng = np.random.default_rng(5)
    for m, k, n in [(1, 64, 8), (9, 260, 70), (130, 1024, 300)]:
        q = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
        w, p_ref, _, wt = make_linear(94, 1, n, k)
        acc = bl.gemm_i32(to_dev(q), to_dev(p_ref))
        np.testing.assert_array_equal(host(acc), q.astype(np.int64) @ wt.astype(np.int64).T)


# The 1..64-token kernel on quantized rows (bmma) owns tiles of RB 16-row
# blocks x TB 16-token blocks, splits the tokens over TS workgroups and gives
# each of its 8 waves NQ quads of 64-input chunks; the shapes below reach
# every RB in {1, 2, 4} and TB in {1..4} with ragged rows, tokens and chunk
# quads (the tile the kernel's cost model picks is noted per shape).
BMMA_SHAPES = [
    (17, 260, 4100),    # RB 2, TB 2; 5 chunks (a partial quad); 4100 % 32 = 4 rows in the last tile
    (33, 1100, 10000),  # RB 4, TB 3; 18 chunks
    (49, 1000, 4100),   # RB 4, TB 2, two token slices
    (49, 1000, 10000),  # RB 4, TB 4
    (17, 2600, 10000),  # RB 4, TB 2, two quads per wave; 41 chunks
    (64, 6912, 2561),   # RB 4, TB 1, four token slices, four quads per wave; one row in the last tile
    (33, 260, 6913),    # RB 2, TB 3
    (5, 8192, 300),     # RB 1, TB 1, 5 tokens (too many inputs for the one-launch kernel)
    (40, 4100, 1000),   # RB 1, TB 1, three token slices, three quads per wave; 65 chunks
    (57, 1100, 4099),   # RB 4, TB 2, two token slices; 3 rows in the last tile
    (20, 5000, 6000),   # RB 4, TB 1, two token slices, three quads per wave; 79 chunks
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m,k,n", BMMA_SHAPES)
def test_forward_bmma_tiles(bl, dtype, m, k, n):
    w, p_ref, g_ref, _ = make_linear(93, 1, n, k)
    x = synth.activations(93, m, k, dtype=dtype, outlier_channels=2, outlier_scale=20.0)
    packed, gamma = bl.pack_weights(to_dev(w))
    y, acc = bl.forward(to_dev(x, dtype), packed, gamma, return_acc=True)
    r = oracle.forward(x, p_ref, g_ref, k, dtype)
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


@pytest.mark.parametrize("m,k,n", [(33, 1100, 10000), (20, 5000, 6000), (49, 1000, 4100)])
def test_gemm_i32_bmma_tiles(bl, m, k, n):
    rng = np.random.default_rng(m * 7919 + k)
    q = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    w, p_ref, _, wt = make_linear(95, 1, n, k)
    acc = bl.gemm_i32(to_dev(q), to_dev(p_ref))
    np.testing.assert_array_equal(host(acc), q.astype(np.int64) @ wt.astype(np.int64).T)


# Shapes whose best GEMM tiling would leave its last round over the 256 CUs at
# most half full: the columns of the full rounds run as one launch and the rest
# as a second one with smaller tiles, writing into the same output rows.
# 2561 x 15488: 1063 tiles of 256x192, split at column 13248; 1153 x 34304:
# 1080 tiles, split at 29376 (the tail on 128-token tiles).
@pytest.mark.parametrize("m,k,n", [(2561, 256, 15488), (1153, 192, 34304)])
def test_forward_gemm_column_split(bl, m, k, n):
    w, p_ref, g_ref, _ = make_linear(97, 1, n, k)
    x = synth.activations(97, m, k, dtype="bf16", outlier_channels=2, outlier_scale=20.0)
    packed, gamma = bl.pack_weights(to_dev(w))
    y, acc = bl.forward(to_dev(x, "bf16"), packed, gamma, return_acc=True)
    r = oracle.forward(x, p_ref, g_ref, k, "bf16")
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


def test_gemm_i32_column_split(bl):
    m, k, n = 2561, 128, 15488
    rng = np.random.default_rng(11)
    q = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    w, p_ref, _, wt = make_linear(98, 1, n, k)
    acc = bl.gemm_i32(to_dev(q), to_dev(p_ref))
    np.testing.assert_array_equal(host(acc), q.astype(np.int64) @ wt.astype(np.int64).T)


# the largest sizes the boundary accepts (BL_MAX_DIM = 2^20 inputs or outputs,
# BL_MAX_TOKENS = 2^22 tokens), each with the other dimensions small
MAX_SHAPES = [(2, 1 << 20, 5), (1, 20, 1 << 20), (1 << 22, 4, 3)]


@pytest.mark.parametrize("m,k,n", MAX_SHAPES)
def test_forward_maximum_sizes(bl, m, k, n):
    w, p_ref, g_ref, _ = make_linear(96, 1, n, k)
    x = synth.activations(96, m, k, dtype="f32", outlier_channels=2, outlier_scale=20.0)
    packed, gamma = bl.pack_weights(to_dev(w))
    assert host(gamma)[0].view(np.uint32) == np.float32(g_ref).view(np.uint32)
    np.testing.assert_array_equal(host(packed), p_ref)
    y, acc = bl.forward(to_dev(x), packed, gamma, return_acc=True)
    r = oracle.forward(x, p_ref, g_ref, k, "f32")
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


def test_forward_deterministic(bl):
    w, _, _, _ = make_linear(95, 1, 6912, 2560)
    packed, gamma = bl.pack_weights(to_dev(w))
    for m in (1, 4, 64, 256):
        x = to_dev(synth.activations(95, m, 2560, dtype="bf16"), "bf16")
        first = host(bl.forward(x, packed, gamma))
        for _ in range(5):
            assert np.array_equal(host(bl.forward(x, packed, gamma)).view(np.uint32), first.view(np.uint32))


# ------------------------------------------------------------------ workload sizes

def _check_forward_full(bl, cfg, m, k, n, tid, dtype="bf16", **act):
    """Whole-tensor parity of one BitLinear layer: packed bytes, gamma bits,
    int32 accumulators bit-exact, y within 1e-5 relative."""
    w, p_ref, g_ref, wt = make_linear(cfg, tid, n, k)
    x = synth.activations(cfg, m, k, dtype=dtype, **act)
    packed, gamma = bl.pack_weights(to_dev(w))
    np.testing.assert_array_equal(host(packed), p_ref)
    assert host(gamma)[0].view(np.uint32) == np.float32(g_ref).view(np.uint32)
    y, acc = bl.forward(to_dev(x, dtype), packed, gamma, return_acc=True)
    r = oracle.forward(x, p_ref, g_ref, k, dtype)
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


@pytest.mark.parametrize("k,n", [(2560, 6912), (6912, 2560)])
def test_workload_decode_gemv(bl, k, n):
    _check_forward_full(bl, 2, 1, k, n, "up" if n > k else "down",
                        outlier_channels=round(0.01 * k), outlier_scale=30.0)


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_workload_batched_decode_layer(bl, m):
    for tid, (k, n) in zip(("qkv", "o", "gate", "up", "down"), synth.WORKLOADS[3]["mats"]):
        _check_forward_full(bl, 3, m, k, n, tid)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("k,n", [(2560, 6912), (6912, 2560)])
def test_workload_prefill_gemm(bl, k, n):
    _check_forward_full(bl, 4, 2048, k, n, "up" if n > k else "down", heavy_channels=round(0.01 * k))


# The accumulator's extreme |acc| = 127 k (the bound of the integer product):
# every weight +-1 (all |w| equal, so gamma = |w| and w / gamma = +-1 exactly),
# every activation of a token equal (s = |x|, q = +-127). Rows alternate in
# sign, tokens alternate in sign, so both +127 k and -127 k occur. One case per
# contraction path: decode GEMV (m <= 4), the 5..64-token kernel quantizing
# inside the launch or reading quantized rows, the long-k kernel for 5..64
# tokens, and the tiled GEMM; k = 14336 (the 8B down projection) and k near
# 2^20, where 127 k needs more than 24 bits and (float)acc rounds.
EXTREME = [
    (1, 14336, 96), (1, 57344, 40), (1, 1 << 20, 8), (3, 14336, 70),  # GEMV; k = 2^20 runs the long-k kernel
    (8, 4096, 300), (8, 8192, 300), (40, 6912, 130),                  # 5..64 tokens, k <= 8192
    (40, 14336, 130), (9, (1 << 20) - 4, 16),                         # 5..64 tokens, long k
    (300, 14336, 70), (130, (1 << 20) - 4, 40),                       # tiled GEMM
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("m,k,n", EXTREME)
def test_accumulator_extreme(bl, m, k, n):
    w = np.full((n, k), 0.25, np.float32)
    w[1::2] = -0.25
    x = np.full((m, k), 2.0, np.float32)   # s = 2, 127 / s = 63.5 exactly, q = +-127
    x[1::2] = -2.0
    packed, gamma = bl.pack_weights(to_dev(w))
    y, acc = bl.forward(to_dev(x), packed, gamma, return_acc=True)
    p_ref, g_ref, _ = oracle.pack_weights(w)
    r = oracle.forward(x, p_ref, g_ref, k, "f32")
    sign = np.where(np.arange(m)[:, None] % 2 == 0, 1, -1) * np.where(np.arange(n)[None, :] % 2 == 0, 1, -1)
    np.testing.assert_array_equal(r["acc"], 127 * k * sign)   # the oracle reaches the bound itself
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


# ------------------------------------------------------------------ FFN

def _ffn_case(bl, cfg, m, hid, f, dtype="bf16"):
    x = synth.activations(cfg, m, hid, dtype=dtype)
    dev_w, ref_w = {}, {}
    for name, shape in (("gate", (f, hid)), ("up", (f, hid)), ("down", (hid, f))):
        w, p_ref, g_ref, _ = make_linear(cfg, name, *shape)
        dev_w[name] = bl.pack_weights(to_dev(w))
        ref_w[name] = (p_ref, g_ref)
    y, hq, hs = bl.ffn(to_dev(x, dtype), dev_w["gate"], dev_w["up"], dev_w["down"], return_hq=True)
    r = oracle.ffn(x, ref_w["gate"], ref_w["up"], ref_w["down"], hid, f, dtype)
    np.testing.assert_array_equal(host(hq), r["qh"])
    np.testing.assert_array_equal(host(hs).view(np.uint32), r["sh"].view(np.uint32))
    assert_y_close(host(y), r["y"])


@pytest.mark.parametrize("m,hid,f", [(1, 256, 512), (3, 260, 516), (4, 512, 1024), (5, 256, 512),
                                     (33, 260, 516), (130, 512, 768),
                                     (1, 256, 20000),  # gate/up pair with more than 64 rows per workgroup
                                     (2, 8, 1 << 20),  # the largest ffn width the boundary accepts
                                     (300, 256, 33024)])  # gate/up pair as two launches (columns split at 27200)
def test_ffn_small(bl, m, hid, f):
    _ffn_case(bl, 96, m, hid, f)


# the gate/up pair on bmma (two weight streams per tile): RB 2 with TB 2, 4
# and 3, and RB 1 with two token slices; the down projections on RB 1 / 2
@pytest.mark.parametrize("m,hid,f", [(17, 260, 4100), (49, 1000, 4100), (33, 1100, 6916), (24, 2600, 2000)])
def test_ffn_bmma_tiles(bl, m, hid, f):
    _ffn_case(bl, 97, m, hid, f)


def test_ffn_hand_worked(bl, golden):
    c = golden["ffn_case"]
    mats = [bl.pack_weights(to_dev(np.array(c[key], np.float32))) for key in ("w_gate", "w_up", "w_down")]
    xb = synth.f32_to_bf16_bits(np.array(c["x_f32"], np.float32))
    y, hq, hs = bl.ffn(to_dev(xb, "bf16"), *mats, return_hq=True)
    np.testing.assert_array_equal(host(hq), c["qh"])
    np.testing.assert_array_equal(host(hs), np.array(c["sh"], np.float32))
    np.testing.assert_array_equal(host(y), np.array(c["y"], np.float32))


def test_workload_ffn_8b_decode(bl):
    _ffn_case(bl, 5, 1, 4096, 14336)


@pytest.mark.timeout(900)
def test_workload_ffn_8b_prefill(bl):
    _ffn_case(bl, 5, 2048, 4096, 14336)


# ------------------------------------------------------------------ HIP graph capture

@pytest.mark.parametrize("m,k,n", [(1, 2560, 6912), (3, 1024, 300), (8, 2560, 700), (64, 2560, 512),
                                   (300, 512, 640)])
def test_graph_replay_matches_eager(bl, m, k, n):
    """The library enqueues only kernels (no allocation, no memset), so a captured
    forward must reproduce the eager result on every replay."""
    w, _, _, _ = make_linear(97, 1, n, k)
    packed, gamma = bl.pack_weights(to_dev(w))
    x = to_dev(synth.activations(97, m, k, dtype="bf16"), "bf16")
    ws_bytes = bl.workspace_size(bl.OP_FORWARD, m, k, n)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    eager = host(bl.forward(x, packed, gamma, workspace=ws if ws_bytes else None)).copy()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bl.forward(x, packed, gamma, out=y, workspace=ws if ws_bytes else None)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        bl.forward(x, packed, gamma, out=y, workspace=ws if ws_bytes else None)
    for rep in range(4):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y).view(np.uint32), eager.view(np.uint32), err_msg=f"replay {rep}")
        # unrelated eager work on the same buffers between replays
        bl.forward(x * 2, packed, gamma, out=y, workspace=ws if ws_bytes else None)
        torch.cuda.synchronize()


# ------------------------------------------------------------------ threshold quantizer

@pytest.mark.parametrize("n,k,factor", [(1, 4, 0.7), (7, 260, 0.7), (256, 256, 0.6), (300, 2560, 0.75),
                                        (6912, 2560, 0.7), (14336, 4096, 0.7), (5, 64, 0.0)])
def test_pack_threshold_bit_exact(bl, n, k, factor):
    w = synth.weights(98, 1, n, k)
    p_ref, a_ref, _, d_ref = oracle.pack_weights_threshold(w, factor)
    packed, alpha, delta = bl.pack_weights_threshold(to_dev(w), factor)
    assert host(delta)[0].view(np.uint32) == np.float32(d_ref).view(np.uint32)
    assert host(alpha)[0].view(np.uint32) == np.float32(a_ref).view(np.uint32)
    np.testing.assert_array_equal(host(packed), p_ref)


def test_pack_threshold_hand_worked(bl, golden):
    for c in golden["threshold_cases"]:
        packed, alpha, delta = bl.pack_weights_threshold(to_dev(np.array(c["w"], np.float32)), c["factor"])
        assert host(delta)[0] == np.float32(c["delta"]) and host(alpha)[0] == np.float32(c["alpha"])
        np.testing.assert_array_equal(host(packed), np.array(c["packed"], np.uint8))
        if "x_f32" in c:
            y, acc = bl.forward(to_dev(np.array(c["x_f32"], np.float32)), packed, alpha, return_acc=True)
            np.testing.assert_array_equal(host(acc), c["acc"])
            np.testing.assert_array_equal(host(y), np.array(c["y"], np.float32))


@pytest.mark.parametrize("m,k,n", [(1, 2560, 6912), (8, 2560, 700), (300, 6912, 256)])
def test_forward_threshold_weights(bl, m, k, n):
    """The threshold quantizer's codes and alpha go through the same forward."""
    w = synth.weights(99, 1, n, k)
    x = synth.activations(99, m, k, dtype="bf16")
    p_ref, a_ref, _, _ = oracle.pack_weights_threshold(w, 0.7)
    packed, alpha, _ = bl.pack_weights_threshold(to_dev(w), 0.7)
    y, acc = bl.forward(to_dev(x, "bf16"), packed, alpha, return_acc=True)
    r = oracle.forward(x, p_ref, a_ref, k, "bf16")
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


# ------------------------------------------------------------------ RMS norm before the quantization

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m,k,gain", [(1, 4, False), (3, 260, True), (4, 2560, True), (7, 6912, False),
                                      (64, 4096, True), (2, 16388, True), (1027, 8196, False), (2, 20000, True)])
def test_quant_act_norm_bit_exact(bl, dtype, m, k, gain):
    x = synth.activations(140, m, k, dtype=dtype, outlier_channels=min(3, k), outlier_scale=30.0)
    g = (1.0 + 0.25 * synth.normal(141, k)).astype(np.float32) if gain else None
    q, s = bl.quant_act_norm(to_dev(x, dtype), to_dev(g) if gain else None)
    q_ref, s_ref = oracle.quant_act_norm(x, dtype, g)
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(q), q_ref)


def test_quant_act_norm_hand_worked(bl, golden):
    for c in golden["norm_cases"]:
        g = to_dev(np.array(c["gain"], np.float32)) if "gain" in c else None
        q, s = bl.quant_act_norm(to_dev(np.array(c["x_f32"], np.float32)), g)
        np.testing.assert_array_equal(host(q), c["q"])
        np.testing.assert_array_equal(host(s), np.array(c["s"], np.float32))


@pytest.mark.parametrize("m,k,n", [(1, 2560, 6912), (1, 6912, 2560), (3, 260, 70), (8, 2560, 700),
                                   (40, 6912, 300), (50, 14336, 64), (300, 2560, 256), (2048, 2560, 6912)])
def test_forward_norm(bl, m, k, n):
    w, p_ref, g_ref, _ = make_linear(142, 1, n, k)
    x = synth.activations(142, m, k, dtype="bf16", outlier_channels=3, outlier_scale=20.0)
    gain = (1.0 + 0.25 * synth.normal(143, k)).astype(np.float32)
    packed, gamma = bl.pack_weights(to_dev(w))
    y, acc = bl.forward_norm(to_dev(x, "bf16"), packed, gamma, to_dev(gain), return_acc=True)
    r = oracle.forward_norm(x, p_ref, g_ref, k, "bf16", gain)
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


# One bf16 token: the norm runs in the decode kernel's prologue (fp64 sum of
# squares over its 512 threads), with and without the gain, k with a ragged
# 64-input block, and up to four resident 16-input groups per thread.
@pytest.mark.parametrize("k,n,gain", [(2576, 300, True), (16384, 100, False), (20000, 64, True), (64, 8, False),
                                      (6912, 2560, False)])
def test_forward_norm_decode(bl, k, n, gain):
    w, p_ref, g_ref, _ = make_linear(144, 1, n, k)
    x = synth.activations(144, 1, k, dtype="bf16", outlier_channels=3, outlier_scale=20.0)
    g = (1.0 + 0.25 * synth.normal(145, k)).astype(np.float32) if gain else None
    packed, gamma = bl.pack_weights(to_dev(w))
    y, acc = bl.forward_norm(to_dev(x, "bf16"), packed, gamma, to_dev(g) if gain else None, return_acc=True)
    r = oracle.forward_norm(x, p_ref, g_ref, k, "bf16", g)
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


# ------------------------------------------------------------------ decode FFN skipping zero channels of h

@pytest.mark.parametrize("n,k", [(4, 4), (8, 260), (300, 512), (4096, 14336)])
def test_pack_kmajor_bit_exact(bl, n, k):
    w, p_ref, _, _ = make_linear(150, 1, n, k)
    pt = bl.pack_kmajor(to_dev(p_ref))
    np.testing.assert_array_equal(host(pt), oracle.pack_kmajor(p_ref, k))


def _ffn_sparse_case(bl, cfg, m, hid, f, dtype="bf16", x=None):
    x = synth.activations(cfg, m, hid, dtype=dtype) if x is None else x
    dev_w, ref_w = {}, {}
    for name, shape in (("gate", (f, hid)), ("up", (f, hid)), ("down", (hid, f))):
        w, p_ref, g_ref, _ = make_linear(cfg, name, *shape)
        dev_w[name] = bl.pack_weights(to_dev(w))
        ref_w[name] = (p_ref, g_ref)
    down_t = (bl.pack_kmajor(dev_w["down"][0]), dev_w["down"][1])
    y, hq, hs = bl.ffn_sparse(to_dev(x, dtype), dev_w["gate"], dev_w["up"], down_t, return_hq=True)
    r = oracle.ffn(x, ref_w["gate"], ref_w["up"], ref_w["down"], hid, f, dtype)
    np.testing.assert_array_equal(host(hq), r["qh"])
    np.testing.assert_array_equal(host(hs).view(np.uint32), r["sh"].view(np.uint32))
    assert_y_close(host(y), r["y"])
    # the dense FFN gives the same bits
    y_dense = bl.ffn(to_dev(x, dtype), dev_w["gate"], dev_w["up"], dev_w["down"])
    np.testing.assert_array_equal(host(y).view(np.uint32), host(y_dense).view(np.uint32))
    return r


@pytest.mark.parametrize("m,hid,f", [(1, 256, 512), (2, 256, 1000), (3, 272, 516), (4, 512, 1024),
                                     (1, 1024, 20000), (1, 4096, 14336), (4, 4096, 14336)])
def test_ffn_sparse(bl, m, hid, f):
    _ffn_sparse_case(bl, 160, m, hid, f)


def test_ffn_sparse_repeated_calls(bl):
    """Calls in a row on one workspace, different inputs: every call writes all
    of the scratch it reads, so each matches the oracle."""
    hid, f = 512, 2048
    ws = torch.empty(bl.workspace_size(bl.OP_FFN_SPARSE, 2, hid, f), dtype=torch.uint8, device="cuda")
    mats = {name: make_linear(161, name, *shape) for name, shape in
            (("gate", (f, hid)), ("up", (f, hid)), ("down", (hid, f)))}
    dev = {k: bl.pack_weights(to_dev(v[0])) for k, v in mats.items()}
    down_t = (bl.pack_kmajor(dev["down"][0]), dev["down"][1])
    for rep in range(4):
        x = synth.activations(170 + rep, 2, hid, dtype="bf16")
        y = bl.ffn_sparse(to_dev(x, "bf16"), dev["gate"], dev["up"], down_t, workspace=ws)
        r = oracle.ffn(x, mats["gate"][1:3], mats["up"][1:3], mats["down"][1:3], hid, f, "bf16")
        assert_y_close(host(y), r["y"])


def test_ffn_sparse_all_zero_and_dense_h(bl):
    """Degenerate sparsity: every channel of h zero (x = 0), and no channel zero
    (h > 0 everywhere: gate and up weights all positive, x > 0)."""
    hid, f = 256, 512
    x0 = np.zeros((1, hid), np.float32)
    _ffn_sparse_case(bl, 162, 1, hid, f, dtype="f32", x=x0)
    dev_w, ref_w = {}, {}
    pos = np.full((f, hid), 0.01, np.float32)
    for name, w in (("gate", pos), ("up", pos), ("down", synth.weights(163, "down", hid, f))):
        p_ref, g_ref, _ = oracle.pack_weights(w)
        dev_w[name] = bl.pack_weights(to_dev(w))
        ref_w[name] = (p_ref, g_ref)
    x = np.abs(synth.activations(163, 1, hid, dtype="f32")) + np.float32(0.5)
    down_t = (bl.pack_kmajor(dev_w["down"][0]), dev_w["down"][1])
    y, hq, hs = bl.ffn_sparse(to_dev(x), dev_w["gate"], dev_w["up"], down_t, return_hq=True)
    r = oracle.ffn(x, ref_w["gate"], ref_w["up"], ref_w["down"], hid, f, "f32")
    assert np.all(r["qh"] != 0)
    np.testing.assert_array_equal(host(hq), r["qh"])
    assert_y_close(host(y), r["y"])


# ------------------------------------------------------------------ 4-bit activations (W1.58A4)

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m,k,keep", [(1, 4, 2), (3, 260, None), (4, 2560, None), (7, 6912, None), (5, 100, 1),
                                      (2, 64, 64), (64, 4096, 1000), (2, 16388, None), (1027, 8196, None),
                                      (2, 20000, 7)])
def test_quant_act_a4_bit_exact(bl, dtype, m, k, keep):
    x = synth.activations(180, m, k, dtype=dtype, outlier_channels=min(3, k), outlier_scale=30.0)
    q, s = bl.quant_act_a4(to_dev(x, dtype), keep)
    q_ref, s_ref = oracle.quant_act_a4(x, dtype, keep)
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(q), q_ref)


def test_quant_act_a4_hand_worked(bl, golden):
    for c in golden["a4_cases"]:
        q, s = bl.quant_act_a4(to_dev(np.array(c["x_f32"], np.float32)), c["keep"])
        np.testing.assert_array_equal(host(q), c["q"], err_msg=c["name"])
        np.testing.assert_array_equal(host(s), np.array(c["s"], np.float32))
        if "w" in c:
            packed, gamma = bl.pack_weights(to_dev(np.array(c["w"], np.float32)))
            y, acc = bl.forward_a4(to_dev(np.array(c["x_f32"], np.float32)), packed, gamma, c["keep"],
                                   return_acc=True)
            np.testing.assert_array_equal(host(acc), c["acc"])
            np.testing.assert_array_equal(host(y), np.array(c["y"], np.float32))


def test_quant_act_a4_ties_everywhere(bl):
    """Many equal magnitudes (bf16 rounding of small integers): every entry tied
    with the threshold is kept on both sides."""
    x = np.round(synth.activations(181, 16, 1024, dtype="f32") * 4).astype(np.float32)
    q, s = bl.quant_act_a4(to_dev(x), 512)
    q_ref, s_ref = oracle.quant_act_a4(x, "f32", 512)
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(s), s_ref)


def test_quant_act_a4_e2m1_rounding_edges(bl):
    """With the row's absmax at 6 the E2M1 input is x itself: every midpoint of
    the grid with both signs, the floats just below and above each midpoint,
    the grid values and a few points near them, all kept."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(7)), grid,
                           np.float32([5.999, 4.999, 0.001])])
    row = np.concatenate([vals, -vals, np.float32([6.0])]).astype(np.float32)
    row = np.concatenate([row, np.zeros((-len(row)) % 4, np.float32)])
    x = np.stack([row, row[::-1].copy()])
    q, s = bl.quant_act_a4(to_dev(x), x.shape[1])
    q_ref, s_ref = oracle.quant_act_a4(x, "f32", x.shape[1])
    assert np.all(s_ref == 6.0)
    np.testing.assert_array_equal(host(s), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)


@pytest.mark.parametrize("m,k,n", [(1, 2560, 6912), (1, 6912, 2560), (3, 260, 70), (8, 2560, 700),
                                   (40, 6912, 300), (50, 14336, 64), (300, 2560, 256), (2048, 2560, 6912)])
def test_forward_a4(bl, m, k, n):
    w, p_ref, g_ref, _ = make_linear(182, 1, n, k)
    x = synth.activations(182, m, k, dtype="bf16", heavy_channels=max(1, k // 100))
    packed, gamma = bl.pack_weights(to_dev(w))
    y, acc = bl.forward_a4(to_dev(x, "bf16"), packed, gamma, return_acc=True)
    r = oracle.forward_a4(x, p_ref, g_ref, k, "bf16")
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


# One bf16 token: the 4-bit codes are made in the decode kernel's prologue
# (the top-K select over its 512 threads). keep = 1, half, all; ragged 64-input
# blocks; up to four resident groups per thread; and a token whose magnitudes
# repeat (ties at tau: every entry with |x| >= tau is kept).
@pytest.mark.parametrize("k,n,keep", [(2576, 300, 1288), (16384, 100, 1), (20000, 64, 20000), (64, 8, 32),
                                      (6912, 2560, 3456), (2560, 6912, None)])
def test_forward_a4_decode(bl, k, n, keep):
    w, p_ref, g_ref, _ = make_linear(183, 1, n, k)
    x = synth.activations(183, 1, k, dtype="bf16", heavy_channels=max(1, k // 100))
    packed, gamma = bl.pack_weights(to_dev(w))
    y, acc = bl.forward_a4(to_dev(x, "bf16"), packed, gamma, keep, return_acc=True)
    r = oracle.forward_a4(x, p_ref, g_ref, k, "bf16", keep)
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"])


def test_forward_a4_decode_ties(bl):
    k, n = 1024, 96
    w, p_ref, g_ref, _ = make_linear(184, 1, n, k)
    levels = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -3.0], np.float32)
    x = levels[np.arange(k) % len(levels)][None, :]
    xb = synth.f32_to_bf16_bits(x)
    packed, gamma = bl.pack_weights(to_dev(w))
    for keep in (1, 100, 300, 512, 1000, k):
        y, acc = bl.forward_a4(to_dev(xb, "bf16"), packed, gamma, keep, return_acc=True)
        r = oracle.forward_a4(xb, p_ref, g_ref, k, "bf16", keep)
        np.testing.assert_array_equal(host(acc), r["acc"])
        assert_y_close(host(y), r["y"])

