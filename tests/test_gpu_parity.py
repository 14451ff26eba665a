"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: packed bytes, gamma bits, int8 codes, per-token scales and int32
accumulators bit-exact; fp32 outputs within 1e-5 relative (they are expected to
be bit-exact too, since both sides use the same fp32 operation order).
Shapes span several tiles and ragged tails (k = 260, n = 7, m = 3, 17, 65) on
both the v_dot4 decode path (m <= 4) and the MFMA path (m > 4), and the full
workload sizes in the launch configuration the benchmark times (oracle on
sampled tokens where the whole product would take too long on the CPU).
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

def _check_forward_full(bl, cfg, m, k, n, tid, dtype="bf16", sample=None, **act):
    w, p_ref, g_ref, wt = make_linear(cfg, tid, n, k)
    x = synth.activations(cfg, m, k, dtype=dtype, **act)
    packed, gamma = bl.pack_weights(to_dev(w))
    np.testing.assert_array_equal(host(packed), p_ref)
    y, acc = bl.forward(to_dev(x, dtype), packed, gamma, return_acc=True)
    rows = np.arange(m) if sample is None else sample
    r = oracle.forward(x[rows], p_ref, g_ref, k, dtype)
    np.testing.assert_array_equal(host(acc)[rows], r["acc"])
    assert_y_close(host(y)[rows], r["y"])


@pytest.mark.parametrize("k,n", [(2560, 6912), (6912, 2560)])
def test_workload_decode_gemv(bl, k, n):
    _check_forward_full(bl, 2, 1, k, n, "up" if n > k else "down",
                        outlier_channels=round(0.01 * k), outlier_scale=30.0)


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_workload_batched_decode_layer(bl, m):
    for tid, (k, n) in zip(("qkv", "o", "gate", "up", "down"), synth.WORKLOADS[3]["mats"]):
        _check_forward_full(bl, 3, m, k, n, tid)


@pytest.mark.parametrize("k,n", [(2560, 6912), (6912, 2560)])
def test_workload_prefill_gemm(bl, k, n):
    sample = np.unique(np.concatenate([np.arange(0, 2048, 97), [127, 128, 255, 256, 2046, 2047]]))
    _check_forward_full(bl, 4, 2048, k, n, "up" if n > k else "down", sample=sample,
                        heavy_channels=round(0.01 * k))


# ------------------------------------------------------------------ FFN

def _ffn_case(bl, cfg, m, hid, f, sample=None, dtype="bf16"):
    x = synth.activations(cfg, m, hid, dtype=dtype)
    dev_w, ref_w = {}, {}
    for name, shape in (("gate", (f, hid)), ("up", (f, hid)), ("down", (hid, f))):
        w, p_ref, g_ref, _ = make_linear(cfg, name, *shape)
        dev_w[name] = bl.pack_weights(to_dev(w))
        ref_w[name] = (p_ref, g_ref)
    y, hq, hs = bl.ffn(to_dev(x, dtype), dev_w["gate"], dev_w["up"], dev_w["down"], return_hq=True)
    rows = np.arange(m) if sample is None else sample
    r = oracle.ffn(x[rows], ref_w["gate"], ref_w["up"], ref_w["down"], hid, f, dtype)
    np.testing.assert_array_equal(host(hq)[rows], r["qh"])
    np.testing.assert_array_equal(host(hs)[rows].view(np.uint32), r["sh"].view(np.uint32))
    assert_y_close(host(y)[rows], r["y"])


@pytest.mark.parametrize("m,hid,f", [(1, 256, 512), (3, 260, 516), (4, 512, 1024), (5, 256, 512),
                                     (33, 260, 516), (130, 512, 768),
                                     (1, 256, 20000),  # gate/up pair with more than 64 rows per workgroup
                                     (2, 8, 1 << 20)])  # the largest ffn width the boundary accepts
def test_ffn_small(bl, m, hid, f):
    _ffn_case(bl, 96, m, hid, f)


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


def test_workload_ffn_8b_prefill(bl):
    _ffn_case(bl, 5, 2048, 4096, 14336, sample=np.array([0, 1, 255, 256, 1023, 2047]))


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
