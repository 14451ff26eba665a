"""bitlinear_forward_noalloc (the forward whose scratch is a library-owned
device array, for callers that cannot allocate) against bitlinear_forward with
a caller workspace, both through the C ABI: int32 accumulators bit-exact and
fp32 outputs identical, on two calls in a row, the second smaller; sizes past
the array's limit are rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle  # noqa: F401  (the comparison is with the existing entry point)
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests.gpu_util import host, to_dev  # noqa: E402

BL_OK, BL_ERR_WORKSPACE = 0, 5
SCRATCH = 32 << 20


@pytest.fixture(scope="module")
def bl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_ternary_weight_bitlinear_amd as m
    lib = m.load_library()
    f = lib.bitlinear_forward_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return m


def _noalloc(bl, x, packed, gamma, n):
    m, k = x.shape
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    acc = torch.full((m, n), -7, dtype=torch.int32, device="cuda")
    dt = 1 if x.dtype == torch.bfloat16 else 0
    st = bl.load_library().bitlinear_forward_noalloc(
        x.data_ptr(), dt, m, k, packed.data_ptr(), gamma.data_ptr(), n, y.data_ptr(), acc.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    return st, y, acc


# (m, k, n) pairs: each pair's second call is smaller than its first, and each
# case needs scratch (m > 4 or k % 64 != 0); the first uses most of the array
PAIRS = [
    ((2048, 6912, 512), (300, 2560, 700)),   # tiled GEMM: 14.2 MB of permuted activations, then less
    ((64, 6912, 1000), (20, 1000, 300)),     # 5..64 tokens with quantized rows; ragged k (padded weights)
    ((16, 2560, 6912), (8, 2500, 70)),       # quantization inside the launch, then ragged k
    ((3, 260, 50), (1, 100, 7)),             # decode kernel with ragged k (padded weight copy)
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_forward(bl, first, second):
    for call, (m, k, n) in enumerate((first, second)):
        w = synth.weights(120 + call, "W", n, k)
        x = to_dev(synth.activations(120 + call, m, k, dtype="bf16", outlier_channels=3, outlier_scale=20.0),
                   "bf16")
        packed, gamma = bl.pack_weights(to_dev(w))
        y_ref, acc_ref = bl.forward(x, packed, gamma, return_acc=True)
        st, y, acc = _noalloc(bl, x, packed, gamma, n)
        assert st == BL_OK, st
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(acc), host(acc_ref), err_msg=f"call {call} {(m, k, n)}")
        np.testing.assert_array_equal(host(y).view(np.uint32), host(y_ref).view(np.uint32),
                                      err_msg=f"call {call} {(m, k, n)}")


def test_noalloc_rejects_sizes_past_the_scratch(bl):
    m, k, n = 4096, 8192, 64                   # 32 MiB of permuted activations alone
    assert bl.workspace_size(bl.OP_FORWARD, m, k, n) > SCRATCH
    x = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    packed = torch.full((n, k // 4), 0x55, dtype=torch.uint8, device="cuda")
    gamma = torch.ones(1, dtype=torch.float32, device="cuda")
    st, y, acc = _noalloc(bl, x, packed, gamma, n)
    torch.cuda.synchronize()
    assert st == BL_ERR_WORKSPACE
    assert torch.isnan(y).all() and (acc == -7).all()      # nothing was enqueued


def test_noalloc_decode_needs_no_scratch(bl):
    m, k, n = 1, 2560, 6912
    w = synth.weights(130, "W", n, k)
    x = to_dev(synth.activations(130, m, k, dtype="bf16"), "bf16")
    packed, gamma = bl.pack_weights(to_dev(w))
    y_ref, acc_ref = bl.forward(x, packed, gamma, return_acc=True)
    st, y, acc = _noalloc(bl, x, packed, gamma, n)
    assert st == BL_OK
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), host(acc_ref))
    np.testing.assert_array_equal(host(y).view(np.uint32), host(y_ref).view(np.uint32))
