"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/bitlinear.h declares, and rejects invalid arguments with the
documented status before anything is enqueued (fake, never-dereferenced
pointer values are enough for that)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_WORKSPACE, BL_ERR_HIP, BL_ERR_VALUE = range(8)
OP_FORWARD, OP_FFN, OP_PACK, OP_GEMM_I32, OP_PACK_THRESHOLD, OP_FORWARD_NORM, OP_FFN_SPARSE, OP_FORWARD_A4 = range(8)
A = 0x10000          # aligned fake device address (never dereferenced)
MIS = 0x10004        # 4-byte aligned only


@pytest.fixture(scope="module")
def lib():
    import bit_ternary_weight_bitlinear_amd as bl
    if not os.path.exists(bl.library_path()):
        from bit_ternary_weight_bitlinear_amd import build
        build.build()
    return bl.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("bitlinear_pack_weights", "bitlinear_quant_act", "bitlinear_forward", "bitlinear_ffn",
              "bitlinear_gemm_i32", "bitlinear_workspace_size", "bitlinear_status_string",
              "bitlinear_pack_weights_threshold", "bitlinear_quant_act_norm", "bitlinear_forward_norm",
              "bitlinear_pack_kmajor", "bitlinear_ffn_sparse", "bitlinear_quant_act_a4", "bitlinear_forward_a4"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(8):
        assert lib.bitlinear_status_string(s)
        assert not lib.bitlinear_status_string(s).startswith(b"unknown")
    assert b"unknown" in lib.bitlinear_status_string(99)


def test_workspace_size_rules(lib):
    ws = lib.bitlinear_workspace_size
    assert ws(OP_FORWARD, 1, 2560, 6912) == 0                     # decode path needs none
    assert ws(OP_FORWARD, 2048, 2560, 6912) >= 2048 * 2560          # qperm activations
    assert ws(OP_FORWARD, 1, 260, 7) >= 7 * 320 // 4                # padded weight copy for ragged k
    assert ws(OP_PACK, 0, 4096, 14336) >= 14336 * 8                 # per-row sums
    assert ws(OP_FFN, 1, 4096, 14336) >= 14336 * 4                  # h buffer
    assert ws(OP_GEMM_I32, 1, 256, 8) >= 256 * 256                  # qperm copy of q
    assert ws(OP_FORWARD, 0, 256, 256) == 0 and ws(OP_FORWARD, 1, 6, 8) == 0   # invalid shapes
    assert ws(9, 1, 256, 256) == 0 and ws(-1, 1, 256, 256) == 0


def test_op_numbering_matches_header():
    """bl_op: 0 = forward and 1 = FFN (the two per-batch calls), then pack and
    the bare integer product; the binding uses the same numbers."""
    text = open(HEADER).read()
    body = re.search(r"typedef enum \{([^}]*)\} bl_op;", text).group(1)
    vals = {k: int(v) for k, v in re.findall(r"(BL_OP_\w+)\s*=\s*(\d+)", body)}
    assert vals == {"BL_OP_FORWARD": OP_FORWARD, "BL_OP_FFN": OP_FFN, "BL_OP_PACK": OP_PACK,
                    "BL_OP_GEMM_I32": OP_GEMM_I32, "BL_OP_PACK_THRESHOLD": OP_PACK_THRESHOLD,
                    "BL_OP_FORWARD_NORM": OP_FORWARD_NORM, "BL_OP_FFN_SPARSE": OP_FFN_SPARSE,
                    "BL_OP_FORWARD_A4": OP_FORWARD_A4}
    import bit_ternary_weight_bitlinear_amd as bl
    assert (bl.OP_FORWARD, bl.OP_FFN, bl.OP_PACK, bl.OP_GEMM_I32, bl.OP_PACK_THRESHOLD,
            bl.OP_FORWARD_NORM, bl.OP_FFN_SPARSE, bl.OP_FORWARD_A4) == tuple(range(8))


def test_forward_argument_errors(lib):
    f = lib.bitlinear_forward
    assert f(None, 0, 1, 256, A, A, 8, A, None, None, 0, None) == BL_ERR_NULL
    assert f(A, 0, 1, 256, A, A, 8, None, None, None, 0, None) == BL_ERR_NULL
    assert f(A, 7, 1, 256, A, A, 8, A, None, None, 0, None) == BL_ERR_DTYPE
    assert f(A, 0, 0, 256, A, A, 8, A, None, None, 0, None) == BL_ERR_SHAPE
    assert f(A, 0, 1, 258, A, A, 8, A, None, None, 0, None) == BL_ERR_SHAPE
    assert f(A, 0, 1, 0, A, A, 8, A, None, None, 0, None) == BL_ERR_SHAPE
    assert f(A, 0, 1, 256, A, A, 0, A, None, None, 0, None) == BL_ERR_SHAPE
    # one past the largest accepted sizes (2^20 inputs or outputs, 2^22 tokens)
    assert f(A, 0, 1, (1 << 20) + 4, A, A, 8, A, None, None, 0, None) == BL_ERR_SHAPE
    assert f(A, 0, 1, 256, A, A, (1 << 20) + 1, A, None, None, 0, None) == BL_ERR_SHAPE
    assert f(A, 0, (1 << 22) + 1, 256, A, A, 8, A, None, None, 0, None) == BL_ERR_SHAPE
    assert lib.bitlinear_workspace_size(OP_FORWARD, 1 << 22, 4, 3) > 0
    assert lib.bitlinear_workspace_size(OP_FORWARD, (1 << 22) + 1, 4, 3) == 0
    assert f(MIS, 0, 1, 256, A, A, 8, A, None, None, 0, None) == BL_ERR_ALIGN
    assert f(A, 0, 1, 256, MIS, A, 8, A, None, None, 0, None) == BL_ERR_ALIGN
    assert f(A, 0, 1, 256, A, A, 8, A, MIS, None, 0, None) == BL_ERR_ALIGN
    need = lib.bitlinear_workspace_size(OP_FORWARD, 64, 256, 8)
    assert f(A, 1, 64, 256, A, A, 8, A, None, None, 0, None) == BL_ERR_NULL
    assert f(A, 1, 64, 256, A, A, 8, A, None, A, need - 1, None) == BL_ERR_WORKSPACE
    assert f(A, 1, 64, 256, A, A, 8, A, None, A + 16, need, None) == BL_ERR_ALIGN


def test_other_entry_points_argument_errors(lib):
    assert lib.bitlinear_pack_weights(None, 8, 256, A, A, A, 1 << 20, None) == BL_ERR_NULL
    assert lib.bitlinear_pack_weights(A, 8, 255, A, A, A, 1 << 20, None) == BL_ERR_SHAPE
    assert lib.bitlinear_pack_weights(A, 8, 256, A, A, A, 8, None) == BL_ERR_WORKSPACE
    assert lib.bitlinear_quant_act(A, 2, 1, 256, A, A, None) == BL_ERR_DTYPE
    assert lib.bitlinear_quant_act(A, 0, 1, 2, A, A, None) == BL_ERR_SHAPE
    assert lib.bitlinear_quant_act(A, 1, 1, 256, MIS, A, None) == BL_ERR_ALIGN
    assert lib.bitlinear_gemm_i32(A, 4, 256, A, 8, None, A, 1 << 20, None) == BL_ERR_NULL
    assert lib.bitlinear_gemm_i32(A, 4, 256, A, 8, A, A, 0, None) == BL_ERR_WORKSPACE
    t = lib.bitlinear_pack_weights_threshold
    t.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    need = lib.bitlinear_workspace_size(OP_PACK_THRESHOLD, 0, 256, 8)
    assert need >= 8 * 8
    assert t(None, 8, 256, 0.7, A, A, None, A, need, None) == BL_ERR_NULL
    assert t(A, 8, 256, 0.7, A, None, None, A, need, None) == BL_ERR_NULL
    assert t(A, 8, 250, 0.7, A, A, None, A, need, None) == BL_ERR_SHAPE
    for bad in (-0.1, float("nan"), float("inf")):
        assert t(A, 8, 256, bad, A, A, None, A, need, None) == BL_ERR_VALUE
    assert t(A, 8, 256, 0.7, A, A, MIS + 1, A, need, None) == BL_ERR_ALIGN
    assert t(A, 8, 256, 0.7, A, A, None, A, need - 1, None) == BL_ERR_WORKSPACE
    assert t(A, 8, 256, 0.7, A, A, None, None, need, None) == BL_ERR_NULL
    ffn = lib.bitlinear_ffn
    assert ffn(A, 1, 1, 256, 512, A, A, A, A, None, A, A, None, None, A, 1 << 20, None) == BL_ERR_NULL
    assert ffn(A, 1, 1, 256, 510, A, A, A, A, A, A, A, None, None, A, 1 << 20, None) == BL_ERR_SHAPE
    assert ffn(A, 1, 1, 256, 512, A, A, A, A, A, A, A, MIS, None, A, 1 << 20, None) == BL_ERR_ALIGN
    assert ffn(A, 1, 1, 256, 512, A, A, A, A, A, A, A, None, None, A, 16, None) == BL_ERR_WORKSPACE


def test_norm_entry_points_argument_errors(lib):
    qn = lib.bitlinear_quant_act_norm
    assert qn(None, 1, 1, 256, None, A, A, None) == BL_ERR_NULL
    assert qn(A, 3, 1, 256, None, A, A, None) == BL_ERR_DTYPE
    assert qn(A, 1, 1, 254, None, A, A, None) == BL_ERR_SHAPE
    assert qn(A, 1, 1, 256, MIS, A, A, None) == BL_ERR_ALIGN      # gain must be 16-byte aligned
    fn = lib.bitlinear_forward_norm
    need = lib.bitlinear_workspace_size(OP_FORWARD_NORM, 1, 256, 8)
    assert need >= 256 * 256                                       # the quantized rows always go through it
    assert fn(A, 1, 1, 256, None, A, A, 8, None, None, A, need, None) == BL_ERR_NULL
    assert fn(A, 1, 1, 256, MIS, A, A, 8, A, None, A, need, None) == BL_ERR_ALIGN
    assert fn(A, 1, 1, 256, None, A, A, 8, A, None, A, need - 1, None) == BL_ERR_WORKSPACE
    assert fn(A, 1, 1, 256, None, A, A, 8, A, None, None, 0, None) == BL_ERR_NULL


def test_sparse_ffn_argument_errors(lib):
    pk = lib.bitlinear_pack_kmajor
    assert pk(None, 8, 256, A, None) == BL_ERR_NULL
    assert pk(A, 6, 256, A, None) == BL_ERR_SHAPE                 # n % 4 != 0
    assert pk(A, 8, 256, MIS, None) == BL_ERR_ALIGN
    f = lib.bitlinear_ffn_sparse
    ws = lib.bitlinear_workspace_size
    need = ws(OP_FFN_SPARSE, 1, 4096, 14336)
    assert need >= 14336 * 4 + 4096 * 4                             # h and the down sums
    assert ws(OP_FFN_SPARSE, 5, 4096, 14336) == 0                   # decode only
    assert ws(OP_FFN_SPARSE, 1, 4104, 14336) == 0                   # hidden % 16 != 0
    assert f(A, 1, 1, 4096, 14336, A, A, A, A, None, A, A, None, None, A, need, None) == BL_ERR_NULL
    assert f(A, 1, 5, 4096, 14336, A, A, A, A, A, A, A, None, None, A, need, None) == BL_ERR_SHAPE
    assert f(A, 1, 1, 4104, 14336, A, A, A, A, A, A, A, None, None, A, need, None) == BL_ERR_SHAPE
    assert f(A, 1, 1, 4096, 14336, A, A, A, A, MIS, A, A, None, None, A, need, None) == BL_ERR_ALIGN
    assert f(A, 1, 1, 4096, 14336, A, A, A, A, A, A, A, None, None, A, need - 1, None) == BL_ERR_WORKSPACE


def test_a4_argument_errors(lib):
    qa = lib.bitlinear_quant_act_a4
    assert qa(None, 1, 1, 256, 128, A, A, None) == BL_ERR_NULL
    assert qa(A, 1, 1, 256, 0, A, A, None) == BL_ERR_VALUE
    assert qa(A, 1, 1, 256, 257, A, A, None) == BL_ERR_VALUE
    assert qa(A, 1, 1, 255, 128, A, A, None) == BL_ERR_SHAPE
    fa = lib.bitlinear_forward_a4
    need = lib.bitlinear_workspace_size(OP_FORWARD_A4, 1, 256, 8)
    assert need >= 256 * 256
    assert fa(A, 1, 1, 256, 0, A, A, 8, A, None, A, need, None) == BL_ERR_VALUE
    assert fa(A, 1, 1, 256, 128, A, A, 8, A, None, A, need - 1, None) == BL_ERR_WORKSPACE


def test_noalloc_argument_errors(lib):
    """The variant without a workspace rejects bad arguments, and sizes whose
    scratch would exceed its 32 MiB array, before touching the device."""
    f = lib.bitlinear_forward_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 1, 64, 256, A, A, 8, A, None, None) == BL_ERR_NULL
    assert f(A, 9, 64, 256, A, A, 8, A, None, None) == BL_ERR_DTYPE
    assert f(A, 1, 64, 258, A, A, 8, A, None, None) == BL_ERR_SHAPE
    assert f(A, 1, 64, 256, MIS, A, 8, A, None, None) == BL_ERR_ALIGN
    assert lib.bitlinear_workspace_size(OP_FORWARD, 4096, 8192, 64) > 32 << 20
    assert f(A, 1, 4096, 8192, A, A, 64, A, None, None) == BL_ERR_WORKSPACE


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """No CPU fallback: with the shared library absent, every call raises."""
    import bit_ternary_weight_bitlinear_amd as bl
    monkeypatch.setattr(bl, "_lib", None)
    monkeypatch.setattr(bl, "_LIB_PATH", str(tmp_path / "libbitlinear.so"))
    with pytest.raises(bl.BitLinearError):
        bl.load_library()
    with pytest.raises(bl.BitLinearError):
        bl.workspace_size(bl.OP_FORWARD, 1, 256, 256)
