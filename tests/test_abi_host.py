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

BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_WORKSPACE, BL_ERR_HIP = range(7)
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
              "bitlinear_gemm_i32", "bitlinear_workspace_size", "bitlinear_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(7):
        assert lib.bitlinear_status_string(s)
    assert b"unknown" in lib.bitlinear_status_string(99)


def test_workspace_size_rules(lib):
    ws = lib.bitlinear_workspace_size
    assert ws(1, 1, 2560, 6912) == 0                       # decode path needs none
    assert ws(1, 2048, 2560, 6912) >= 2048 * 2560            # qperm activations
    assert ws(1, 1, 260, 7) >= 7 * 320 // 4                  # padded weight copy for ragged k
    assert ws(0, 0, 4096, 14336) >= 14336 * 8                # per-row sums
    assert ws(2, 1, 4096, 14336) >= 14336 * 4                # h buffer
    assert ws(1, 0, 256, 256) == 0 and ws(1, 1, 6, 8) == 0   # invalid shapes
    assert ws(9, 1, 256, 256) == 0


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
    assert lib.bitlinear_workspace_size(1, 1 << 22, 4, 3) > 0
    assert lib.bitlinear_workspace_size(1, (1 << 22) + 1, 4, 3) == 0
    assert f(MIS, 0, 1, 256, A, A, 8, A, None, None, 0, None) == BL_ERR_ALIGN
    assert f(A, 0, 1, 256, MIS, A, 8, A, None, None, 0, None) == BL_ERR_ALIGN
    assert f(A, 0, 1, 256, A, A, 8, A, MIS, None, 0, None) == BL_ERR_ALIGN
    need = lib.bitlinear_workspace_size(1, 64, 256, 8)
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
    ffn = lib.bitlinear_ffn
    assert ffn(A, 1, 1, 256, 512, A, A, A, A, None, A, A, None, None, A, 1 << 20, None) == BL_ERR_NULL
    assert ffn(A, 1, 1, 256, 510, A, A, A, A, A, A, A, None, None, A, 1 << 20, None) == BL_ERR_SHAPE
    assert ffn(A, 1, 1, 256, 512, A, A, A, A, A, A, A, MIS, None, A, 1 << 20, None) == BL_ERR_ALIGN
    assert ffn(A, 1, 1, 256, 512, A, A, A, A, A, A, A, None, None, A, 16, None) == BL_ERR_WORKSPACE


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """No CPU fallback: with the shared library absent, every call raises."""
    import bit_ternary_weight_bitlinear_amd as bl
    monkeypatch.setattr(bl, "_lib", None)
    monkeypatch.setattr(bl, "_LIB_PATH", str(tmp_path / "libbitlinear.so"))
    with pytest.raises(bl.BitLinearError):
        bl.load_library()
    with pytest.raises(bl.BitLinearError):
        bl.workspace_size(bl.OP_FORWARD, 1, 256, 256)
