"""MI355X (gfx950) BitNet b1.58 BitLinear: thin Python binding of libbitlinear.so.

Every function here only marshals torch tensors (device memory) and the current
HIP stream into the C ABI declared in include/bitlinear.h; all arithmetic runs in
the library's HIP kernels. If the library is not built, importing works but every
call raises -- there is no fallback.

Functions mirror the C entry points:
  pack_weights(w)                      -> (packed uint8 [n][k/4], gamma fp32 [1])
  pack_weights_threshold(w, factor)    -> (packed uint8 [n][k/4], alpha fp32 [1], delta fp32 [1])
  quant_act(x)                         -> (q int8 [m][k], scale fp32 [m])
  quant_act_norm(x, gain=None)         -> the same for the RMS-normalized x
  forward_norm(x, packed, gamma, gain=None) -> y fp32 [m][n] of the RMS-normalized x
  quant_act_a4(x, keep=None)           -> (q int8 [m][k] doubled E2M1 codes, scale fp32 [m])
  forward_a4(x, packed, gamma, keep=None) -> y fp32 [m][n] of the W1.58A4 product
  forward(x, packed, gamma)            -> y fp32 [m][n]        (return_acc=True adds acc)
  ffn(x, gate, up, down)               -> y fp32 [m][hidden]   (return_hq=True adds qh, sh)
  pack_kmajor(packed)                  -> input-major copy [k][n/4] of packed [n][k/4]
  ffn_sparse(x, gate, up, down_t)      -> ffn() for m <= 4 with an input-major down matrix
  gemm_i32(q, packed)                  -> acc int32 [m][n]
  workspace_size(op, m, k, n)          -> bytes
Activations may be float32 or bfloat16 CUDA (HIP) tensors, contiguous, [m][k].
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["pack_weights", "pack_weights_threshold", "quant_act", "quant_act_norm", "forward_norm", "forward", "ffn", "gemm_i32", "workspace_size",
           "library_path", "load_library", "BitLinearError", "OP_FORWARD", "OP_FFN", "OP_PACK",
           "OP_GEMM_I32", "OP_PACK_THRESHOLD", "OP_FORWARD_NORM", "OP_FFN_SPARSE", "OP_FORWARD_A4",
           "pack_kmajor", "ffn_sparse", "quant_act_a4", "forward_a4"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

(OP_FORWARD, OP_FFN, OP_PACK, OP_GEMM_I32, OP_PACK_THRESHOLD, OP_FORWARD_NORM, OP_FFN_SPARSE,
 OP_FORWARD_A4) = range(8)  # bl_op in include/bitlinear.h
_F32, _BF16 = 0, 1

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size = ctypes.c_size_t

_SIGNATURES = {
    "bitlinear_workspace_size": (_c_size, [_c_int, _c_i64, _c_i64, _c_i64]),
    "bitlinear_status_string": (ctypes.c_char_p, [_c_int]),
    "bitlinear_pack_weights": (_c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_size, _c_p]),
    "bitlinear_pack_weights_threshold": (_c_int, [_c_p, _c_i64, _c_i64, ctypes.c_float, _c_p, _c_p, _c_p,
                                                  _c_p, _c_size, _c_p]),
    "bitlinear_quant_act": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "bitlinear_quant_act_norm": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "bitlinear_forward_norm": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p,
                                        _c_p, _c_size, _c_p]),
    "bitlinear_forward": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_p,
                                   _c_p, _c_size, _c_p]),
    "bitlinear_ffn": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p,
                               _c_p, _c_p, _c_p, _c_p, _c_p, _c_size, _c_p]),
    "bitlinear_quant_act_a4": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "bitlinear_forward_a4": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_p,
                                      _c_p, _c_size, _c_p]),
    "bitlinear_pack_kmajor": (_c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p]),
    "bitlinear_ffn_sparse": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p,
                                      _c_p, _c_p, _c_p, _c_p, _c_p, _c_size, _c_p]),
    "bitlinear_gemm_i32": (_c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
}

_lib = None


class BitLinearError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libbitlinear.so (built by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise BitLinearError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                             "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().bitlinear_status_string(status).decode()
        raise BitLinearError(f"{what}: {msg}")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise BitLinearError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise BitLinearError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise BitLinearError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _act_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return _F32
    if x.dtype == torch.bfloat16:
        return _BF16
    raise BitLinearError(f"activations must be float32 or bfloat16, got {x.dtype}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(op: int, m: int, k: int, n: int, device) -> torch.Tensor | None:
    nbytes = workspace_size(op, m, k, n)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ws_args(ws):
    return (ws.data_ptr(), ws.numel() * ws.element_size()) if ws is not None else (None, 0)


def _caller_workspace(ws: torch.Tensor, op: int, m: int, k: int, n: int) -> torch.Tensor | None:
    """A caller-supplied workspace must be a contiguous device tensor of at least
    workspace_size() bytes (the C ABI trusts the size it is given)."""
    need = workspace_size(op, m, k, n)
    if need == 0:
        return None
    _dev(ws, "workspace")
    if ws.numel() * ws.element_size() < need:
        raise BitLinearError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {need} needed")
    return ws


def _check_out(out: torch.Tensor, shape, dtype, name: str):
    _dev(out, name, dtype)
    if tuple(out.shape) != tuple(shape):
        raise BitLinearError(f"{name} must have shape {tuple(shape)}, got {tuple(out.shape)}")


def workspace_size(op: int, m: int, k: int, n: int) -> int:
    return int(load_library().bitlinear_workspace_size(op, m, k, n))


def pack_weights(w: torch.Tensor):
    """fp32 weights [n][k] -> (packed uint8 [n][k/4], gamma fp32 [1])."""
    lib = load_library()
    n, k = w.shape
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device=w.device)
    gamma = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = _workspace(OP_PACK, 0, k, n, w.device)
    wp, wn = _ws_args(ws)
    _check(lib.bitlinear_pack_weights(_dev(w, "w", torch.float32), n, k, packed.data_ptr(),
                                      gamma.data_ptr(), wp, wn, _stream(w.device)),
           "bitlinear_pack_weights")
    return packed, gamma


def pack_weights_threshold(w: torch.Tensor, factor: float = 0.7):
    """fp32 weights [n][k] -> (packed uint8 [n][k/4], alpha fp32 [1], delta fp32 [1]) of the
    threshold quantizer; (packed, alpha) is used like (packed, gamma)."""
    lib = load_library()
    n, k = w.shape
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device=w.device)
    alpha = torch.empty(1, dtype=torch.float32, device=w.device)
    delta = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = _workspace(OP_PACK_THRESHOLD, 0, k, n, w.device)
    wp, wn = _ws_args(ws)
    _check(lib.bitlinear_pack_weights_threshold(_dev(w, "w", torch.float32), n, k, float(factor),
                                                packed.data_ptr(), alpha.data_ptr(), delta.data_ptr(), wp, wn,
                                                _stream(w.device)), "bitlinear_pack_weights_threshold")
    return packed, alpha, delta


def quant_act(x: torch.Tensor):
    """activations [m][k] -> (q int8 [m][k], scale fp32 [m])."""
    lib = load_library()
    m, k = x.shape
    q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    s = torch.empty(m, dtype=torch.float32, device=x.device)
    _check(lib.bitlinear_quant_act(_dev(x, "x"), _act_dtype(x), m, k, q.data_ptr(), s.data_ptr(),
                                   _stream(x.device)), "bitlinear_quant_act")
    return q, s


def _gain(gain, k: int):
    if gain is None:
        return None
    if gain.numel() != k:
        raise BitLinearError(f"gain must have {k} entries, got {gain.numel()}")
    return _dev(gain, "gain", torch.float32)


def quant_act_norm(x: torch.Tensor, gain: torch.Tensor | None = None):
    """RMS-normalized activations [m][k] -> (q int8 [m][k], scale fp32 [m])."""
    lib = load_library()
    m, k = x.shape
    q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    s = torch.empty(m, dtype=torch.float32, device=x.device)
    _check(lib.bitlinear_quant_act_norm(_dev(x, "x"), _act_dtype(x), m, k, _gain(gain, k), q.data_ptr(),
                                        s.data_ptr(), _stream(x.device)), "bitlinear_quant_act_norm")
    return q, s


def forward_norm(x: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor, gain: torch.Tensor | None = None,
                 *, return_acc: bool = False, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None):
    """BitLinear forward of the RMS-normalized x (the normalization fused into the quantization)."""
    lib = load_library()
    m, k = x.shape
    n = packed.shape[0]
    if packed.shape[1] * 4 != k:
        raise BitLinearError("packed weights do not match the activation width")
    if out is not None:
        _check_out(out, (m, n), torch.float32, "out")
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if return_acc else None
    ws = (_caller_workspace(workspace, OP_FORWARD_NORM, m, k, n) if workspace is not None
          else _workspace(OP_FORWARD_NORM, m, k, n, x.device))
    wp, wn = _ws_args(ws)
    _check(lib.bitlinear_forward_norm(_dev(x, "x"), _act_dtype(x), m, k, _gain(gain, k),
                                      _dev(packed, "packed", torch.uint8), _dev(gamma, "gamma", torch.float32), n,
                                      _dev(y, "y", torch.float32), acc.data_ptr() if acc is not None else None,
                                      wp, wn, _stream(x.device)), "bitlinear_forward_norm")
    return (y, acc) if return_acc else y


def quant_act_a4(x: torch.Tensor, keep: int | None = None):
    """4-bit activations [m][k] -> (q int8 [m][k] holding 2e, scale fp32 [m]); keep defaults to ceil(k / 2)."""
    lib = load_library()
    m, k = x.shape
    keep = (k + 1) // 2 if keep is None else int(keep)
    q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    s = torch.empty(m, dtype=torch.float32, device=x.device)
    _check(lib.bitlinear_quant_act_a4(_dev(x, "x"), _act_dtype(x), m, k, keep, q.data_ptr(), s.data_ptr(),
                                      _stream(x.device)), "bitlinear_quant_act_a4")
    return q, s


def forward_a4(x: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor, keep: int | None = None,
               *, return_acc: bool = False, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None):
    """W1.58A4 forward: 4-bit top-K activations times the ternary weights."""
    lib = load_library()
    m, k = x.shape
    n = packed.shape[0]
    keep = (k + 1) // 2 if keep is None else int(keep)
    if packed.shape[1] * 4 != k:
        raise BitLinearError("packed weights do not match the activation width")
    if out is not None:
        _check_out(out, (m, n), torch.float32, "out")
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if return_acc else None
    ws = (_caller_workspace(workspace, OP_FORWARD_A4, m, k, n) if workspace is not None
          else _workspace(OP_FORWARD_A4, m, k, n, x.device))
    wp, wn = _ws_args(ws)
    _check(lib.bitlinear_forward_a4(_dev(x, "x"), _act_dtype(x), m, k, keep, _dev(packed, "packed", torch.uint8),
                                    _dev(gamma, "gamma", torch.float32), n, _dev(y, "y", torch.float32),
                                    acc.data_ptr() if acc is not None else None, wp, wn, _stream(x.device)),
           "bitlinear_forward_a4")
    return (y, acc) if return_acc else y


def forward(x: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor, *, return_acc: bool = False,
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """BitLinear forward. x [m][k] (fp32/bf16), packed uint8 [n][k/4], gamma fp32 [1]."""
    lib = load_library()
    m, k = x.shape
    n = packed.shape[0]
    if packed.shape[1] * 4 != k:
        raise BitLinearError("packed weights do not match the activation width")
    if out is not None:
        _check_out(out, (m, n), torch.float32, "out")
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if return_acc else None
    ws = (_caller_workspace(workspace, OP_FORWARD, m, k, n) if workspace is not None
          else _workspace(OP_FORWARD, m, k, n, x.device))
    wp, wn = _ws_args(ws)
    _check(lib.bitlinear_forward(_dev(x, "x"), _act_dtype(x), m, k, _dev(packed, "packed", torch.uint8),
                                 _dev(gamma, "gamma", torch.float32), n, _dev(y, "y", torch.float32),
                                 acc.data_ptr() if acc is not None else None, wp, wn,
                                 _stream(x.device)), "bitlinear_forward")
    return (y, acc) if return_acc else y


def ffn(x: torch.Tensor, gate, up, down, *, return_hq: bool = False,
        workspace: torch.Tensor | None = None):
    """Squared-ReLU gated FFN. gate/up/down are (packed, gamma) pairs:
    gate/up packed [ffn][hidden/4], down packed [hidden][ffn/4]."""
    lib = load_library()
    m, hidden = x.shape
    ffn_dim = gate[0].shape[0]
    if gate[0].shape[1] * 4 != hidden or up[0].shape != gate[0].shape or \
            down[0].shape != (hidden, ffn_dim // 4):
        raise BitLinearError("FFN weight shapes do not match")
    y = torch.empty((m, hidden), dtype=torch.float32, device=x.device)
    hq = torch.empty((m, ffn_dim), dtype=torch.int8, device=x.device) if return_hq else None
    hs = torch.empty(m, dtype=torch.float32, device=x.device) if return_hq else None
    ws = (_caller_workspace(workspace, OP_FFN, m, hidden, ffn_dim) if workspace is not None
          else _workspace(OP_FFN, m, hidden, ffn_dim, x.device))
    wp, wn = _ws_args(ws)
    _check(lib.bitlinear_ffn(_dev(x, "x"), _act_dtype(x), m, hidden, ffn_dim,
                             _dev(gate[0], "gate_packed", torch.uint8),
                             _dev(gate[1], "gate_gamma", torch.float32),
                             _dev(up[0], "up_packed", torch.uint8), _dev(up[1], "up_gamma", torch.float32),
                             _dev(down[0], "down_packed", torch.uint8),
                             _dev(down[1], "down_gamma", torch.float32),
                             y.data_ptr(), hq.data_ptr() if hq is not None else None,
                             hs.data_ptr() if hs is not None else None, wp, wn, _stream(x.device)),
           "bitlinear_ffn")
    return (y, hq, hs) if return_hq else y


def pack_kmajor(packed: torch.Tensor):
    """packed [n][k/4] -> the input-major packing [k][n/4] of the same codes (n % 4 == 0)."""
    lib = load_library()
    n, kb = packed.shape
    out = torch.empty((4 * kb, n // 4), dtype=torch.uint8, device=packed.device)
    _check(lib.bitlinear_pack_kmajor(_dev(packed, "packed", torch.uint8), n, 4 * kb, out.data_ptr(),
                                     _stream(packed.device)), "bitlinear_pack_kmajor")
    return out


def ffn_sparse(x: torch.Tensor, gate, up, down_t, *, return_hq: bool = False,
               workspace: torch.Tensor | None = None):
    """Decode FFN (m <= 4) skipping the zero channels of h in the down projection.
    gate/up are (packed [ffn][hidden/4], gamma); down_t is (pack_kmajor(down packed), gamma)."""
    lib = load_library()
    m, hidden = x.shape
    ffn_dim = gate[0].shape[0]
    if gate[0].shape[1] * 4 != hidden or up[0].shape != gate[0].shape or \
            down_t[0].shape != (ffn_dim, hidden // 4):
        raise BitLinearError("FFN weight shapes do not match")
    y = torch.empty((m, hidden), dtype=torch.float32, device=x.device)
    hq = torch.empty((m, ffn_dim), dtype=torch.int8, device=x.device) if return_hq else None
    hs = torch.empty(m, dtype=torch.float32, device=x.device) if return_hq else None
    ws = (_caller_workspace(workspace, OP_FFN_SPARSE, m, hidden, ffn_dim) if workspace is not None
          else _workspace(OP_FFN_SPARSE, m, hidden, ffn_dim, x.device))
    wp, wn = _ws_args(ws)
    _check(lib.bitlinear_ffn_sparse(_dev(x, "x"), _act_dtype(x), m, hidden, ffn_dim,
                                    _dev(gate[0], "gate_packed", torch.uint8),
                                    _dev(gate[1], "gate_gamma", torch.float32),
                                    _dev(up[0], "up_packed", torch.uint8), _dev(up[1], "up_gamma", torch.float32),
                                    _dev(down_t[0], "down_packed_t", torch.uint8),
                                    _dev(down_t[1], "down_gamma", torch.float32),
                                    y.data_ptr(), hq.data_ptr() if hq is not None else None,
                                    hs.data_ptr() if hs is not None else None, wp, wn, _stream(x.device)),
           "bitlinear_ffn_sparse")
    return (y, hq, hs) if return_hq else y


def gemm_i32(q: torch.Tensor, packed: torch.Tensor):
    """Bare int8 x ternary product: q int8 [m][k], packed [n][k/4] -> acc int32 [m][n]."""
    lib = load_library()
    m, k = q.shape
    n = packed.shape[0]
    acc = torch.empty((m, n), dtype=torch.int32, device=q.device)
    ws = _workspace(OP_GEMM_I32, m, k, n, q.device)
    wp, wn = _ws_args(ws)
    _check(lib.bitlinear_gemm_i32(_dev(q, "q", torch.int8), m, k, _dev(packed, "packed", torch.uint8), n,
                                  acc.data_ptr(), wp, wn, _stream(q.device)), "bitlinear_gemm_i32")
    return acc
