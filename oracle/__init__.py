"""CPU oracle for the BitNet b1.58 BitLinear forward pass (W1.58A8).

TEST INFRASTRUCTURE ONLY. Only the tests, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` may import this package. The HIP library does not
depend on it and shares no code with it.

The arithmetic lives in `bitlinear_oracle.c` (plain C loops, one function per
step of the method); this module marshals numpy arrays and composes the steps in
the order the pages give:

  pack:     gamma = mean|W|  ->  W~ = RoundClip(W / gamma, -1, 1)  ->  2-bit codes
  forward:  per-token absmax int8 quantization of x  ->  int32 product with W~
            ->  y = acc * (s / 127) * gamma
  ffn:      one quantization of x shared by gate and up  ->  h = relu(g)^2 * u
            ->  per-token requantization of h  ->  down projection

  rms norm (subln) before the activation quantization, per token:
            S = sum_k x^2 (correctly rounded fp64)  ->  ms = fp32(S / k)
            ->  r = 1 / sqrt(ms + 1e-5) (fp32)  ->  x^ = (x * r) * g  ->  absmax int8 of x^
  4-bit activations (W1.58A4), per token: keep |x| >= the keep-th largest
            |x| (top-K, ties kept)  ->  s = max(max|x|, 1e-5)  ->  v = x * (6 / s)
            ->  nearest E2M1 value e (ties to even), stored doubled (2e in [-12, 12])
            ->  the same int32 product  ->  y = acc * (s / 12) * gamma
  threshold pack (a second weight quantizer): delta = factor * mean|W|
            ->  W~ = sign(W) where |W| > delta, else 0  ->  alpha = mean(|W| * mask)
            ->  the same 2-bit codes; alpha takes gamma's place in forward/ffn

Sources: "BitNet 1-bit LLM 的混合精度微调技术：渐进量化策略" (BitLinear paragraph,
operational-parameter paragraph); "BitNet 中使用直通估计器工程化三元权重训练"
(section 工程化训练流程与参数配置, activation item); "穿越1比特的奇幻旅程" summary of
the BitNet b1.58 2B4T report (sections 架构创新 and 推理实现 / GPU端); "BitNet
三元权重阈值优化工程实践" (section on the core principle of threshold optimization).

Parity pins for every function live in tests/test_oracle_pins.py; none of them
is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_absmean.restype = ctypes.c_float
    lib.oracle_absmean.argtypes = [_p, _i64, _i64]
    lib.oracle_ternarize.argtypes = [_p, _i64, _i64, ctypes.c_float, _p]
    lib.oracle_threshold_ternarize.restype = ctypes.c_float
    lib.oracle_threshold_ternarize.argtypes = [_p, _i64, _i64, ctypes.c_float, _p, _p]
    lib.oracle_pack.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_pack_kmajor.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_unpack.restype = _i64
    lib.oracle_unpack.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_quant_act.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_bf16_to_f32.argtypes = [_p, _i64, _p]
    lib.oracle_matmul_i32.argtypes = [_p, _i64, _i64, _p, _i64, _p]
    lib.oracle_rescale.argtypes = [_p, _i64, _i64, _p, ctypes.c_float, _p]
    lib.oracle_rescale_q.argtypes = [_p, _i64, _i64, _p, ctypes.c_float, ctypes.c_float, _p]
    lib.oracle_e2m1_doubled.restype = ctypes.c_int
    lib.oracle_e2m1_doubled.argtypes = [ctypes.c_float]
    lib.oracle_quant_act_a4.argtypes = [_p, _i64, _i64, _i64, _p, _p]
    lib.oracle_sqrelu_gate.argtypes = [_p, _p, _i64, _p]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(t: int) -> None:
    _load().oracle_set_num_threads(int(t))


# ------------------------------------------------------------------ steps

def bf16_to_f32(xb: np.ndarray) -> np.ndarray:
    xb = _c(xb, np.uint16)
    out = np.empty(xb.shape, dtype=np.float32)
    _load().oracle_bf16_to_f32(_ptr(xb), xb.size, _ptr(out))
    return out


def absmean(w: np.ndarray) -> np.float32:
    w = _c(w, np.float32)
    n, k = w.shape
    return np.float32(_load().oracle_absmean(_ptr(w), n, k))


def ternarize(w: np.ndarray, gamma) -> np.ndarray:
    w = _c(w, np.float32)
    n, k = w.shape
    out = np.empty((n, k), dtype=np.int8)
    _load().oracle_ternarize(_ptr(w), n, k, float(np.float32(gamma)), _ptr(out))
    return out


def pack(wt: np.ndarray) -> np.ndarray:
    wt = _c(wt, np.int8)
    n, k = wt.shape
    if k % 4:
        raise ValueError("k must be a multiple of 4")
    out = np.empty((n, k // 4), dtype=np.uint8)
    _load().oracle_pack(_ptr(wt), n, k, _ptr(out))
    return out


def unpack(packed: np.ndarray, k: int) -> np.ndarray:
    """Ternary weights from packed bytes; raises on the invalid code 3."""
    packed = _c(packed, np.uint8)
    n = packed.shape[0]
    if packed.shape[1] * 4 != k:
        raise ValueError("packed width does not match k")
    out = np.empty((n, k), dtype=np.int8)
    bad = _load().oracle_unpack(_ptr(packed), n, k, _ptr(out))
    if bad:
        raise ValueError(f"{bad} invalid 2-bit codes (3) in packed weights")
    return out


def pack_kmajor(packed: np.ndarray, k: int) -> np.ndarray:
    """Packed [n][k/4] -> the input-major packing [k][n/4] of the same codes (n % 4 == 0)."""
    packed = _c(packed, np.uint8)
    n = packed.shape[0]
    if packed.shape[1] * 4 != k or n % 4:
        raise ValueError("need packed [n][k/4] with n % 4 == 0")
    out = np.empty((k, n // 4), dtype=np.uint8)
    _load().oracle_pack_kmajor(_ptr(packed), n, k, _ptr(out))
    return out


def pack_weights(w: np.ndarray):
    """Offline weight step: (packed uint8 [n][k/4], gamma fp32, ternary int8 [n][k])."""
    g = absmean(w)
    wt = ternarize(w, g)
    return pack(wt), g, wt


def threshold_ternarize(w: np.ndarray, factor: float = 0.7):
    """(ternary int8 [n][k], alpha fp32, delta fp32) of the threshold quantizer."""
    w = _c(w, np.float32)
    n, k = w.shape
    wt = np.empty((n, k), dtype=np.int8)
    delta = np.zeros(1, dtype=np.float32)
    alpha = _load().oracle_threshold_ternarize(_ptr(w), n, k, float(np.float32(factor)), _ptr(wt), _ptr(delta))
    return wt, np.float32(alpha), delta[0]


def pack_weights_threshold(w: np.ndarray, factor: float = 0.7):
    """Threshold weight step: (packed uint8 [n][k/4], alpha fp32, ternary int8, delta fp32)."""
    wt, alpha, delta = threshold_ternarize(w, factor)
    return pack(wt), alpha, wt, delta


def _as_f32_acts(x, dtype: str):
    if dtype == "bf16":
        return bf16_to_f32(x)
    if dtype == "f32":
        return _c(x, np.float32)
    raise ValueError(dtype)


def quant_act(x: np.ndarray, dtype: str = "f32"):
    """(q int8 [m][k], s fp32 [m]) for activations x (fp32, or bf16 bit patterns)."""
    xf = _as_f32_acts(x, dtype)
    m, k = xf.shape
    q = np.empty((m, k), dtype=np.int8)
    s = np.empty(m, dtype=np.float32)
    _load().oracle_quant_act(_ptr(xf), m, k, _ptr(q), _ptr(s))
    return q, s


NORM_EPS = np.float32(1e-5)


def rms_norm(x: np.ndarray, dtype: str = "f32", gain: np.ndarray | None = None) -> np.ndarray:
    """Per-token RMS normalization ("subln" of "穿越1比特的奇幻旅程", section 架构创新:
    a normalization added for the stability of 1-bit training; "BitNet 中使用直通估计器
    工程化三元权重训练", section 工程化训练流程与参数配置: layer normalization keeps the
    variance, epsilon 1e-5). Reading: RMSNorm without mean subtraction or bias,
    an optional per-channel gain g, epsilon 1e-5 inside the square root:
      S  = sum_k x_k^2      every square exact in fp64, the sum correctly rounded
                            to fp64 (math.fsum)
      ms = fp32(S / k)      one fp64 division, one rounding to fp32
      r  = 1 / sqrt(ms + 1e-5)          each fp32 operation correctly rounded
      x^ = (x * r) * g      fp32, in that order (x * r without a gain)
    Returns x^ as fp32 [m][k]."""
    xf = _as_f32_acts(x, dtype)
    m, k = xf.shape
    g = None if gain is None else _c(gain, np.float32).reshape(k)
    out = np.empty((m, k), dtype=np.float32)
    for t in range(m):
        sq = xf[t].astype(np.float64) ** 2
        s_sum = math.fsum(sq.tolist())
        ms = np.float32(s_sum / k)
        d = np.float32(ms + NORM_EPS)
        r = np.float32(np.float32(1.0) / np.sqrt(d))
        row = xf[t] * r
        if g is not None:
            row = row * g
        out[t] = row
    return out


def quant_act_norm(x: np.ndarray, dtype: str = "f32", gain: np.ndarray | None = None):
    """(q int8 [m][k], s fp32 [m]) of the absmax quantization of rms_norm(x)."""
    return quant_act(rms_norm(x, dtype, gain), "f32")


def matmul_i32(q: np.ndarray, wt: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    wt = _c(wt, np.int8)
    m, k = q.shape
    n, k2 = wt.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    acc = np.empty((m, n), dtype=np.int32)
    _load().oracle_matmul_i32(_ptr(q), m, k, _ptr(wt), n, _ptr(acc))
    return acc


def e2m1_doubled(v: float) -> int:
    """Nearest E2M1 value of a float32, doubled (an integer in [-12, 12])."""
    return int(_load().oracle_e2m1_doubled(float(np.float32(v))))


def quant_act_a4(x: np.ndarray, dtype: str = "f32", keep: int | None = None):
    """4-bit activations: (q int8 [m][k] holding 2e, s fp32 [m]); keep defaults to ceil(k / 2)."""
    xf = _as_f32_acts(x, dtype)
    m, k = xf.shape
    keep = (k + 1) // 2 if keep is None else int(keep)
    if not 1 <= keep <= k:
        raise ValueError("keep must be in [1, k]")
    q = np.empty((m, k), dtype=np.int8)
    s = np.empty(m, dtype=np.float32)
    _load().oracle_quant_act_a4(_ptr(xf), m, k, keep, _ptr(q), _ptr(s))
    return q, s


def rescale_q(acc: np.ndarray, s: np.ndarray, gamma, qmax: float) -> np.ndarray:
    acc = _c(acc, np.int32)
    s = _c(s, np.float32)
    m, n = acc.shape
    y = np.empty((m, n), dtype=np.float32)
    _load().oracle_rescale_q(_ptr(acc), m, n, _ptr(s), float(np.float32(gamma)), float(np.float32(qmax)), _ptr(y))
    return y


def rescale(acc: np.ndarray, s: np.ndarray, gamma) -> np.ndarray:
    acc = _c(acc, np.int32)
    s = _c(s, np.float32)
    m, n = acc.shape
    y = np.empty((m, n), dtype=np.float32)
    _load().oracle_rescale(_ptr(acc), m, n, _ptr(s), float(np.float32(gamma)), _ptr(y))
    return y


def sqrelu_gate(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    h = np.empty(g.shape, dtype=np.float32)
    _load().oracle_sqrelu_gate(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


# ------------------------------------------------------------ compositions

def forward(x: np.ndarray, packed: np.ndarray, gamma, k: int, dtype: str = "f32"):
    """BitLinear forward from packed weights. Returns dict(q, s, acc, y)."""
    wt = unpack(packed, k)
    q, s = quant_act(x, dtype)
    acc = matmul_i32(q, wt)
    y = rescale(acc, s, gamma)
    return dict(q=q, s=s, acc=acc, y=y)


def forward_norm(x: np.ndarray, packed: np.ndarray, gamma, k: int, dtype: str = "f32",
                 gain: np.ndarray | None = None):
    """BitLinear forward with the RMS norm before the quantization. dict(xn, q, s, acc, y)."""
    xn = rms_norm(x, dtype, gain)
    r = forward(xn, packed, gamma, k, "f32")
    r["xn"] = xn
    return r


def forward_a4(x: np.ndarray, packed: np.ndarray, gamma, k: int, dtype: str = "f32", keep: int | None = None):
    """W1.58A4 forward: 4-bit top-K activations, the int32 product, y = acc * (s / 12) * gamma."""
    wt = unpack(packed, k)
    q, s = quant_act_a4(x, dtype, keep)
    acc = matmul_i32(q, wt)
    return dict(q=q, s=s, acc=acc, y=rescale_q(acc, s, gamma, 12.0))


def ffn(x: np.ndarray, gate, up, down, hidden: int, ffn_dim: int, dtype: str = "bf16"):
    """Squared-ReLU gated FFN of BitLinear layers. gate/up/down are (packed, gamma)
    pairs with packed shapes [ffn][hidden/4], [ffn][hidden/4], [hidden][ffn/4].
    Returns dict(q, s, g, u, h, qh, sh, acc_down, y)."""
    wg = unpack(gate[0], hidden)
    wu = unpack(up[0], hidden)
    wd = unpack(down[0], ffn_dim)
    q, s = quant_act(x, dtype)
    g = rescale(matmul_i32(q, wg), s, gate[1])
    u = rescale(matmul_i32(q, wu), s, up[1])
    h = sqrelu_gate(g, u)
    qh, sh = quant_act(h, "f32")
    acc_d = matmul_i32(qh, wd)
    y = rescale(acc_d, sh, down[1])
    return dict(q=q, s=s, g=g, u=u, h=h, qh=qh, sh=sh, acc_down=acc_d, y=y)
