"""Seeded synthetic inputs for the BitLinear workloads.

This module is the only code shared by the oracle side and the GPU side of the
tests and the benchmark. It draws random numbers and shapes tensors; it holds
none of the quantization or contraction arithmetic.

Generator (bit-reproducible for a given numpy/libm):
  * splitmix64 counter stream, state_i = seed + (i + 1) * 0x9E3779B97F4A7C15,
    mixed with the published splitmix64 finaliser (Steele, Lea, Flood 2014).
  * uniform doubles from the top 53 bits; u1 is shifted into (0, 1].
  * standard normals by Box-Muller (cosine branch, one normal per pair).
  * Student-t with nu = 3 as Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3).
  * fp32 = (float)double; bf16 = round-to-nearest-even of the fp32 bits.
  * outlier channels: a seeded partial Fisher-Yates shuffle over the input
    features picks the channels; the whole column is scaled before rounding.

Seeds: seed = 0xB17 ^ (config_id << 8) ^ tensor_id with tensor ids
W=1, x=2, gate=3, up=4, down=5, qkv=6, o=7 (extra ids are free to use).
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_IDS = {"W": 1, "x": 2, "gate": 3, "up": 4, "down": 5, "qkv": 6, "o": 7}


def seed_for(config_id: int, tensor: str | int) -> int:
    tid = TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    return (0xB17 ^ (int(config_id) << 8) ^ tid) & 0xFFFFFFFFFFFFFFFF


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the splitmix64 stream for `seed`."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed) + idx * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def _uniform_pair(seed: int, start: int, count: int):
    bits = splitmix64(seed, 2 * start, 2 * count)
    top = (bits >> np.uint64(11)).astype(np.float64)
    u1 = (top[0::2] + 1.0) * (2.0 ** -53)   # (0, 1]
    u2 = top[1::2] * (2.0 ** -53)           # [0, 1)
    return u1, u2


def normal(seed: int, count: int, start: int = 0, chunk: int = 1 << 22) -> np.ndarray:
    """`count` standard normals (float64), Box-Muller over the splitmix64 stream."""
    out = np.empty(count, dtype=np.float64)
    for off in range(0, count, chunk):
        n = min(chunk, count - off)
        u1, u2 = _uniform_pair(seed, start + off, n)
        out[off:off + n] = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return out


def student_t3(seed: int, count: int) -> np.ndarray:
    """`count` Student-t(nu=3) draws: one normal over an independent chi^2_3 / 3."""
    z = normal(seed, 4 * count)
    num = z[0::4]
    den = np.sqrt((z[1::4] ** 2 + z[2::4] ** 2 + z[3::4] ** 2) / 3.0)
    return num / den


def pick_channels(seed: int, k: int, count: int) -> np.ndarray:
    """Seeded partial Fisher-Yates: the first `count` of a shuffle of range(k)."""
    perm = np.arange(k, dtype=np.int64)
    bits = splitmix64(seed ^ 0x5EED, 0, max(count, 1))
    for i in range(count):
        j = i + int(bits[i] % np.uint64(k - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of fp32 values to bf16, returned as uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- tensors

def weights(config_id: int, tensor: str | int, n: int, k: int, sigma: float = 0.02) -> np.ndarray:
    """fp32 weights [n][k] (out x in), N(0, sigma^2)."""
    w = normal(seed_for(config_id, tensor), n * k) * sigma
    return w.astype(np.float32).reshape(n, k)


def activations(config_id: int, m: int, k: int, *, dtype: str = "bf16",
                outlier_channels: int = 0, outlier_scale: float = 1.0,
                heavy_channels: int = 0, tensor: str | int = "x") -> np.ndarray:
    """Activations [m][k]: N(0,1), optional scaled outlier channels and
    Student-t(3) heavy-tailed channels. Returns float32 (dtype='f32') or the
    bf16 bit patterns as uint16 (dtype='bf16')."""
    seed = seed_for(config_id, tensor)
    x = normal(seed, m * k).reshape(m, k)
    if outlier_channels:
        ch = pick_channels(seed, k, outlier_channels)
        x[:, ch] *= outlier_scale
    if heavy_channels:
        ch = pick_channels(seed ^ 0xA5A5, k, heavy_channels)
        x[:, ch] = student_t3(seed ^ 0x7777, m * len(ch)).reshape(len(ch), m).T
    x32 = x.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


# ---------------------------------------------------------------- workloads
# Shapes of the five workloads (2B-class and 8B-class BitLinear layers).

WORKLOADS = {
    1: dict(name="bitlinear_m4_k256_n256", m=4, k=256, n=256, act="f32",
            outliers=2, outlier_scale=20.0),
    2: dict(name="decode_gemv_m1_2b_ffn_up_down", m=1,
            mats=[(2560, 6912), (6912, 2560)], act="bf16", outlier_frac=0.01, outlier_scale=30.0),
    3: dict(name="batched_decode_2b_layer", ms=[1, 8, 32, 64],
            mats=[(2560, 3840), (2560, 2560), (2560, 6912), (2560, 6912), (6912, 2560)], act="bf16"),
    4: dict(name="prefill_gemm_m2048_2b_ffn_up_down", m=2048,
            mats=[(2560, 6912), (6912, 2560)], act="bf16", heavy_frac=0.01),
    5: dict(name="ffn_8b_h4096_f14336", ms=[1, 2048], hidden=4096, ffn=14336, act="bf16"),
}
