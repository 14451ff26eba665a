"""Helpers for the GPU parity tests: move seeded numpy inputs to the device and
compare device results with the CPU oracle."""
from __future__ import annotations

import numpy as np

import oracle
import synth


def to_dev(a: np.ndarray, dtype: str | None = None):
    import torch
    dev = torch.device("cuda:0")
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def make_linear(cfg: int, tid, n: int, k: int):
    """(fp32 weights, oracle packed, oracle gamma, oracle ternary) for a seeded matrix."""
    w = synth.weights(cfg, tid, n, k)
    packed, gamma, wt = oracle.pack_weights(w)
    return w, packed, gamma, wt


def assert_y_close(y_dev: np.ndarray, y_ref: np.ndarray, rtol: float = 1e-5):
    """fp32 outputs: within rtol relative to each element (zeros must match exactly)."""
    y_dev = np.asarray(y_dev, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    err = np.abs(y_dev - y_ref)
    bad = err > rtol * np.abs(y_ref)
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outputs outside rtol={rtol}; "
                           f"worst rel {np.max(err / np.maximum(np.abs(y_ref), 1e-30)):.3g}")
