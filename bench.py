#!/usr/bin/env python3
"""BitLinear W1.58A8 benchmark on one MI355X.

Headline (the JSON line's `value`): decode, 1 token through the 2B-class FFN up
(2560 -> 6912) and down (6912 -> 2560) BitLinear layers. One step = the whole
hot path for that token: per-token int8 quantization (fused into the decode
kernel's prologue), ternary x int8 product, rescale -- for both matrices.
value = packed-weight bytes per step / step time (GB/s).

Every other workload is measured in the same run: prefill at 2048 tokens
through the two FFN matrices (int8 TOPS, "prefill"), and under "extra" the
small M=4, 256x256 layer (latency), one 2B-class layer at 1/8/32/64 tokens
(packed GB/s), the 8B-class FFN block at 1 and 2048 tokens (with the sparse
down projection at one token), and the variants: the RMS norm fused into the
quantization and 4-bit top-K activations on the decode and prefill shapes,
the three activation quantizers alone, and the two weight quantizers.

Cold weights: the packed matrices of the HBM-bound workloads rotate through a
pool of distinct copies larger than 2x the 256 MB last-level cache, and before
every timed region 1 GiB of unrelated memory is streamed through the caches,
so whatever --steps is, each timed step reads its weights from HBM.

Timing: steps are captured in HIP graphs (no host launch overhead) and timed
with HIP events on the stream the library launches on (torch's current
stream). The headline times exactly --steps steps after --warmup eager ones.
Before every timed region the region's own graph is also replayed untimed for
0.25 s: this GPU raises its clocks over the first ~0.1 s of sustained load, and
compute-bound workloads run ~10 % slower in a region started from idle.
`roofline` is for the dominant kernel of the headline, the decode GEMV: its
average launch duration comes from graphs of that kernel alone over the pool
(events, this run); the figure from the committed rocprofv3 kernel trace is
reported beside it while the kernel's sources match the ones traced. `read`
is the plain streaming read of the same cold matrices (the achievable
ceiling): once with the GEMV's grid and access pattern, once with the best
grid found. `cpu_baseline` times the CPU oracle on bounded samples of every
workload.

`--profile decode|prefill|layer8|layer32|layer64|ffn1|ffn1sparse|ffn2048|variants` runs one workload
eagerly (no graphs, no JSON line) for profilers: --steps steps, then one plain
256 MiB device copy whose HBM byte counters calibrate those of the kernels.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, TOP/s
METRIC = "W1.58A8 BitLinear: decode GB/s vs HBM peak; prefill int8 TOPS vs MFMA peak"

DECODE_PROFILE = os.path.join("profiles", "gemv_decode_m1_2560x6912_6912x2560.md")
DECODE_SOURCES = [os.path.join("bit_ternary_weight_bitlinear_amd", "csrc", f) for f in ("gemv.hip", "common.hpp")]
FLUSH_BYTES = 512 << 20        # each of the two flush buffers; a flush moves 1 GiB


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def r4(v):
    return None if v is None else round(float(v), 4)


# --------------------------------------------------------------------------- timing

class Timer:
    """Times graph replays with HIP events on torch's current stream (the stream
    the library launches on). `flush` streams 1 GiB of unrelated memory through
    the caches before each timed region.

    Before each timed region the workload's own graph is replayed untimed for
    at least WARM_S seconds: this GPU raises its clocks over the first ~0.1 s of
    sustained load (the 8B FFN at 2048 tokens takes ~408 us per call in a region
    started from idle and ~370 us from 0.1 s of load on), so a region started
    cold measures the clock ramp, not the kernels."""

    WARM_S = 0.25

    def __init__(self, torch, dev):
        self.torch = torch
        self.src = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.dst = torch.empty_like(self.src)

    def flush(self):
        self.dst.copy_(self.src)

    def capture(self, fn, n, start=0):
        t = self.torch
        g = t.cuda.CUDAGraph()
        side = t.cuda.Stream()
        side.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(side):
            fn(start)  # one eager call on the capture stream before capturing
        t.cuda.current_stream().wait_stream(side)
        with t.cuda.graph(g):
            for i in range(n):
                fn(start + i)
        t.cuda.synchronize()
        return g

    def warm(self, graphs):
        """Replays the graphs untimed until WARM_S seconds have passed (at least once)."""
        t0 = time.perf_counter()
        while True:
            for g in graphs:
                g.replay()
            self.torch.cuda.synchronize()
            if time.perf_counter() - t0 >= self.WARM_S:
                return

    def _events(self, body):
        t = self.torch
        st = t.cuda.current_stream()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record(st)
        body()
        b.record(st)
        t.cuda.synchronize()
        return a.elapsed_time(b) / 1e3

    def steps_region(self, fn, steps, cycle):
        """Exactly `steps` steps: a graph of one pool cycle replayed steps // cycle
        times, then a graph of the remaining steps. The graphs are replayed untimed
        for WARM_S seconds, then the caches are flushed. Returns seconds per step."""
        steps = max(1, steps)
        reps, rest = divmod(steps, cycle)
        g = self.capture(fn, cycle) if reps else None
        g_rest = self.capture(fn, rest) if rest else None
        self.warm([gr for gr in (g, g_rest) if gr is not None])
        self.flush()

        def body():
            for _ in range(reps):
                g.replay()
            if g_rest is not None:
                g_rest.replay()
        return self._events(body) / steps

    def launch_mean(self, fn, cycle, seconds=0.3):
        """Mean time per call of `fn` from a graph of `cycle` calls (one pool
        cycle) replayed for about `seconds`, after WARM_S seconds of untimed
        replays and a flush."""
        g = self.capture(fn, cycle)
        self.warm([g])
        t0 = time.perf_counter()
        g.replay()
        self.torch.cuda.synchronize()
        per = max(time.perf_counter() - t0, 1e-6)
        reps = int(min(5000, max(3, seconds / per)))
        self.flush()
        return self._events(lambda: [g.replay() for _ in range(reps)]) / (reps * cycle)


# --------------------------------------------------------------------------- inputs

_WEIGHTS = {}


def weights(cfg, tid, n, k):
    """Seeded fp32 weights, generated once per run and shared by the GPU legs and
    the CPU baseline (each side quantizes them itself)."""
    key = (cfg, tid, n, k)
    if key not in _WEIGHTS:
        _WEIGHTS[key] = synth.weights(cfg, tid, n, k)
    return _WEIGHTS[key]


def make_weights(bl, torch, cfg, tid, n, k, dev):
    w = torch.from_numpy(weights(cfg, tid, n, k)).to(dev)
    packed, gamma = bl.pack_weights(w)
    del w
    return packed, gamma


def act_tensor(torch, cfg, m, k, dev, dtype="bf16", **kw):
    x = synth.activations(cfg, m, k, dtype=dtype, **kw)
    if dtype == "f32":
        return torch.from_numpy(x).to(dev)
    return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)


def rotation_pool(mats, pool_bytes):
    """Distinct device copies of the packed matrices, cycled per step."""
    per = sum(p.numel() for p, _ in mats)
    copies = max(2, int(np.ceil(pool_bytes / per)))
    pool = [[(p.clone(), g) for p, g in mats] for _ in range(copies)]
    return pool, copies * per


def decode_inputs(bl, torch, dev):
    cfg = synth.WORKLOADS[2]
    mats, xs = [], []
    for tid, (k, n) in zip(("up", "down"), cfg["mats"]):
        mats.append(make_weights(bl, torch, 2, tid, n, k, dev))
        xs.append(act_tensor(torch, 2, 1, k, dev, outlier_channels=round(0.01 * k),
                             outlier_scale=cfg["outlier_scale"]))
    return cfg, mats, xs


def profile_fields():
    """Machine-readable fields of the committed decode profile, and whether the
    decode kernel's sources still hash to the ones that were profiled."""
    try:
        with open(os.path.join(ROOT, DECODE_PROFILE)) as f:
            text = f.read()
    except OSError:
        return {}, False
    fields = dict(re.findall(r"^([a-z0-9_-]+): (.+)$", text, re.M))
    h = hashlib.sha256()
    for src in DECODE_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return fields, fields.get("source-sha256") == h.hexdigest()


class ReadLib:
    """The plain streaming-read kernels of libbitlinear_bench.so."""

    def __init__(self, bl, torch, dev):
        path = os.path.join(os.path.dirname(bl.library_path()), "libbitlinear_bench.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        self.lib = ctypes.CDLL(path)
        i64, p, ci, cu = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32
        self.lib.blbench_read_rows.argtypes = [p, i64, i64, ci, ci, cu, p, p]
        self.lib.blbench_read_linear.argtypes = [p, i64, ci, ci, cu, p, p]
        self.sink = torch.zeros(65536, dtype=torch.int32, device=dev)
        self.torch = torch

    def rows(self, packed, grid, threads):
        n, ldw = packed.shape
        rc = self.lib.blbench_read_rows(packed.data_ptr(), n, ldw, grid, threads, 0x9E3779B9,
                                        self.sink.data_ptr(), self.torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"blbench_read_rows: {rc}")

    def linear(self, packed, grid, threads):
        rc = self.lib.blbench_read_linear(packed.data_ptr(), packed.numel(), grid, threads, 0x9E3779B9,
                                          self.sink.data_ptr(), self.torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"blbench_read_linear: {rc}")


# --------------------------------------------------------------------------- workloads

def bench_decode(bl, torch, dev, tm, steps, warmup, pool_mb):
    cfg, mats, xs = decode_inputs(bl, torch, dev)
    ys = [torch.empty((1, n), dtype=torch.float32, device=dev) for _, n in cfg["mats"]]
    pool, pool_bytes = rotation_pool(mats, pool_mb << 20)
    P = len(pool)
    packed_bytes = sum(p.numel() for p, _ in mats)
    algo_bytes = [p.numel() + x.numel() * 2 + y.numel() * 4 for (p, _), x, y in zip(mats, xs, ys)]

    def step(i):
        ws = pool[i % P]
        for j in range(2):
            bl.forward(xs[j], ws[j][0], ws[j][1], out=ys[j])

    for i in range(warmup):
        step(P - 1 - (i % P))
    t_step = tm.steps_region(step, steps, P)

    # the dominant kernel alone, per shape, and the plain reads of the same matrices
    rd = ReadLib(bl, torch, dev)
    per_shape, read_rows, read_lin = [], [], []
    for j in range(2):
        per_shape.append(tm.launch_mean(lambda i, j=j: bl.forward(xs[j], pool[i % P][j][0], pool[i % P][j][1],
                                                                   out=ys[j]), P))
        read_rows.append(tm.launch_mean(lambda i, j=j: rd.rows(pool[i % P][j][0], 256, 512), P))
        read_lin.append(tm.launch_mean(lambda i, j=j: rd.linear(pool[i % P][j][0], 1024, 256), P))
    return dict(ms_per_step=t_step * 1e3, steps=steps, packed_bytes_per_step=packed_bytes,
                gbs=packed_bytes / t_step / 1e9, kernel_s=per_shape, algo_bytes=algo_bytes,
                read_rows_s=read_rows, read_linear_s=read_lin, pool_bytes=pool_bytes, shapes=cfg["mats"])


def bench_small(bl, torch, dev, tm):
    cfg = synth.WORKLOADS[1]
    m, k, n = cfg["m"], cfg["k"], cfg["n"]
    packed, gamma = make_weights(bl, torch, 1, "W", n, k, dev)
    x = act_tensor(torch, 1, m, k, dev, dtype="f32", outlier_channels=cfg["outliers"],
                   outlier_scale=cfg["outlier_scale"])
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    t = tm.launch_mean(lambda i: bl.forward(x, packed, gamma, out=y), 100, seconds=0.1)
    return dict(workload="M=4, K=N=256, fp32 activations (2 channels x20)", us_per_forward=round(t * 1e6, 3))


def bench_layer(bl, torch, dev, tm, steps, warmup, pool_mb):
    cfg = synth.WORKLOADS[3]
    mats = [make_weights(bl, torch, 3, tid, n, k, dev)
            for tid, (k, n) in zip(("qkv", "o", "gate", "up", "down"), cfg["mats"])]
    pool, pool_bytes = rotation_pool(mats, pool_mb << 20)
    P = len(pool)
    packed_bytes = sum(p.numel() for p, _ in mats)
    out = dict(workload="one 2B-class layer: QKV 2560->3840, O 2560->2560, gate/up 2560->6912, "
                        "down 6912->2560, bf16 activations, weights cold from HBM",
               packed_bytes_per_layer=packed_bytes, pool_bytes=pool_bytes)
    for m in cfg["ms"]:
        xs = [act_tensor(torch, 3, m, k, dev) for k, _ in cfg["mats"]]
        ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for _, n in cfg["mats"]]
        wss = [torch.empty(max(1, bl.workspace_size(bl.OP_FORWARD, m, k, n)), dtype=torch.uint8, device=dev)
               for k, n in cfg["mats"]]

        def step(i):
            ws = pool[i % P]
            for j in range(len(mats)):
                bl.forward(xs[j], ws[j][0], ws[j][1], out=ys[j],
                           workspace=wss[j] if wss[j].numel() > 1 else None)

        for i in range(warmup):
            step(P - 1 - (i % P))
        t = tm.steps_region(step, steps, P)
        out[f"m{m}"] = dict(us_per_layer=round(t * 1e6, 3), packed_gbs=round(packed_bytes / t / 1e9, 2),
                            frac_of_hbm_peak=r4(packed_bytes / t / 1e9 / HBM_PEAK_GBS))
    return out


def bench_prefill(bl, torch, dev, tm, steps, warmup):
    cfg = synth.WORKLOADS[4]
    m = cfg["m"]
    mats, xs, ys, wss = [], [], [], []
    for tid, (k, n) in zip(("up", "down"), cfg["mats"]):
        mats.append(make_weights(bl, torch, 4, tid, n, k, dev))
        xs.append(act_tensor(torch, 4, m, k, dev, heavy_channels=round(0.01 * k)))
        ys.append(torch.empty((m, n), dtype=torch.float32, device=dev))
        wss.append(torch.empty(bl.workspace_size(bl.OP_FORWARD, m, k, n), dtype=torch.uint8, device=dev))

    def one(j):
        bl.forward(xs[j], mats[j][0], mats[j][1], out=ys[j], workspace=wss[j])

    for _ in range(warmup):
        one(0)
        one(1)
    t = tm.steps_region(lambda i: (one(0), one(1)), steps, min(steps, 8))
    per = [tm.launch_mean(lambda i, j=j: one(j), 8, seconds=0.2) for j in range(2)]
    ops = [2.0 * m * n * k for k, n in cfg["mats"]]
    return dict(workload="prefill m=2048: 2560->6912 + 6912->2560, bf16 activations (1% Student-t channels), "
                         "act-quant + GEMM per layer",
                ms_per_step=round(t * 1e3, 4), tops=round(sum(ops) / t / 1e12, 2),
                frac_of_int8_mfma_peak=r4(sum(ops) / t / 1e12 / INT8_MFMA_PEAK_TOPS),
                per_layer_us=[round(v * 1e6, 2) for v in per],
                per_layer_tops=[round(o / v / 1e12, 1) for o, v in zip(ops, per)])


def bench_ffn_sparse(bl, torch, tm, pool, x, steps, warmup, packed_bytes):
    """The one-token FFN with the down projection reading only the rows of the
    non-zero channels of h (input-major down weights, one copy per pool entry)."""
    hid = x.shape[1]
    f = pool[0][0][0].shape[0]
    tpool = [(g, u, (bl.pack_kmajor(d[0]), d[1])) for g, u, d in pool]
    ws = torch.empty(bl.workspace_size(bl.OP_FFN_SPARSE, 1, hid, f), dtype=torch.uint8, device=x.device)

    def step(i):
        g, u, dt = tpool[i % len(tpool)]
        bl.ffn_sparse(x, g, u, dt, workspace=ws)

    for i in range(warmup):
        step(len(tpool) - 1 - (i % len(tpool)))
    t = tm.steps_region(step, steps, len(tpool))
    _, hq, _ = bl.ffn_sparse(x, *tpool[0], return_hq=True)
    nz = float((hq != 0).float().mean().item())
    read = (2 * f * hid + nz * f * hid) / 4   # gate and up, then the down rows of the non-zero channels
    return dict(us_per_ffn=round(t * 1e6, 3), zero_channel_frac=round(1.0 - nz, 4),
                weight_bytes_read=int(read), read_gbs=round(read / t / 1e9, 2),
                packed_equiv_gbs=round(packed_bytes / t / 1e9, 2))


def bench_ffn(bl, torch, dev, tm, steps, warmup, pool_mb):
    cfg = synth.WORKLOADS[5]
    hid, f = cfg["hidden"], cfg["ffn"]
    mats = [make_weights(bl, torch, 5, "gate", f, hid, dev), make_weights(bl, torch, 5, "up", f, hid, dev),
            make_weights(bl, torch, 5, "down", hid, f, dev)]
    packed_bytes = 3 * f * hid // 4
    out = dict(workload="8B-class FFN block: gate+up 4096->14336, relu(g)^2*u, requant, down 14336->4096",
               packed_bytes=packed_bytes)
    for m in cfg["ms"]:
        # one token: weights cold from a rotation pool (HBM-bound); 2048 tokens:
        # compute-bound, one copy
        pool, pool_bytes = rotation_pool(mats, pool_mb << 20) if m == 1 else ([mats], packed_bytes)
        x = act_tensor(torch, 5, m, hid, dev)
        ws = torch.empty(bl.workspace_size(bl.OP_FFN, m, hid, f), dtype=torch.uint8, device=dev)

        def step(i):
            g, u, d = pool[i % len(pool)]
            bl.ffn(x, g, u, d, workspace=ws)

        for i in range(warmup):
            step(len(pool) - 1 - (i % len(pool)))
        t = tm.steps_region(step, steps, len(pool) if m == 1 else min(steps, 8))
        ops = 2.0 * m * 3 * f * hid
        if m == 1:
            out["m1"] = dict(us_per_ffn=round(t * 1e6, 3), packed_gbs=round(packed_bytes / t / 1e9, 2),
                             frac_of_hbm_peak=r4(packed_bytes / t / 1e9 / HBM_PEAK_GBS), pool_bytes=pool_bytes)
            out["m1_sparse_down"] = bench_ffn_sparse(bl, torch, tm, pool, x, steps, warmup, packed_bytes)
        else:
            out[f"m{m}"] = dict(ms_per_ffn=round(t * 1e3, 4), tops=round(ops / t / 1e12, 2),
                                frac_of_int8_mfma_peak=r4(ops / t / 1e12 / INT8_MFMA_PEAK_TOPS))
        del pool
    return out


def bench_variants(bl, torch, dev, tm, steps, warmup, pool_mb):
    """The other quantizers on the same shapes: the RMS norm fused into the
    activation quantization, 4-bit top-K activations (W1.58A4), and the
    threshold weight quantizer against the absmean one."""
    out = {}
    cfg = synth.WORKLOADS[2]
    _, mats, xs = decode_inputs(bl, torch, dev)
    pool, _ = rotation_pool(mats, pool_mb << 20)
    P = len(pool)
    packed_bytes = sum(p.numel() for p, _ in mats)
    gains = [(1.0 + 0.25 * torch.randn(x.shape[1], device=dev)).float().contiguous() for x in xs]
    wss = [torch.empty(max(bl.workspace_size(op, 1, k, n) for op in (bl.OP_FORWARD_NORM, bl.OP_FORWARD_A4)),
                       dtype=torch.uint8, device=dev) for k, n in cfg["mats"]]
    ys = [torch.empty((1, n), dtype=torch.float32, device=dev) for _, n in cfg["mats"]]
    dec = {}
    for name, fn in (("norm", lambda j, w: bl.forward_norm(xs[j], w[j][0], w[j][1], gains[j], out=ys[j],
                                                          workspace=wss[j])),
                     ("a4", lambda j, w: bl.forward_a4(xs[j], w[j][0], w[j][1], out=ys[j], workspace=wss[j]))):
        def step(i, fn=fn):
            w = pool[i % P]
            fn(0, w)
            fn(1, w)
        for i in range(warmup):
            step(P - 1 - (i % P))
        t = tm.steps_region(step, steps, P)
        dec[name] = dict(us_per_step=round(t * 1e6, 3), packed_gbs=round(packed_bytes / t / 1e9, 2),
                         frac_of_hbm_peak=r4(packed_bytes / t / 1e9 / HBM_PEAK_GBS))
    out["decode_m1_2560x6912_6912x2560"] = dec

    c4 = synth.WORKLOADS[4]
    m = c4["m"]
    pre, quant = {}, {}
    for (k, n), tid in zip(c4["mats"], ("up", "down")):
        x = act_tensor(torch, 4, m, k, dev, heavy_channels=round(0.01 * k))
        q = torch.empty((m, k), dtype=torch.int8, device=dev)
        sc = torch.empty(m, dtype=torch.float32, device=dev)
        lib = bl.load_library()
        stream = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
        calls = {"absmax_int8": lambda i: lib.bitlinear_quant_act(x.data_ptr(), 1, m, k, q.data_ptr(), sc.data_ptr(),
                                                                   stream()),
                 "rms_norm_int8": lambda i: lib.bitlinear_quant_act_norm(x.data_ptr(), 1, m, k, None, q.data_ptr(),
                                                                         sc.data_ptr(), stream()),
                 "topk_e2m1": lambda i: lib.bitlinear_quant_act_a4(x.data_ptr(), 1, m, k, (k + 1) // 2, q.data_ptr(),
                                                                   sc.data_ptr(), stream())}
        moved = m * k * 3  # bf16 in, int8 out
        quant[f"k{k}"] = {name: dict(us=round(tm.launch_mean(c, 8, seconds=0.1) * 1e6, 2),
                                     gbs=round(moved / tm.launch_mean(c, 8, seconds=0.1) / 1e9, 1))
                          for name, c in calls.items()}
        packed, gamma = make_weights(bl, torch, 4, tid, n, k, dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        ws = torch.empty(bl.workspace_size(bl.OP_FORWARD_A4, m, k, n), dtype=torch.uint8, device=dev)
        ops = 2.0 * m * n * k
        pre[f"{k}x{n}"] = {}
        for name, fn in (("norm", lambda i: bl.forward_norm(x, packed, gamma, out=y, workspace=ws)),
                         ("a4", lambda i: bl.forward_a4(x, packed, gamma, out=y, workspace=ws))):
            for _ in range(warmup):
                fn(0)
            t = tm.launch_mean(fn, 8, seconds=0.2)
            pre[f"{k}x{n}"][name] = dict(us=round(t * 1e6, 2), tops=round(ops / t / 1e12, 1),
                                         frac_of_int8_mfma_peak=r4(ops / t / 1e12 / INT8_MFMA_PEAK_TOPS))
    out["prefill_m2048"] = pre
    out["quantizers_m2048_us"] = quant

    packs = {}
    for n, k in ((6912, 2560), (14336, 4096)):
        w = torch.from_numpy(weights(5 if n == 14336 else 2, "gate" if n == 14336 else "up", n, k)).to(dev)
        pk = torch.empty((n, k // 4), dtype=torch.uint8, device=dev)
        g = torch.empty(4, dtype=torch.float32, device=dev)
        wsb = torch.empty(bl.workspace_size(bl.OP_PACK_THRESHOLD, 0, k, n), dtype=torch.uint8, device=dev)
        lib = bl.load_library()
        ab = lambda i: lib.bitlinear_pack_weights(w.data_ptr(), n, k, pk.data_ptr(), g.data_ptr(),  # noqa: E731
                                                  wsb.data_ptr(), wsb.numel(),
                                                  torch.cuda.current_stream().cuda_stream)
        th = lambda i: lib.bitlinear_pack_weights_threshold(w.data_ptr(), n, k, 0.7, pk.data_ptr(),  # noqa: E731
                                                            g.data_ptr(), g[1:].data_ptr(), wsb.data_ptr(),
                                                            wsb.numel(), torch.cuda.current_stream().cuda_stream)
        ta, tt = tm.launch_mean(ab, 2, seconds=0.2), tm.launch_mean(th, 2, seconds=0.2)
        packs[f"{n}x{k}"] = dict(absmean_us=round(ta * 1e6, 1), threshold_us=round(tt * 1e6, 1),
                                 fp32_weight_mb=round(n * k * 4 / 1e6, 1))
        del w
    out["weight_pack_offline"] = packs
    return out


# --------------------------------------------------------------------------- profiling

def profile_run(bl, torch, dev, what, steps, pool_mb):
    """Eager launches of one workload for rocprofv3, then a 256 MiB copy."""
    if what == "decode":
        cfg, mats, xs = decode_inputs(bl, torch, dev)
        ys = [torch.empty((1, n), dtype=torch.float32, device=dev) for _, n in cfg["mats"]]
        pool, _ = rotation_pool(mats, pool_mb << 20)
        rd = ReadLib(bl, torch, dev)
        for i in range(steps):
            ws = pool[i % len(pool)]
            for j in range(2):
                bl.forward(xs[j], ws[j][0], ws[j][1], out=ys[j])
        # the plain reads of the same cold matrices (GEMV grid and pattern, then linear)
        for i in range(steps):
            for j in range(2):
                rd.rows(pool[(i + steps) % len(pool)][j][0], 256, 512)
        for i in range(steps):
            for j in range(2):
                rd.linear(pool[(i + 2 * steps) % len(pool)][j][0], 1024, 256)
    elif what in ("layer8", "layer32", "layer64"):
        cfg = synth.WORKLOADS[3]
        m = int(what[len("layer"):])
        mats = [make_weights(bl, torch, 3, tid, n, k, dev)
                for tid, (k, n) in zip(("qkv", "o", "gate", "up", "down"), cfg["mats"])]
        pool, _ = rotation_pool(mats, pool_mb << 20)
        xs = [act_tensor(torch, 3, m, k, dev) for k, _ in cfg["mats"]]
        ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for _, n in cfg["mats"]]
        wss = [torch.empty(max(1, bl.workspace_size(bl.OP_FORWARD, m, k, n)), dtype=torch.uint8, device=dev)
               for k, n in cfg["mats"]]
        for i in range(steps):
            ws = pool[i % len(pool)]
            for j in range(len(mats)):
                bl.forward(xs[j], ws[j][0], ws[j][1], out=ys[j], workspace=wss[j] if wss[j].numel() > 1 else None)
    elif what in ("ffn1", "ffn1sparse"):
        cfg = synth.WORKLOADS[5]
        hid, f = cfg["hidden"], cfg["ffn"]
        mats = [make_weights(bl, torch, 5, "gate", f, hid, dev), make_weights(bl, torch, 5, "up", f, hid, dev),
                make_weights(bl, torch, 5, "down", hid, f, dev)]
        pool, _ = rotation_pool(mats, pool_mb << 20)
        x = act_tensor(torch, 5, 1, hid, dev)
        if what == "ffn1":
            ws = torch.empty(bl.workspace_size(bl.OP_FFN, 1, hid, f), dtype=torch.uint8, device=dev)
            for i in range(steps):
                g, u, d = pool[i % len(pool)]
                bl.ffn(x, g, u, d, workspace=ws)
        else:
            tpool = [(g, u, (bl.pack_kmajor(d[0]), d[1])) for g, u, d in pool]
            ws = torch.empty(bl.workspace_size(bl.OP_FFN_SPARSE, 1, hid, f), dtype=torch.uint8, device=dev)
            for i in range(steps):
                g, u, dt = tpool[i % len(tpool)]
                bl.ffn_sparse(x, g, u, dt, workspace=ws)
    elif what == "variants":
        # the RMS-norm and 4-bit forwards (decode, cold weights; 2048 tokens),
        # the threshold and absmean packs
        cfg, mats, xs = decode_inputs(bl, torch, dev)
        pool, _ = rotation_pool(mats, pool_mb << 20)
        for i in range(steps):
            ws = pool[i % len(pool)]
            for j in range(2):
                bl.forward_norm(xs[j], ws[j][0], ws[j][1])
        for i in range(steps):
            ws = pool[(i + steps) % len(pool)]
            for j in range(2):
                bl.forward_a4(xs[j], ws[j][0], ws[j][1])
        c4 = synth.WORKLOADS[4]
        for tid, (k, n) in zip(("up", "down"), c4["mats"]):
            packed, gamma = make_weights(bl, torch, 4, tid, n, k, dev)
            x = act_tensor(torch, 4, c4["m"], k, dev, heavy_channels=round(0.01 * k))
            for i in range(max(1, steps // 10)):
                bl.forward_norm(x, packed, gamma)
                bl.forward_a4(x, packed, gamma)
                bl.quant_act(x)
        w = torch.from_numpy(weights(5, "gate", 14336, 4096)).to(dev)
        for i in range(3):
            bl.pack_weights(w)
            bl.pack_weights_threshold(w, 0.7)
    elif what == "ffn2048":
        cfg = synth.WORKLOADS[5]
        hid, f, m = cfg["hidden"], cfg["ffn"], max(cfg["ms"])
        g = make_weights(bl, torch, 5, "gate", f, hid, dev)
        u = make_weights(bl, torch, 5, "up", f, hid, dev)
        d = make_weights(bl, torch, 5, "down", hid, f, dev)
        x = act_tensor(torch, 5, m, hid, dev)
        ws = torch.empty(bl.workspace_size(bl.OP_FFN, m, hid, f), dtype=torch.uint8, device=dev)
        for i in range(steps):
            bl.ffn(x, g, u, d, workspace=ws)
    else:
        cfg = synth.WORKLOADS[4]
        m = cfg["m"]
        for tid, (k, n) in zip(("up", "down"), cfg["mats"]):
            packed, gamma = make_weights(bl, torch, 4, tid, n, k, dev)
            x = act_tensor(torch, 4, m, k, dev, heavy_channels=round(0.01 * k))
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            ws = torch.empty(bl.workspace_size(bl.OP_FORWARD, m, k, n), dtype=torch.uint8, device=dev)
            for i in range(steps):
                bl.forward(x, packed, gamma, out=y, workspace=ws)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"profile {what}: {steps} steps, then one 256 MiB copy")


# --------------------------------------------------------------------------- CPU baseline

def _median_time(fn, reps=3):
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_baseline():
    """The CPU oracle, as it stands, on bounded samples of every workload: the
    median of 3 runs with all host threads (OpenMP over output rows), and for
    the small, decode and batched-decode workloads also with one thread. Large
    token counts are sampled (the rate per operation does not depend on how
    many tokens there are); each entry says what it ran."""
    import oracle
    nthreads = oracle.num_threads()
    out = {}

    def layer(cfg, tid, k, n, m, **act):
        p, g, _ = oracle.pack_weights(weights(cfg, tid, n, k))
        x = synth.activations(cfg, m, k, **act)
        return p, g, x

    def timed(run, threads):
        oracle.set_num_threads(threads)
        try:
            return _median_time(run)
        finally:
            oracle.set_num_threads(nthreads)

    # 1: m=4, 256x256, fp32 activations
    c1 = synth.WORKLOADS[1]
    p, g, x = layer(1, "W", c1["k"], c1["n"], c1["m"], dtype="f32", outlier_channels=2, outlier_scale=20.0)
    run = lambda: oracle.forward(x, p, g, c1["k"], "f32")  # noqa: E731
    out["small_m4_256x256"] = dict(us_all_threads=round(timed(run, nthreads) * 1e6, 1),
                                   us_1_thread=round(timed(run, 1) * 1e6, 1))

    # 2: decode, both matrices, one token
    c2 = synth.WORKLOADS[2]
    dec = [layer(2, tid, k, n, 1, outlier_channels=round(0.01 * k), outlier_scale=c2["outlier_scale"])
           for tid, (k, n) in zip(("up", "down"), c2["mats"])]
    dec_bytes = sum(p.size for p, _, _ in dec)
    run = lambda: [oracle.forward(x, p, g, x.shape[1], "bf16") for p, g, x in dec]  # noqa: E731
    t_all, t_one = timed(run, nthreads), timed(run, 1)
    out["decode_m1"] = dict(gbs_all_threads=round(dec_bytes / t_all / 1e9, 4),
                            gbs_1_thread=round(dec_bytes / t_one / 1e9, 4), us_per_step=round(t_all * 1e6, 1))
    headline = dec_bytes / t_all / 1e9

    # 3: one 2B-class layer; one thread at 1 and 8 tokens only (bounded)
    c3 = synth.WORKLOADS[3]
    lay = [(tid, k, n, oracle.pack_weights(weights(3, tid, n, k))[:2])
           for tid, (k, n) in zip(("qkv", "o", "gate", "up", "down"), c3["mats"])]
    lay_bytes = sum(pg[0].size for _, _, _, pg in lay)
    res3 = {}
    for m in c3["ms"]:
        xs = [synth.activations(3, m, k) for _, k, _, _ in lay]
        run = lambda xs=xs: [oracle.forward(x, pg[0], pg[1], k, "bf16")  # noqa: E731
                             for x, (_, k, _, pg) in zip(xs, lay)]
        e = dict(gbs_all_threads=round(lay_bytes / timed(run, nthreads) / 1e9, 4))
        if m <= 8:
            e["gbs_1_thread"] = round(lay_bytes / timed(run, 1) / 1e9, 4)
        res3[f"m{m}"] = e
    out["layer_2b"] = res3

    # 4: prefill, 128 of the 2048 tokens through both matrices (int8 TOPS)
    c4 = synth.WORKLOADS[4]
    ms = 128
    pre = []
    for tid, (k, n) in zip(("up", "down"), c4["mats"]):
        p, g, x = layer(4, tid, k, n, c4["m"], heavy_channels=round(0.01 * k))
        pre.append((p, g, x[:ms], k, n))
    run = lambda: [oracle.forward(x, p, g, k, "bf16") for p, g, x, k, _ in pre]  # noqa: E731
    ops = sum(2.0 * ms * n * k for _, _, _, k, n in pre)
    out["prefill_m2048"] = dict(tops_all_threads=round(ops / timed(run, nthreads) / 1e12, 5),
                                sample="128 of the 2048 tokens")

    # 5: 8B FFN at one token (GB/s) and 32 of the 2048 tokens (TOPS, one run)
    c5 = synth.WORKLOADS[5]
    hid, f = c5["hidden"], c5["ffn"]
    ws_ = {nm: oracle.pack_weights(weights(5, nm, *sh))[:2]
           for nm, sh in (("gate", (f, hid)), ("up", (f, hid)), ("down", (hid, f)))}
    x1 = synth.activations(5, 1, hid)
    t1 = timed(lambda: oracle.ffn(x1, ws_["gate"], ws_["up"], ws_["down"], hid, f, "bf16"), nthreads)
    xs = synth.activations(5, 2048, hid)[:32]
    oracle.set_num_threads(nthreads)
    t0 = time.perf_counter()
    oracle.ffn(xs, ws_["gate"], ws_["up"], ws_["down"], hid, f, "bf16")
    t32 = time.perf_counter() - t0
    out["ffn_8b"] = dict(m1_gbs_all_threads=round(3 * f * hid / 4 / t1 / 1e9, 4),
                         m2048_tops_all_threads=round(2.0 * 32 * 3 * f * hid / t32 / 1e12, 5),
                         m2048_sample="32 of the 2048 tokens, one run")
    return dict(value=round(headline, 4), unit="GB/s", cores=nthreads, kind="oracle",
                sample=(f"decode: both matrices (1 token through 2560->6912 and 6912->2560), median of 3 runs "
                        f"with {nthreads} OpenMP threads; per_config holds every workload (bounded samples "
                        f"as stated) and one-thread runs; CPU: {cpu_model()}, {os.cpu_count()} logical cores"),
                per_config=out)


# --------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pool-mb", type=int, default=640, help="rotation pool of packed weights (MB)")
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", choices=["decode", "prefill", "layer8", "layer32", "layer64", "ffn1", "ffn1sparse", "ffn2048",
                                          "variants"],
                    default=None, help="eager launches for a profiler; prints no JSON line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build measures one GPU only (--gpus 1); runs on several GPUs are not supported",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_ternary_weight_bitlinear_amd as bl
    bl.load_library()
    dev = torch.device("cuda:0")
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.profile:
        profile_run(bl, torch, dev, args.profile, args.steps, args.pool_mb)
        return

    tm = Timer(torch, dev)
    dec = bench_decode(bl, torch, dev, tm, args.steps, args.warmup, args.pool_mb)
    log(f"decode: {dec['ms_per_step']*1e3:.2f} us/step, {dec['gbs']:.1f} GB/s packed; GEMV "
        f"{[round(v * 1e6, 3) for v in dec['kernel_s']]} us, read (GEMV grid) "
        f"{[round(v * 1e6, 3) for v in dec['read_rows_s']]} us, read (1024 wg) "
        f"{[round(v * 1e6, 3) for v in dec['read_linear_s']]} us")
    heavy_steps, heavy_warmup = max(10, args.steps // 10), max(3, args.warmup // 5)
    extra = {}
    if not args.headline_only:
        extra["small"] = bench_small(bl, torch, dev, tm)
        log("small:", json.dumps(extra["small"]))
        extra["batched_decode_layer"] = bench_layer(bl, torch, dev, tm, args.steps, args.warmup, args.pool_mb)
        log("layer:", json.dumps(extra["batched_decode_layer"]))
    prefill = bench_prefill(bl, torch, dev, tm, heavy_steps, heavy_warmup)
    log("prefill:", json.dumps(prefill))
    if not args.headline_only:
        extra["ffn_8b"] = bench_ffn(bl, torch, dev, tm, heavy_steps, heavy_warmup, args.pool_mb)
        log("ffn:", json.dumps(extra["ffn_8b"]))
        extra["variants"] = bench_variants(bl, torch, dev, tm, args.steps, args.warmup, args.pool_mb)
        log("variants:", json.dumps(extra["variants"]))

    algo = float(np.mean(dec["algo_bytes"]))
    kmean = float(np.mean(dec["kernel_s"]))
    achieved = algo / kmean / 1e9
    fields, fresh = profile_fields()
    trace_us = float(fields["trace_gemv_mean_us"]) if fresh and "trace_gemv_mean_us" in fields else None
    traffic = int(fields["traffic_bytes_per_launch"]) if fresh and "traffic_bytes_per_launch" in fields else None
    read_rows_us = [v * 1e6 for v in dec["read_rows_s"]]
    read_lin_us = [v * 1e6 for v in dec["read_linear_s"]]
    roofline = dict(
        bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
        frac=r4(achieved / HBM_PEAK_GBS), traffic=traffic,
        kernel="gemv_kernel (decode: act-quant fused, v_dot4 on packed ternary codes)",
        algo_bytes_per_launch=algo,
        mean_launch_us=round(kmean * 1e6, 3),
        per_shape_launch_us=[round(v * 1e6, 3) for v in dec["kernel_s"]],
        timing="HIP events over graphs of this kernel alone (one matrix per launch, weights cold), this run",
        trace=(dict(mean_launch_us=trace_us, achieved=round(algo / (trace_us * 1e-6) / 1e9, 2),
                    frac=r4(algo / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBS),
                    read_gemv_grid_us=float(fields["trace_read_rows_mean_us"]),
                    read_best_grid_us=float(fields["trace_read_linear_mean_us"]),
                    source=f"rocprofv3 kernel trace of the bench, {DECODE_PROFILE}") if trace_us else None),
        traffic_note=(f"HBM bytes per launch from FETCH_SIZE/WRITE_SIZE, {DECODE_PROFILE}" if traffic else
                      "no counter summary for the current decode kernel sources"),
        read=dict(gemv_grid_us_per_shape=[round(v, 3) for v in read_rows_us],
                  gemv_grid_gbs=round(sum(dec["shapes"][j][0] * dec["shapes"][j][1] / 4 for j in range(2)) /
                                      (sum(read_rows_us) * 1e-6) / 1e9, 1),
                  best_grid_us_per_shape=[round(v, 3) for v in read_lin_us],
                  best_grid_gbs=round(sum(dec["shapes"][j][0] * dec["shapes"][j][1] / 4 for j in range(2)) /
                                      (sum(read_lin_us) * 1e-6) / 1e9, 1),
                  note="plain 16-byte non-temporal reads of the same cold packed matrices: 256 x 512 threads "
                       "in the GEMV's pattern, and 1024 x 256 threads linear"),
    )
    cpu = None if args.no_cpu_baseline else cpu_baseline()

    line = {
        "metric": METRIC,
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": dec["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x ternary -> int32 (bf16 in, fp32 out)",
        "data": "synthetic",
        "config": {"workload": "decode GEMV m=1: 2B-class FFN up 2560->6912 + down 6912->2560, bf16 "
                               "activations (1% channels x30), packed weights cold from HBM",
                   "m": 1, "shapes_k_n": dec["shapes"], "packed_bytes_per_step": dec["packed_bytes_per_step"],
                   "rotation_pool_bytes": dec["pool_bytes"], "cache_flush_bytes_before_timing": 2 * FLUSH_BYTES,
                   "untimed_replay_s_before_timing": Timer.WARM_S},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
