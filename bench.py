#!/usr/bin/env python3
"""BitLinear W1.58A8 benchmark on one MI355X.

Headline (the JSON line's `value`): decode, 1 token through the 2B-class FFN up
(2560 -> 6912) and down (6912 -> 2560) BitLinear layers. One step = the whole
hot path for that token: per-token int8 quantization (fused into the decode
kernel's prologue), ternary x int8 product, rescale -- for both matrices. The
packed weights rotate through a pool of distinct copies larger than 2x the
256 MB last-level cache, so every step reads its weights from HBM.
value = packed-weight bytes per step / step time (GB/s).

Secondary (`prefill`, always measured): 2048 tokens through the same two
layers on the int8 MFMA path; TOPS = 2*M*N*K per layer / step time.
`--workload all` adds the batched-decode layer (m = 1, 8, 32, 64) and the
8B-class FFN block (m = 1, 2048) under "extra".

Timing: HIP events on the stream the kernels run on. `roofline` uses the
dominant kernel's average launch duration: a graph of launches of that kernel
alone (one matrix at a time, the same weight pool), timed over K launches.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

`--profile decode|prefill|layer8|ffn1|ffn2048` runs one workload eagerly (no graph
capture, no JSON line) for profilers: `--steps` steps, then one plain device
copy of 256 MiB whose HBM byte counters calibrate those of the kernels.
layer8 is the batched-decode layer at 8 tokens, ffn1 / ffn2048 the 8B FFN at
one / 2048 tokens.
"""
from __future__ import annotations

import argparse
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


DECODE_COUNTERS = os.path.join("profiles", "gemv_decode_m1_2560x6912_6912x2560.md")
DECODE_SOURCES = [os.path.join("bit_ternary_weight_bitlinear_amd", "csrc", f) for f in ("gemv.hip", "common.hpp")]


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


# --------------------------------------------------------------------------- helpers

class Timer:
    """Times work on torch's current stream (the stream the library launches on)
    with HIP events. Steps are captured into a HIP graph first, so the host's
    launch overhead is not part of the measurement; the graph is replayed."""

    def __init__(self, torch):
        self.torch = torch

    def capture(self, fn, n):
        t = self.torch
        g = t.cuda.CUDAGraph()
        side = t.cuda.Stream()
        side.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(side):
            fn(0)  # one eager call on the capture stream before capturing
        t.cuda.current_stream().wait_stream(side)
        with t.cuda.graph(g):
            for i in range(n):
                fn(i)
        t.cuda.synchronize()
        return g

    def graph_region(self, fn, steps, per_graph):
        """Times exactly `steps` steps: a graph of `per_graph` steps (one cycle
        of the weight pool) replayed steps // per_graph times, then a graph of
        the remaining steps. Returns (seconds per step, steps done)."""
        t = self.torch
        steps = max(1, steps)
        reps, rest = divmod(steps, per_graph)
        g = self.capture(fn, per_graph) if reps else None
        g_rest = self.capture(fn, rest) if rest else None
        for gr in (g, g_rest):  # warm replays
            if gr is not None:
                gr.replay()
        t.cuda.synchronize()
        st = t.cuda.current_stream()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            g.replay()
        if g_rest is not None:
            g_rest.replay()
        b.record(st)
        t.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / steps, steps


def make_weights(bl, torch, cfg, tid, n, k, dev):
    w = torch.from_numpy(synth.weights(cfg, tid, n, k)).to(dev)
    packed, gamma = bl.pack_weights(w)
    del w
    return packed, gamma


def act_tensor(torch, cfg, m, k, dev, **kw):
    xb = synth.activations(cfg, m, k, dtype="bf16", **kw)
    return torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)


def rotation_pool(torch, mats, pool_bytes):
    """Distinct device copies of the packed matrices, cycled per step."""
    per = sum(p.numel() for p, _ in mats)
    copies = max(2, int(np.ceil(pool_bytes / per)))
    pool = [[(p.clone(), g) for p, g in mats] for _ in range(copies)]
    return pool, copies * per


def counter_traffic():
    """HBM bytes per launch of the decode kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary (each counter scaled by what it reads for a
    plain copy of known size), or None when the kernel's sources differ from
    the ones the counters were taken with."""
    try:
        with open(os.path.join(ROOT, DECODE_COUNTERS)) as f:
            text = f.read()
    except OSError:
        return None
    fields = dict(re.findall(r"^(traffic_bytes_per_launch|source-sha256): (\S+)$", text, re.M))
    h = hashlib.sha256()
    for src in DECODE_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if fields.get("source-sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


# --------------------------------------------------------------------------- workloads

def bench_decode(bl, torch, dev, steps, warmup, pool_mb):
    cfg = synth.WORKLOADS[2]
    mats, xs, ys = [], [], []
    for tid, (k, n) in zip(("up", "down"), cfg["mats"]):
        mats.append(make_weights(bl, torch, 2, tid, n, k, dev))
        xs.append(act_tensor(torch, 2, 1, k, dev, outlier_channels=round(0.01 * k),
                             outlier_scale=cfg["outlier_scale"]))
        ys.append(torch.empty((1, n), dtype=torch.float32, device=dev))
    pool, pool_bytes = rotation_pool(torch, mats, pool_mb << 20)
    packed_bytes = sum(p.numel() for p, _ in mats)
    algo_bytes = [p.numel() + x.numel() * 2 + y.numel() * 4 for (p, _), x, y in zip(mats, xs, ys)]

    def step(i):
        ws = pool[i % len(pool)]
        for j in range(2):
            bl.forward(xs[j], ws[j][0], ws[j][1], out=ys[j])

    for i in range(warmup):
        step(i)
    tm = Timer(torch)
    t_step, done = tm.graph_region(step, steps, len(pool))
    # the dominant kernel alone, per shape: a graph of launches of one matrix, cycling the pool
    per_shape = []
    for j in range(2):
        def one(i, j=j):
            ws = pool[i % len(pool)]
            bl.forward(xs[j], ws[j][0], ws[j][1], out=ys[j])
        tl, _ = tm.graph_region(one, steps, len(pool))
        per_shape.append(tl)
    res = dict(ms_per_step=t_step * 1e3, steps_done=done, packed_bytes_per_step=packed_bytes,
               gbs=packed_bytes / t_step / 1e9,
               kernel_mean_s=float(np.mean(per_shape)), kernel_per_shape_s=per_shape,
               algo_bytes_per_launch=float(np.mean(algo_bytes)),
               pool_bytes=pool_bytes, shapes=cfg["mats"])
    return res, (mats, xs)


def bench_prefill(bl, torch, dev, steps, warmup):
    cfg = synth.WORKLOADS[4]
    m = cfg["m"]
    mats, xs, ys, wss = [], [], [], []
    for tid, (k, n) in zip(("up", "down"), cfg["mats"]):
        mats.append(make_weights(bl, torch, 4, tid, n, k, dev))
        xs.append(act_tensor(torch, 4, m, k, dev, heavy_channels=round(0.01 * k)))
        ys.append(torch.empty((m, n), dtype=torch.float32, device=dev))
        wss.append(torch.empty(bl.workspace_size(bl.OP_FORWARD, m, k, n), dtype=torch.uint8, device=dev))

    def step(i):
        for j in range(2):
            bl.forward(xs[j], mats[j][0], mats[j][1], out=ys[j], workspace=wss[j])

    for i in range(warmup):
        step(i)
    t, _ = Timer(torch).graph_region(step, steps, min(steps, 8))
    ops = sum(2.0 * m * n * k for k, n in cfg["mats"])
    return dict(ms_per_step=t * 1e3, tops=ops / t / 1e12, ops_per_step=ops,
                frac_of_mfma_peak=ops / t / 1e12 / INT8_MFMA_PEAK_TOPS, m=m, shapes=cfg["mats"])


def bench_layer(bl, torch, dev, steps, warmup, pool_mb):
    cfg = synth.WORKLOADS[3]
    mats = [make_weights(bl, torch, 3, tid, n, k, dev)
            for tid, (k, n) in zip(("qkv", "o", "gate", "up", "down"), cfg["mats"])]
    pool, pool_bytes = rotation_pool(torch, mats, pool_mb << 20)
    packed_bytes = sum(p.numel() for p, _ in mats)
    out = {}
    for m in cfg["ms"]:
        xs = [act_tensor(torch, 3, m, k, dev) for k, _ in cfg["mats"]]
        ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for _, n in cfg["mats"]]
        wss = [torch.empty(max(1, bl.workspace_size(bl.OP_FORWARD, m, k, n)), dtype=torch.uint8, device=dev)
               for k, n in cfg["mats"]]

        def step(i):
            ws = pool[i % len(pool)]
            for j in range(len(mats)):
                bl.forward(xs[j], ws[j][0], ws[j][1], out=ys[j], workspace=wss[j])

        for i in range(warmup):
            step(i)
        t, _ = Timer(torch).graph_region(step, steps, len(pool))
        out[f"m{m}"] = dict(ms_per_step=t * 1e3, packed_gbs=packed_bytes / t / 1e9,
                            frac_of_hbm_peak=packed_bytes / t / 1e9 / HBM_PEAK_GBS)
    out["packed_bytes_per_layer"] = packed_bytes
    out["pool_bytes"] = pool_bytes
    return out


def bench_ffn(bl, torch, dev, steps, warmup, pool_mb):
    cfg = synth.WORKLOADS[5]
    hid, f = cfg["hidden"], cfg["ffn"]
    mats = [make_weights(bl, torch, 5, "gate", f, hid, dev), make_weights(bl, torch, 5, "up", f, hid, dev),
            make_weights(bl, torch, 5, "down", hid, f, dev)]
    packed_bytes = 3 * f * hid // 4
    out = {}
    for m in cfg["ms"]:
        # one token: the weights rotate through distinct copies (cold from HBM,
        # as for decode); 2048 tokens: compute-bound, one copy
        pool, pool_bytes = rotation_pool(torch, mats, pool_mb << 20) if m == 1 else ([mats], packed_bytes)
        x = act_tensor(torch, 5, m, hid, dev)
        ws = torch.empty(bl.workspace_size(bl.OP_FFN, m, hid, f), dtype=torch.uint8, device=dev)

        def step(i):
            g, u, d = pool[i % len(pool)]
            bl.ffn(x, g, u, d, workspace=ws)

        for i in range(warmup):
            step(i)
        t, _ = Timer(torch).graph_region(step, steps, len(pool) if m == 1 else min(steps, 8))
        ops = 2.0 * m * 3 * f * hid
        out[f"m{m}"] = dict(ms_per_step=t * 1e3, packed_gbs=packed_bytes / t / 1e9, tops=ops / t / 1e12,
                            pool_bytes=pool_bytes)
        del pool
    return out


def profile_run(bl, torch, dev, what, steps, pool_mb):
    """Eager launches of one workload for rocprofv3, then a 256 MiB copy."""
    if what == "decode":
        cfg = synth.WORKLOADS[2]
        mats, xs, ys = [], [], []
        for tid, (k, n) in zip(("up", "down"), cfg["mats"]):
            mats.append(make_weights(bl, torch, 2, tid, n, k, dev))
            xs.append(act_tensor(torch, 2, 1, k, dev, outlier_channels=round(0.01 * k),
                                 outlier_scale=cfg["outlier_scale"]))
            ys.append(torch.empty((1, n), dtype=torch.float32, device=dev))
        pool, _ = rotation_pool(torch, mats, pool_mb << 20)
        for i in range(steps):
            ws = pool[i % len(pool)]
            for j in range(2):
                bl.forward(xs[j], ws[j][0], ws[j][1], out=ys[j])
    elif what == "layer8":
        # the 2B-class layer at 8 tokens, weights cold from the rotation pool
        cfg = synth.WORKLOADS[3]
        m = 8
        mats = [make_weights(bl, torch, 3, tid, n, k, dev)
                for tid, (k, n) in zip(("qkv", "o", "gate", "up", "down"), cfg["mats"])]
        pool, _ = rotation_pool(torch, mats, pool_mb << 20)
        xs = [act_tensor(torch, 3, m, k, dev) for k, _ in cfg["mats"]]
        ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for _, n in cfg["mats"]]
        wss = [torch.empty(max(1, bl.workspace_size(bl.OP_FORWARD, m, k, n)), dtype=torch.uint8, device=dev)
               for k, n in cfg["mats"]]
        for i in range(steps):
            ws = pool[i % len(pool)]
            for j in range(len(mats)):
                bl.forward(xs[j], ws[j][0], ws[j][1], out=ys[j], workspace=wss[j])
    elif what == "ffn1":
        # the 8B-class FFN block at one token, weights cold from the rotation pool
        cfg = synth.WORKLOADS[5]
        hid, f = cfg["hidden"], cfg["ffn"]
        mats = [make_weights(bl, torch, 5, "gate", f, hid, dev), make_weights(bl, torch, 5, "up", f, hid, dev),
                make_weights(bl, torch, 5, "down", hid, f, dev)]
        pool, _ = rotation_pool(torch, mats, pool_mb << 20)
        x = act_tensor(torch, 5, 1, hid, dev)
        ws = torch.empty(bl.workspace_size(bl.OP_FFN, 1, hid, f), dtype=torch.uint8, device=dev)
        for i in range(steps):
            g, u, d = pool[i % len(pool)]
            bl.ffn(x, g, u, d, workspace=ws)
    elif what == "ffn2048":
        # the 8B-class FFN block at 2048 tokens (compute-bound: one copy of the weights)
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

def cpu_baseline(budget_s: float = 12.0):
    """The CPU oracle on a bounded sample of the decode workload: whole steps
    (both matrices, one token each) until ~budget_s of CPU time is used."""
    import oracle
    cfg = synth.WORKLOADS[2]
    mats, xs = [], []
    for tid, (k, n) in zip(("up", "down"), cfg["mats"]):
        w = synth.weights(2, tid, n, k)
        p, g, _ = oracle.pack_weights(w)
        mats.append((p, g, k))
        xs.append(synth.activations(2, 1, k, dtype="bf16", outlier_channels=round(0.01 * k),
                                    outlier_scale=cfg["outlier_scale"]))
    packed_bytes = sum(p.size for p, _, _ in mats)
    steps, t0 = 0, time.perf_counter()
    while True:
        for (p, g, k), x in zip(mats, xs):
            oracle.forward(x, p, g, k, "bf16")
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 10000:
            break
    return dict(value=packed_bytes * steps / el / 1e9, unit="GB/s", cores=oracle.num_threads(),
                kind="oracle", sample=f"{steps} decode steps (1 token through 2560->6912 and 6912->2560) "
                                      f"in {el:.1f} s; CPU: {cpu_model()}, {os.cpu_count()} logical cores")


# --------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pool-mb", type=int, default=640, help="rotation pool of packed weights (MB)")
    ap.add_argument("--workload", choices=["default", "all"], default="default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", choices=["decode", "prefill", "layer8", "ffn1", "ffn2048"], default=None,
                    help="eager launches for a profiler; prints no JSON line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build measures one GPU only (--gpus 1); multi-GPU runs are not supported",
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

    dec, _ = bench_decode(bl, torch, dev, args.steps, args.warmup, args.pool_mb)
    log(f"decode: {dec['ms_per_step']*1e3:.2f} us/step, {dec['gbs']:.1f} GB/s packed, "
        f"kernel {dec['kernel_mean_s']*1e6:.2f} us mean")
    pre = bench_prefill(bl, torch, dev, max(10, args.steps // 10), max(3, args.warmup // 5))
    log(f"prefill: {pre['ms_per_step']:.3f} ms/step, {pre['tops']:.1f} TOPS")
    extra = {}
    if args.workload == "all":
        extra["batched_decode_layer"] = bench_layer(bl, torch, dev, args.steps, args.warmup, args.pool_mb)
        log("layer:", json.dumps(extra["batched_decode_layer"]))
        extra["ffn_8b"] = bench_ffn(bl, torch, dev, max(10, args.steps // 10), max(3, args.warmup // 5), args.pool_mb)
        log("ffn:", json.dumps(extra["ffn_8b"]))

    achieved = dec["algo_bytes_per_launch"] / dec["kernel_mean_s"] / 1e9
    traffic = counter_traffic()
    roofline = dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    traffic_note=(f"HBM bytes per launch, {DECODE_COUNTERS}" if traffic else
                                  "no counter summary for the current decode kernel sources"),
                    kernel="gemv_kernel (decode, fused act-quant + v_dot4)",
                    algo_bytes_per_launch=dec["algo_bytes_per_launch"],
                    mean_launch_us=round(dec["kernel_mean_s"] * 1e6, 3),
                    per_shape_launch_us=[round(v * 1e6, 3) for v in dec["kernel_per_shape_s"]])
    cpu = None if args.no_cpu_baseline else cpu_baseline()

    line = {
        "metric": METRIC,
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": dec["steps_done"],
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xternary->int32 (bf16 in, fp32 out)",
        "data": "synthetic",
        "config": {"workload": "decode GEMV m=1: 2B-class FFN up 2560->6912 + down 6912->2560, bf16 "
                               "activations (1% channels x30), packed weights cold from HBM",
                   "m": 1, "shapes_k_n": dec["shapes"], "packed_bytes_per_step": dec["packed_bytes_per_step"],
                   "rotation_pool_bytes": dec["pool_bytes"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prefill": {"workload": "prefill GEMM m=2048: 2560->6912 + 6912->2560, bf16 activations "
                                "(1% Student-t channels)", "tops": round(pre["tops"], 2),
                    "ms_per_step": round(pre["ms_per_step"], 4),
                    "frac_of_int8_mfma_peak": round(pre["frac_of_mfma_peak"], 4)},
    }
    if extra:
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
