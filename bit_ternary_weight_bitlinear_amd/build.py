"""Compile the gfx950 HIP sources into bit_ternary_weight_bitlinear_amd/libbitlinear.so
(the product library) and libbitlinear_bench.so (the benchmark's plain read
kernels, loaded by bench.py only).

Flags: correctly rounded fp32 division, no FMA contraction, no fast-math, no
denormal flushing (the quantizers decide integers in fp32 and must match the
definition bit for bit), and packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbitlinear.so")
BENCH_LIB = os.path.join(HERE, "libbitlinear_bench.so")
SOURCES = ["api.hip", "pack.hip", "act_quant.hip", "gemv.hip", "bgemv.hip", "gemm.hip", "skinny.hip",
           "sparse_down.hip", "bmma.hip"]
BENCH_SOURCES = ["bench_read.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, out_dir: str | None = None) -> str:
    out_dir = out_dir or os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, flush=True)
        return obj

    all_src = SOURCES + BENCH_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(all_src), os.cpu_count() or 1)) as ex:
        objs = dict(zip(all_src, ex.map(compile_one, all_src)))
    for lib, srcs in ((LIB, SOURCES), (BENCH_LIB, BENCH_SOURCES)):
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[objs[s] for s in srcs], "-o", lib + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
