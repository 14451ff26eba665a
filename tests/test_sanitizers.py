"""The CPU oracle and the host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed). Each is built into its own
executable with the sanitizers on host code only and run as a subprocess; a
sanitizer report or a failed check fails the test."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-ffp-contract=off", os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "bitlinear_oracle.c"), "-o", exe, "-lm"], ROOT)
    r = _run([exe], ROOT)
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
def test_abi_host_validation_under_asan_ubsan(tmp_path):
    """api.hip's host code (argument checks, workspace sizes) with the
    sanitizers on its host pass only, linked with the kernels' ordinary objects
    from the library build (never launched here)."""
    from bit_ternary_weight_bitlinear_amd import build as hip_build
    hipcc = "/opt/rocm/bin/hipcc"
    csrc = os.path.join(ROOT, "bit_ternary_weight_bitlinear_amd", "csrc")
    objdir = os.path.join(ROOT, "bit_ternary_weight_bitlinear_amd", "_build")
    kernels = [s for s in hip_build.SOURCES if s != "api.hip"]
    if not all(os.path.exists(os.path.join(objdir, s.replace(".hip", ".o"))) for s in kernels):
        hip_build.build()
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    host_san = [a for f in san for a in ("-Xarch_host", f)]
    api = str(tmp_path / "api.o")
    _run([hipcc, *hip_build.FLAGS, *host_san, "-g", "-c", os.path.join(csrc, "api.hip"), "-o", api], ROOT)
    drv = str(tmp_path / "abi_driver.o")
    _run(["g++", "-std=c++17", "-g", *san, "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", drv], ROOT)
    exe = str(tmp_path / "abi_driver")
    _run([hipcc, "--offload-arch=gfx950", *host_san, drv, api,
          *[os.path.join(objdir, s.replace(".hip", ".o")) for s in kernels], "-o", exe], ROOT)
    r = _run([exe], ROOT)
    assert "abi driver: ok" in r.stdout
