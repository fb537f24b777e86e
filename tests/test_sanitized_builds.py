"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

  * the C oracle (oracle/qsa_oracle.c) linked into a driver that checks it
    on closed-form inputs with padded strides (tests/pins/oracle_sanitize_main.c);
  * the host side of the C ABI (csrc/qsa_api.hip compiled for the host only,
    with the sanitizers on the host pass) linked into a driver with stand-in
    launchers that checks every refusal, empty call and launch sizing
    (tests/pins/abi_host_check.cpp).
Device code is never built with a sanitizer here."""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "pins")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
          "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-o", exe, os.path.join(ROOT, "oracle", "qsa_oracle.c"),
          os.path.join(PINS, "oracle_sanitize_main.c"), "-lm"])
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert "passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm compilers not installed")
def test_abi_host_side_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "sparse_attention_block_qsa_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o, drv_o = str(tmp_path / "api.o"), str(tmp_path / "drv.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *san, *inc,
          "-c", os.path.join(csrc, "qsa_api.hip"), "-o", api_o])
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *san, *inc, "-x", "hip",
          "-c", os.path.join(PINS, "abi_host_check.cpp"), "-o", drv_o])
    exe = str(tmp_path / "abi_san")
    # host link only (no device code on this line)
    _run([CLANGXX, "-fsanitize=address,undefined", "-o", exe, api_o, drv_o])
    r = _run([exe], env=SAN_ENV, timeout=120)
    assert "passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
