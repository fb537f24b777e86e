"""Builds sparse_attention_block_qsa_amd/libqsa.so for gfx950 with hipcc.

Every kernel file is compiled to its own object in parallel, then the
objects are linked into one shared library.  Flags:
  --offload-arch=gfx950      CDNA4 only
  -O3 -ffp-contract=off      every fused multiply-add is written explicitly
  -target-feature -packed-fp32-ops
                             keep the compiler from forming packed fp32
                             arithmetic (v_pk_* on fp32)
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqsa.so")
OBJDIR = os.path.join(ROOT, "_build", "qsa")
SOURCES = ["qsa_api.hip", "qsa_attention.hip", "qsa_blockkeys.hip", "qsa_convert.hip",
           "qsa_decode.hip", "qsa_noalloc.hip", "qsa_score.hip", "qsa_small.hip", "qsa_tail.hip",
           "qsa_topk.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, extra: list[str], verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


BENCH_SRC = os.path.join(HERE, "bench_kernels", "qsa_bench.hip")
BENCH_LIB = os.path.join(HERE, "libqsa_bench.so")


def build_bench(verbose: bool = False) -> str:
    """libqsa_bench.so: the benchmark's measurement kernels (an MFMA loop and
    a streaming read), kept out of libqsa.so."""
    cmd = [HIPCC, *FLAGS, "-shared", "-o", BENCH_LIB + ".tmp", BENCH_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BENCH_LIB + ".tmp", BENCH_LIB)
    return BENCH_LIB


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    extra = list(extra or [])
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, verbose), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    build_bench(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
