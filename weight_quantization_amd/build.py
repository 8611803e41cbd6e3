"""Build libhlwq.so (HIP, gfx950) in-tree.

Steps:
1. compile and run the host table generator (Lloyd-Max codebooks and the
   bucket-search tables, verified by brute force while generating);
2. compile the kernels and the C ABI with hipcc into ``libhlwq.so`` next to
   this file;
3. compile the streaming-bandwidth probe that bench.py uses as its HBM ceiling
   into ``libhlwq_stream.so`` (include/hlwq_stream.h).

Run ``python -m weight_quantization_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libhlwq.so")
STREAM_LIB = os.path.join(HERE, "libhlwq_stream.so")

ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # one IEEE rounding per written operation: no mul+add contraction
    "-ffp-contract=off",
    # correctly rounded fp32 division and sqrt (the norm and its reciprocal)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # fp32 denormals kept, not flushed: the code search forms its bucket index
    # as a denormal, and blocks of tiny values have denormal squares
    "-fno-gpu-flush-denormals-to-zero",
    # keep fp32 arithmetic on unpacked VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def generate_tables() -> str:
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "gen_tables")
    _run(["g++", "-O2", "-std=c++17", "-Wall", "-o", exe, os.path.join(CSRC, "gen_tables.cpp")])
    r = _run([exe])
    inc = os.path.join(BUILD, "hlwq_tables.inc")
    with open(inc, "w") as f:
        f.write(r.stdout)
    return inc


def build_library(extra_flags=(), out: str = LIB, source: str | None = None) -> str:
    generate_tables()
    src = source or os.path.join(CSRC, "hlwq.hip")
    tmp = out + ".tmp"
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", BUILD, src, "-o", tmp]
    _run(cmd)
    os.replace(tmp, out)
    return out


def build_stream_library(out: str = STREAM_LIB) -> str:
    tmp = out + ".tmp"
    _run([_hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, os.path.join(CSRC, "stream_ceiling.hip"), "-o", tmp])
    os.replace(tmp, out)
    return out


def build(verbose: bool = True) -> str:
    path = build_library()
    stream = build_stream_library()
    if verbose:
        print(f"built {path} and {stream}", file=sys.stderr)
    return path


if __name__ == "__main__":
    build()
