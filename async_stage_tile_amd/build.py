"""Build the tile-stream library for gfx950 with hipcc, in-tree.

libpipetile.so -- the tile stream: all kernels + the C ABI of include/pipe_tile.h.

Every translation unit compiles to its own object, in parallel; the stream
kernel source is compiled once per group of stage counts. Then the library
is linked and moved into place atomically.

Usage: python -m async_stage_tile_amd.build  (or build() from Python).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpipetile.so")
ARCH = "gfx950"

# (source, object, extra defines)
UNITS = [
    ("pipe_api.hip", "pipe_api.o", []),
    ("pipe_stream_aux.hip", "pipe_stream_aux.o", []),
    ("pipe_stream.hip", "pipe_stream_s1_2.o", ["PIPE_STREAM_STAGES_LO=1", "PIPE_STREAM_STAGES_HI=2"]),
    ("pipe_stream.hip", "pipe_stream_s3_4.o", ["PIPE_STREAM_STAGES_LO=3", "PIPE_STREAM_STAGES_HI=4"]),
    ("pipe_stream.hip", "pipe_stream_s5_6.o", ["PIPE_STREAM_STAGES_LO=5", "PIPE_STREAM_STAGES_HI=6"]),
    ("pipe_stream.hip", "pipe_stream_s7_8.o", ["PIPE_STREAM_STAGES_LO=7", "PIPE_STREAM_STAGES_HI=8"]),
    ("pipe_unified.hip", "pipe_unified.o", []),
    ("pipe_gemm.hip", "pipe_gemm_ring.o", ["PIPE_GEMM_PART=1"]),
    ("pipe_gemm.hip", "pipe_gemm_unified.o", ["PIPE_GEMM_PART=2"]),
]
# Kept for callers that list the tile-stream sources.
SOURCES = sorted({u[0] for u in UNITS})


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpipetile.so")


def compile_command(src: str, obj: str, defines: list) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
        # Packed fp32 VALU forms are kept out of the generated code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        *[f"-D{d}" for d in defines],
        os.path.join(CSRC, src), "-o", obj,
    ]


def link_command(objs: list, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", out]


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {cmd[-3]}")


def _link(units: list, out: str, verbose: bool) -> None:
    objs = [os.path.join(OBJ, o) for (_, o, _) in units]
    tmp = out + ".tmp"
    _run(link_command(objs, tmp), verbose)
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    units = UNITS
    jobs = jobs or min(len(units), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, compile_command(s, os.path.join(OBJ, o), d), verbose)
                for (s, o, d) in units]
        for f in futs:
            f.result()
    _link(UNITS, LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
