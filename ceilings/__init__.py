"""Benchmark support, not part of the tile-stream library: ctypes binding and
build of libpipeceil.so (ceiling.hip, pipe_ceiling.h in this folder).

Context-only HBM and LDS ceilings, timed beside the tile stream by bench.py:
plain grid-stride streaming copy and read kernels, the runtime's
device-to-device copy, plain kernels that walk column strips the way the tile
stream does, and LDS rates per instruction kind. They take no part in the
tile stream, and the library (libpipetile.so) neither builds nor loads them.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpipeceil.so")
SYMBOLS = ("ceil_copy", "ceil_read", "ceil_memcpy", "ceil_strip_copy", "ceil_strip_read",
           "ceil_strip_write", "ceil_lds")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python -m ceilings")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.ceil_copy.argtypes = [vp, vp, sz, i, i, i, vp]
        L.ceil_read.argtypes = [vp, vp, sz, i, i, vp]
        L.ceil_memcpy.argtypes = [vp, vp, sz, vp]
        i64 = ctypes.c_int64
        L.ceil_strip_copy.argtypes = [vp, vp, i64, i64, i64, i, i, vp]
        L.ceil_strip_read.argtypes = [vp, vp, i64, i64, i64, i, i, vp]
        L.ceil_strip_write.argtypes = [vp, i64, i64, i64, i, i, vp]
        L.ceil_lds.argtypes = [i, vp, vp, vp, i, i, vp]
        for f in SYMBOLS:
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def copy(src, dst, grid: int, unroll: int = 4, nt: int = 1, stream=None) -> None:
    """dst <- src (torch tensors of equal byte size) with the plain streaming copy."""
    _check(lib().ceil_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(),
                           grid, unroll, nt, stream), "ceil_copy")


def read(src, sink, grid: int, nt: int = 1, stream=None) -> None:
    """Stream-read every byte of src; sink is a 1-element int32 device tensor."""
    _check(lib().ceil_read(src.data_ptr(), sink.data_ptr(), src.numel() * src.element_size(),
                           grid, nt, stream), "ceil_read")


def memcpy(src, dst, stream=None) -> None:
    _check(lib().ceil_memcpy(dst.data_ptr(), src.data_ptr(), src.numel() * src.element_size(),
                             stream), "ceil_memcpy")


def _region(t):
    """(rows, pitch bytes, width bytes) of a row-major 2-D tensor whose rows do
    not overlap."""
    if t.dim() != 2 or t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) < t.shape[1]):
        raise ValueError("a 2-D row-major tensor with non-overlapping rows is required")
    es = t.element_size()
    return t.shape[0], max(t.stride(0), t.shape[1]) * es, t.shape[1] * es


def strip_copy(src, dst, strip_bytes: int, split: int = 1, stream=None) -> None:
    """dst <- src (2-D tensors of one shape and pitch), walked as column strips."""
    rows, pitch, width = _region(src)
    assert dst.shape == src.shape and dst.stride() == src.stride()
    _check(lib().ceil_strip_copy(src.data_ptr(), dst.data_ptr(), rows, pitch, width, strip_bytes,
                                 split, stream), "ceil_strip_copy")


def strip_read(src, sink, strip_bytes: int, split: int = 1, stream=None) -> None:
    rows, pitch, width = _region(src)
    _check(lib().ceil_strip_read(src.data_ptr(), sink.data_ptr(), rows, pitch, width, strip_bytes,
                                 split, stream), "ceil_strip_read")


def strip_write(dst, strip_bytes: int, split: int = 1, stream=None) -> None:
    rows, pitch, width = _region(dst)
    _check(lib().ceil_strip_write(dst.data_ptr(), rows, pitch, width, strip_bytes, split, stream),
           "ceil_strip_write")


# op: (name, bytes per wave instruction, waves that move bytes per workgroup)
LDS_OPS = {0: ("ds_read_b128", 1024, 8), 1: ("ds_read_b64_tr_b16", 512, 8),
           2: ("global_load_lds_dwordx4", 1024, 8), 3: ("ds_write_b128", 1024, 8),
           4: ("dma_waves_0_3_with_read_waves_4_7", 1024, 8), 5: ("read_waves_4_7_alone", 1024, 4),
           6: ("dma_waves_0_3_alone", 1024, 4)}


def lds(op: int, src, fold, clocks, grid: int, iters: int, stream=None) -> None:
    """One launch of the LDS ceiling kernel (see include/pipe_ceiling.h)."""
    _check(lib().ceil_lds(op, src.data_ptr() if src is not None else None, fold.data_ptr(),
                          clocks.data_ptr(), grid, iters, stream), "ceil_lds")


def lds_bytes(op: int, grid: int, iters: int) -> int:
    """Bytes one launch moves: the active waves x 8 instructions per iteration
    (for op 4, half of them by DMA and half by reads)."""
    _, per_instr, waves = LDS_OPS[op]
    return grid * waves * iters * 8 * per_instr


def build(verbose: bool = False) -> str:
    """Compile ceiling.hip for gfx950 into libpipeceil.so in this folder."""
    import subprocess
    import sys

    from async_stage_tile_amd.build import ARCH, hipcc
    here = os.path.dirname(os.path.abspath(__file__))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", here, os.path.join(here, "ceiling.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: ceiling.hip")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH
