"""Benchmark of the pipelined tile stream on one MI355X.

Headline (the JSON line's `value`): achieved HBM bandwidth (read + write) of
the streaming tile copy, fp16 16384 x 16384 (1 GiB moved per step), 128 x 64
tiles through an S-slot LDS ring, persistent workgroups each streaming one
column strip. One step = one launch of the whole hot path over the matrix
(tile walk, cursor/barrier handshakes, direct-to-LDS producer, consumer
copy-out, release, tail).

Also reported (in "extras"):
  * the copy's ring-depth sweep S = 1..8;
  * per-launch kernel times (median and min) of the headline copy and of the
    row sum, both back to back ("hot") and with the 256 MB MALL flushed by
    writing a 1 GiB scratch buffer before every launch ("cold", untimed flush);
  * the row sum of fp16 8192 x 65536 (GB/s) and the GEMM mainloop 4096^3 bf16
    (TFLOP/s) at the library's default configuration;
  * the unified (non-specialised) variant of the copy and the row sum;
  * context ceilings on the same device: the runtime's device-to-device copy,
    torch's copy and plain streaming copy / read kernels with no LDS ring
    (libpipeceil.so), and plain kernels that read, write or copy the headline
    matrix in the tile stream's own pattern (column strips 128 or 512 bytes
    wide);
  * the CPU oracle on bounded samples of the copy, row sum and GEMM, on one
    thread and on all host threads;
  * per-launch latency of the two small functional workloads (256 x 128 in
    2 x 2 tiles through one slot; 128 x 512 through a three-slot ring of one
    workgroup with per-tile checksums), each checked bit for bit.

roofline.traffic: HBM bytes per launch of the headline kernel from rocprofv3
FETCH_SIZE / WRITE_SIZE counters (scaled by the counts the same counters give
for a known-size device copy), read from the committed counter summary under
profiles/ -- reported only while the kernel sources are unchanged since.

Timing: first `--settle` seconds (default 1) of untimed headline copies so
that the device reaches steady clocks; then, per measurement, `warmup`
untimed steps and exactly `steps` steps between synchronisations; per-launch
kernel time from HIP events recorded on the launch stream. Inputs are
generated on the device before the timed region.

cpu_baseline: the CPU oracle (oracle.results.tile_copy) timed on a bounded
sample of the same matrix on the host, single-threaded numpy.

`--only copy|rowsum|gemm|ceiling|calib` times one workload (for profiling)
and prints no JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (read+write) of pipelined tile stream, % of peak, 1 GPU"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0

COPY_M = COPY_N = 16384
ROWSUM_M, ROWSUM_N = 8192, 65536
GEMM_N = 4096


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "copy_16384x16384_counters.md")
KERNEL_SOURCES = ("pipe_device.hpp", "pipe_kernels.hpp", "pipe_rowsum.hpp", "pipe_stream.hip")
MALL_FLUSH_BYTES = 1 << 30

# Wider 16 KiB tiles (64 x 128, 32 x 256) at the launch shapes measured best for
# them on MI355X: enough interleaved strip segments to give every CU a
# workgroup, 4 producer waves, lazy commits for the copy.
_NT, _RM, _IL, _LZ, _U = 0x4, 0x10, 0x20, 0x80, 0x40
WIDE_COPY = {
    "64x128": dict(tile_m=64, tile_n=128, stages=3, producer_waves=4, consumer_waves=4, split=2,
                   flags=_NT | _RM | _IL | _LZ),
    "32x256": dict(tile_m=32, tile_n=256, stages=2, producer_waves=4, consumer_waves=8, split=4,
                   flags=_NT | _RM | _IL | _LZ),
}
# 128 x 64 tiles down column strips 4 tile columns wide (PIPE_FLAG_STRIP_GROUPS):
# consumers store a tile row of the strip as 512-byte row runs; 4 interleaved
# segments per strip, the best ring measured for it (non-temporal, no XCD remap).
_G = 0x4000
GROUPED_COPY = dict(stages=5, producer_waves=2, consumer_waves=4, flags=_NT | _IL | _LZ | _G)
# The same strips with grouped loads (PIPE_FLAG_GROUP_LOADS): producers fill the
# 4 slots of a tile row with 2-row x 512-byte loads. 16 interleaved segments per
# strip: 1024 workgroups of 32 tiles, four in a row on each CU (the best of the
# ring depth, wave count and segment sweeps measured for it).
_GL = 0x80000
GROUP_LOAD_COPY = dict(stages=8, producer_waves=4, consumer_waves=4, split=16,
                       flags=_NT | _IL | _LZ | _G | _GL)
# The GEMM without warp specialisation: 256 x 256 output tiles, all 16 waves
# load a share of each stage and all compute, one barrier per K step.
UNIFIED_GEMM = dict(tile_m=256, tile_n=256, consumer_waves=16, flags=_U)
# The same with 4 waves of 128 x 128 output blocks (one wave per SIMD): 64-K
# stages in two slots, or 32-K stages in four.
WIDE_GEMM = dict(tile_m=256, tile_n=256, consumer_waves=4, flags=_U)
DEEP_GEMM = dict(tile_m=256, tile_n=256, tile_k=32, consumer_waves=4, flags=_U)
# The register producer engine (PIPE_FLAG_PRODUCER_VGPR): global_load_dwordx4
# into registers, then ds_write_b128 into the slot.
_V = 0x8000
REGS_COPY = dict(stages=2, producer_waves=4, consumer_waves=4, flags=_NT | _RM | _V)
REGS_ROWSUM = dict(stages=4, producer_waves=4, consumer_waves=4, flags=_NT | _RM | _V)
WIDE_ROWSUM = {
    "64x128": dict(tile_m=64, tile_n=128, stages=3, producer_waves=4, consumer_waves=4, split=2,
                   flags=_NT | _RM),
    "32x256": dict(tile_m=32, tile_n=256, stages=3, producer_waves=4, consumer_waves=4, split=1,
                   flags=_NT | _RM),
    "32x256_unified": dict(tile_m=32, tile_n=256, stages=2, consumer_waves=4, split=2,
                           flags=_U | _NT | _RM),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def strip_comments(src):
    """C/C++ source text without comments and with every run of whitespace
    reduced to one space (string and character literals kept as they are), so
    that edits to comments or layout do not count as kernel changes."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(read=None):
    """sha256 (first 16 hex digits) of the stream kernel's device sources with
    comments and layout removed (strip_comments). `read(name)` returns a
    source's text (default: the file under async_stage_tile_amd/csrc)."""
    import hashlib

    def read_file(name):
        with open(os.path.join(ROOT, "async_stage_tile_amd", "csrc", name)) as fh:
            return fh.read()

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(strip_comments((read or read_file)(f)).encode())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_name):
    """HBM bytes per launch measured by rocprofv3 counters for this exact kernel.

    Read from the `traffic_record:` line of the committed counter summary; None
    when there is none, or when the kernel or its sources changed since the
    counters were taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            lines = [ln for ln in f if ln.startswith("traffic_record:")]
    except OSError:
        return None
    for ln in lines:
        rec = json.loads(ln.split(":", 1)[1])
        if rec.get("kernel") == kernel_name and rec.get("source_hash") == kernel_source_hash():
            return rec.get("traffic_bytes_per_launch")
    return None


def timed_launches(fn, steps, warmup):
    """Run fn() warmup times, then exactly `steps` times back to back.

    One HIP event pair on the launch stream brackets the `steps` launches; the
    host clock brackets the same region between two synchronisations.
    Returns (wall ms per step, event ms per step)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    kern = a.elapsed_time(b) / steps
    return wall, kern


def launch_stats(fn, reps, warmup, before=None):
    """Per-launch kernel time: each of `reps` launches between its own event
    pair; before() (e.g. a cache flush) runs ahead of each pair, untimed.
    Returns (median ms, min ms)."""
    import statistics

    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    return statistics.median(times), min(times)


_FLUSH = {}


def mall_flush():
    """Write a 1 GiB scratch buffer: evicts the inputs from the 256 MB MALL."""
    import torch
    if "buf" not in _FLUSH:
        _FLUSH["buf"] = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        _FLUSH["k"] = 0
    _FLUSH["k"] = (_FLUSH["k"] + 1) % 251
    _FLUSH["buf"].fill_(_FLUSH["k"])


def hot_cold(fn, nbytes, reps, warmup):
    out = {}
    for name, before in (("hot", None), ("cold", mall_flush)):
        med, mn = launch_stats(fn, reps, warmup, before)
        out[name] = {"median_ms": med, "min_ms": mn, "median_gbs": nbytes / (med * 1e-3) / 1e9,
                     "best_gbs": nbytes / (mn * 1e-3) / 1e9}
    return out


_COPY_BUF = {}


def copy_buffers():
    import torch

    import synth
    if not _COPY_BUF:
        src = synth.uniform((COPY_M, COPY_N), torch.float16, seed=42, device="cuda")
        _COPY_BUF["src"] = src
        _COPY_BUF["dst"] = torch.empty_like(src)
    return _COPY_BUF["src"], _COPY_BUF["dst"]


def bench_copy_pitch(steps, warmup, cols=16320):
    """The default copy on a contiguous 16384 x `cols` fp16 matrix: with 16320
    columns the row pitch is 32 640 bytes instead of the headline's 32 768
    (context for the headline: the same kernel and tiles, another pitch)."""
    import torch

    import async_stage_tile_amd as pt
    import synth
    src = synth.uniform((COPY_M, cols), torch.float16, seed=42, device="cuda")
    dst = torch.empty_like(src)
    fn = pt.copy_launcher(src, dst)
    wall, kern = timed_launches(fn, steps, warmup)
    nbytes = 2 * src.numel() * 2
    ok = torch.equal(dst.view(torch.int16), src.view(torch.int16))
    return {"shape": [COPY_M, cols], "row_pitch_bytes": cols * 2, "kernel_ms": kern,
            "gbs": nbytes / (wall * 1e-3) / 1e9, "kernel_gbs": nbytes / (kern * 1e-3) / 1e9,
            "bit_exact": ok}


def run_for(fn, seconds):
    """Untimed launches of `fn` for about `seconds`, synchronising every 100
    launches; returns the number of launches."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(100):
            fn()
        torch.cuda.synchronize()
        n += 100
    return n


def settle(seconds):
    """Untimed headline copies for about `seconds`, so that clocks and power
    state settle before anything is timed."""
    import async_stage_tile_amd as pt
    src, dst = copy_buffers()
    t0 = time.perf_counter()
    n = run_for(pt.copy_launcher(src, dst), seconds)
    log(f"[bench] settle: {n} untimed copies in {time.perf_counter() - t0:.2f} s")


def device_memory_peak():
    """The HBM peak the device reports, as a cross-check of the 8 TB/s used for
    the roofline: memory bus width and memory clock from hipDeviceGetAttribute
    (attributes 59 and 60 of hipDeviceAttribute_t in ROCm 7's
    hip_runtime_api.h), and the GB/s they give at 2 and at 4 transfers per
    clock (which of the two the reported clock implies depends on the memory
    type)."""
    import ctypes

    import torch

    import async_stage_tile_amd as pt
    # dlsym on the library's handle also searches its dependencies: this is the
    # HIP runtime the library itself runs on (no second runtime is loaded).
    hip = pt.lib()
    dev = torch.cuda.current_device()
    width, clock = ctypes.c_int(0), ctypes.c_int(0)
    if (hip.hipDeviceGetAttribute(ctypes.byref(width), 59, dev) != 0 or
            hip.hipDeviceGetAttribute(ctypes.byref(clock), 60, dev) != 0):
        return None
    per_clock = width.value / 8 * clock.value * 1e3 / 1e9   # GB/s at one transfer per clock
    return {"bus_width_bits": width.value, "memory_clock_khz": clock.value,
            "gbs_at_2_per_clock": round(2 * per_clock, 1),
            "gbs_at_4_per_clock": round(4 * per_clock, 1)}


def kernel_resources(op, M, N, K, launch_grid, launch_threads, **cfg):
    """Compiled resources of the main kernel an op launches (HIP runtime
    attributes) and how many of its workgroups and waves one CU holds at once:
    the least of what the grid gives each of the 256 CUs, what 160 KiB of LDS
    holds, and what 512 VGPRs per SIMD lane allow (4 SIMDs per CU, at most 8
    waves each)."""
    import async_stage_tile_amd as pt
    res = pt.pipe_kernel_resources(op, M, N, K, **cfg)
    waves_per_wg = launch_threads // 64
    per_simd = min(8, 512 // max(1, res["vgprs"]))
    resident = min(-(-launch_grid // 256), 163840 // max(1, res["lds_bytes"]),
                   (4 * per_simd) // waves_per_wg)
    res["threads"] = launch_threads
    res["resident_workgroups_per_cu"] = resident
    res["resident_waves_per_cu"] = resident * waves_per_wg
    return res


def bench_copy(stages, steps, warmup, stats=False, **cfg):
    """The library's default copy configuration, with `stages` and any overrides."""
    import torch

    import async_stage_tile_amd as pt
    src, dst = copy_buffers()
    dst.zero_()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kw = dict(cfg, stages=stages)
    fn = pt.copy_launcher(src, dst, status=st, **kw)
    wall, kern = timed_launches(fn, steps, warmup)
    timing = hot_cold(fn, 2 * COPY_M * COPY_N * 2, max(steps, 20), 2) if stats else None
    ok = int(st.item()) == 0 and torch.equal(dst.view(torch.int16), src.view(torch.int16))
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, COPY_M, COPY_N, **kw)
    c = pt.make_config(pt.PIPE_OP_COPY, **kw)
    nbytes = 2 * COPY_M * COPY_N * 2
    return {"tile": f"{c.tile_m}x{c.tile_n}", "stages": stages,
            "producer_waves": c.producer_waves,
            "consumer_waves": c.consumer_waves, "flags": c.flags, "split": q["split"],
            "grid": q["grid"], "lds_bytes": q["lds_bytes"], "wall_ms": wall, "kernel_ms": kern,
            "bytes": nbytes, "gbs": nbytes / (wall * 1e-3) / 1e9,
            "kernel_gbs": nbytes / (kern * 1e-3) / 1e9, "bit_exact": ok,
            "resources": kernel_resources(pt.PIPE_OP_COPY, COPY_M, COPY_N, 0, q["grid"],
                                          q["threads"], **kw),
            **({"per_launch": timing} if timing else {})}


_ROWSUM_BUF = {}


SAMPLE_ROWS = 64


def _sample_rows(n, seed):
    import numpy as np
    return np.sort(np.random.default_rng(seed).choice(n, SAMPLE_ROWS, replace=False))


def _within(got, ref, rel):
    """max |got - ref| / max(|ref|, rms(ref)) over the sample, and whether it is
    within `rel` (the tolerance the parity tests use)."""
    import torch
    scale = torch.maximum(ref.abs(), ref.pow(2).mean().sqrt())
    err = float(((got - ref).abs() / scale).max())
    return err, bool(err <= rel)


def rowsum_check(A, out, st):
    """After the timed launches: the status word is clear, and 64 sampled rows
    match a float64 torch sum of the same rows within 1e-3 (a plain reduction
    on the host, independent of the kernels)."""
    import torch
    torch.cuda.synchronize()
    status = int(st.item())
    rows = torch.as_tensor(_sample_rows(A.shape[0], 5))
    ref = A[rows.to(A.device)].cpu().double().sum(dim=1)
    err, ok = _within(out[rows.to(out.device)].cpu().double(), ref, 1e-3)
    return {"status": status, "sample_max_rel_err": err, "ok": ok and status == 0}


def gemm_check(A, B, C, st):
    """After the timed launches: the status word is clear, and 64 sampled rows
    of C match a float64 torch product of the same rows within 1e-2."""
    import torch
    torch.cuda.synchronize()
    status = int(st.item())
    rows = torch.as_tensor(_sample_rows(A.shape[0], 9)).to(A.device)
    ref = A[rows].cpu().double() @ B.cpu().double()
    err, ok = _within(C[rows].cpu().double(), ref, 1e-2)
    return {"status": status, "sample_max_rel_err": err, "ok": ok and status == 0}


def bench_rowsum(steps, warmup, stages=None, stats=False, settle_s=0.3, **cfg):
    """The library's default row-sum configuration, with any overrides.
    `settle_s` seconds of untimed launches come first: after the copies, the
    first row-sum launches run several percent slow (measured: 5.8-6.0 TB/s for
    the first 60 launches, 6.6 from then on, wherever the input is placed)."""
    import torch

    import async_stage_tile_amd as pt
    import synth
    if not _ROWSUM_BUF:
        _ROWSUM_BUF["A"] = synth.normal((ROWSUM_M, ROWSUM_N), torch.float16, seed=42,
                                        device="cuda")
    A = _ROWSUM_BUF["A"]
    kw = dict(cfg)
    if stages is not None:
        kw["stages"] = stages
    out = torch.full((ROWSUM_M,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, pt.pipe_rowsum_workspace_bytes(ROWSUM_M, ROWSUM_N, **kw)),
                     dtype=torch.uint8, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fn = pt.rowsum_launcher(A, out, ws, status=st, **kw)
    if settle_s > 0:
        run_for(fn, settle_s)
    wall, kern = timed_launches(fn, steps, warmup)
    nbytes = ROWSUM_M * ROWSUM_N * 2 + ROWSUM_M * 4
    timing = hot_cold(fn, nbytes, max(steps, 20), 2) if stats else None
    check = rowsum_check(A, out, st)
    q = pt.pipe_query_kernel(pt.PIPE_OP_ROWSUM, ROWSUM_M, ROWSUM_N, **kw)
    c = pt.make_config(pt.PIPE_OP_ROWSUM, **kw)
    r = {"tile": f"{c.tile_m}x{c.tile_n}", "stages": c.stages, "producer_waves": c.producer_waves,
         "consumer_waves": c.consumer_waves, "flags": c.flags, "split": q["split"],
         "grid": q["grid"], "wall_ms": wall, "kernel_ms": kern, "bytes": nbytes,
         "gbs": nbytes / (wall * 1e-3) / 1e9, "kernel_gbs": nbytes / (kern * 1e-3) / 1e9,
         "resources": kernel_resources(pt.PIPE_OP_ROWSUM, ROWSUM_M, ROWSUM_N, 0, q["grid"],
                                       q["threads"], **kw),
         **check}
    if timing:
        r["per_launch"] = timing
    return r


def bench_gemm(steps, warmup, stages=None, out_dtype=None, settle_s=0.3, b_colmajor=False,
               **cfg):
    """The library's default GEMM configuration (at `stages`, if given); C in
    fp32, or bf16 through the staged epilogue. `settle_s` seconds of untimed
    launches come first: the matrix cores' clock settles apart from the
    streaming kernels'."""
    import torch

    import async_stage_tile_amd as pt
    import synth
    n = GEMM_N
    A = synth.uniform((n, n), torch.bfloat16, seed=42, stream=0, device="cuda")
    B = synth.uniform((n, n), torch.bfloat16, seed=42, stream=1, device="cuda")
    if b_colmajor:  # the same values, stored column-major (B[k][n] at n * K + k)
        B = B.t().contiguous().t()
    C = torch.full((n, n), float("nan"), dtype=out_dtype or torch.float32, device="cuda")
    kw = dict(cfg)
    if stages is not None:
        kw["stages"] = stages
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fn = pt.gemm_launcher(A, B, C, status=st, **kw)
    if settle_s > 0:
        run_for(fn, settle_s)
    wall, kern = timed_launches(fn, steps, warmup)
    med, mn = launch_stats(fn, max(steps, 20), 0)
    check = gemm_check(A, B, C, st)
    flops = 2.0 * n * n * n
    c = pt._gemm_config(C, kw, b_colmajor)
    gcfg = {f: getattr(c, f) for f in ("stages", "producer_waves", "consumer_waves", "tile_m",
                                       "tile_n", "tile_k", "flags", "swizzle_shift", "grid")}
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, n, n, n, **gcfg)
    return {"c_dtype": str(C.dtype).replace("torch.", ""),
            "b_layout": "column-major" if b_colmajor else "row-major", "stages": c.stages,
            "tile": [c.tile_m, c.tile_n, c.tile_k],
            "producer_waves": 0 if c.flags & pt.PIPE_FLAG_UNIFIED else c.producer_waves,
            "flags": c.flags, "wall_ms": wall, "kernel_ms": kern, "flops": flops,
            "tflops": flops / (wall * 1e-3) / 1e12,
            "mfma_frac": flops / (wall * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "per_launch": {"median_ms": med, "min_ms": mn,
                           "median_tflops": flops / (med * 1e-3) / 1e12},
            "resources": kernel_resources(pt.PIPE_OP_GEMM, n, n, n, q["grid"], q["threads"],
                                          **gcfg),
            **check}


def bench_small(reps, warmup):
    """The two small functional workloads, timed per launch (they are too small
    to load HBM, so latency is what they show): a 256 x 128 index-coded matrix
    in 2 x 2 tiles of 128 x 64 through a one-slot ring, and a 128 x 512 matrix
    through a three-slot ring of one workgroup (1 producer + 3 consumer waves)
    with per-tile checksums. Each is checked bit for bit; the checksums against
    a plain tensor sum of each tile's 16-bit codes. `graph_us` is the time per
    launch when 100 launches are captured in one HIP graph and replayed, which
    leaves out the host's per-launch cost."""
    import torch

    import async_stage_tile_amd as pt
    import synth

    def graph_us(make):
        """Per-launch time of 100 launches of make()'s launcher replayed from one
        graph (the launcher is made inside the capture, so it binds the
        capture stream)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            fn = make()
            for _ in range(100):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return round(a.elapsed_time(b) / 1000.0 * 1e3, 2)   # ms per 1000 launches -> us

    out = {}
    src = synth.index_coded(256, 128, device="cuda")
    dst = torch.empty_like(src)
    fn = pt.copy_launcher(src, dst, stages=1)
    med, mn = launch_stats(fn, reps, warmup)
    dst.zero_()
    g_us = graph_us(lambda: pt.copy_launcher(src, dst, stages=1))
    out["copy_256x128_s1"] = {"median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2),
                              "graph_us": g_us,
                              "bit_exact": torch.equal(dst.view(torch.int16),
                                                       src.view(torch.int16))}
    src = synth.uniform((128, 512), torch.float16, seed=42, device="cuda")
    dst = torch.empty_like(src)
    chk = torch.empty(8, dtype=torch.int32, device="cuda")
    fn = pt.copy_launcher(src, dst, checksums=chk, stages=3, producer_waves=1, consumer_waves=3,
                          grid=1, flags=0)
    med, mn = launch_stats(fn, reps, warmup)
    dst.zero_()
    chk.zero_()
    g_us = graph_us(lambda: pt.copy_launcher(src, dst, checksums=chk, stages=3,
                                             producer_waves=1, consumer_waves=3, grid=1,
                                             flags=0))
    codes = src.view(torch.int16).to(torch.int64) & 0xFFFF
    want = codes.view(128, 8, 64).sum(dim=(0, 2))
    out["copy_128x512_s3_1p3c"] = {
        "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2), "graph_us": g_us,
        "bit_exact": torch.equal(dst.view(torch.int16), src.view(torch.int16)),
        "checksums_exact": torch.equal(chk.to(torch.int64) & 0xFFFFFFFF, want)}
    return out


def bench_ceilings(steps, warmup):
    """Context ceilings on this device for the copy's traffic (512 MiB each way)
    and for a 1 GiB read: no LDS ring, no tiles."""
    import torch

    import ceilings as ceiling
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(3)
    out = {}
    cases = {
        "hipMemcpyDtoD": lambda: ceiling.memcpy(src, dst),
        "torch_copy": lambda: dst.copy_(src),
    }
    for grid in (2048, 4096, 8192):
        cases[f"stream_copy_nt_x4_grid{grid}"] = (
            lambda g=grid: ceiling.copy(src, dst, g, unroll=4, nt=1))
    for name, fn in cases.items():
        _, kern = timed_launches(fn, steps, warmup)
        out[name] = 2 * n / (kern * 1e-3) / 1e9
    assert torch.equal(src, dst)
    del dst
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(5)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for grid in (1024, 2048, 4096):
        _, kern = timed_launches(lambda g=grid: ceiling.read(big, sink, g, nt=1), steps, warmup)
        out[f"stream_read_nt_grid{grid}"] = big.numel() / (kern * 1e-3) / 1e9
    best_copy = max(v for k, v in out.items() if "read" not in k)
    best_read = max(v for k, v in out.items() if "read" in k)
    del big
    torch.cuda.empty_cache()
    return {"gbs": out, "best_copy_gbs": best_copy, "best_read_gbs": best_read,
            "column_strips": strip_ceilings(steps, warmup), "lds": lds_ceilings(steps, warmup)}


def lds_ceilings(steps, warmup, grid=512):
    """LDS traffic of one instruction kind at full rate (two 512-thread
    workgroups per CU): the fragment reads and the DMA writes that the GEMM
    mainloop is made of, alone and side by side. Bytes per clock per CU use the
    shader clock that the kernel itself measured; for the side-by-side run each
    half is timed over its own loop (waves 0 and 4 record their cycles)."""
    import torch

    import ceilings as ceiling
    src = torch.zeros(65536 + 1024, dtype=torch.uint8, device="cuda")
    fold = torch.zeros(grid * 512, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(4 * grid, dtype=torch.int64, device="cuda")
    out = {}
    for op, (name, per_instr, waves) in ceiling.LDS_OPS.items():
        iters = 500 if op in (2, 4, 6) else 2000
        _, kern = timed_launches(lambda: ceiling.lds(op, src, fold, clocks, grid, iters), steps,
                                 warmup)
        c = clocks.view(grid, 4).double()
        col = 2 if op == 5 else 0
        ghz = (c[:, col].sum() / (c[:, col + 1].sum() / 100e6)).item() / 1e9
        clk = kern * 1e-3 * ghz * 1e9  # kernel duration in shader clocks
        if op == 4:
            half = grid * 4 * iters * 8 * per_instr
            span = [c[:, k].mean().item() for k in (0, 2)]
            frac = [x / max(span) for x in span]  # share of the kernel each half was busy
            out[name] = {"clock_ghz": round(ghz, 3),
                         "dma_bytes_per_clk_per_cu": round(half / 256 / (clk * frac[0]), 1),
                         "read_bytes_per_clk_per_cu": round(half / 256 / (clk * frac[1]), 1)}
            continue
        nbytes = ceiling.lds_bytes(op, grid, iters)
        out[name] = {"tbs": round(nbytes / (kern * 1e-3) / 1e12, 2), "clock_ghz": round(ghz, 3),
                     "bytes_per_clk_per_cu": round(nbytes / 256 / clk, 1)}
    return out


def strip_ceilings(steps, warmup):
    """Plain kernels (no LDS ring) with the tile stream's access pattern on the
    headline matrix: column strips 128 bytes wide (that of 128 x 64 fp16 tiles)
    and 512 bytes wide (that of 32 x 256 tiles), read only, write only and copy.
    `serial_rw_gbs` is the copy rate if its reads and writes took turns at the
    read-only and write-only rates: 2 / (1 / read + 1 / write)."""
    import torch

    import ceilings as ceiling
    src, dst = copy_buffers()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    nbytes = src.numel() * src.element_size()
    out = {}
    for strip_bytes, split in ((128, 1), (512, 4)):
        r = {}
        _, kern = timed_launches(lambda: ceiling.strip_read(src, sink, strip_bytes, split),
                                 steps, warmup)
        r["read_gbs"] = nbytes / (kern * 1e-3) / 1e9
        _, kern = timed_launches(lambda: ceiling.strip_write(dst, strip_bytes, split), steps,
                                 warmup)
        r["write_gbs"] = nbytes / (kern * 1e-3) / 1e9
        _, kern = timed_launches(lambda: ceiling.strip_copy(src, dst, strip_bytes, split), steps,
                                 warmup)
        r["copy_gbs"] = 2 * nbytes / (kern * 1e-3) / 1e9
        assert torch.equal(src, dst)
        r["serial_rw_gbs"] = 2.0 / (1.0 / r["read_gbs"] + 1.0 / r["write_gbs"])
        r["grid"] = src.shape[1] * src.element_size() // strip_bytes * split
        out[f"{strip_bytes}B"] = {k: (round(v, 1) if isinstance(v, float) else v)
                                  for k, v in r.items()}
    return out


def cpu_baseline(rows, min_seconds=10.0):
    """The oracle's tile copy on the first `rows` x 16384 of the same matrix, on
    one host thread, repeated until `min_seconds` of CPU work have elapsed."""
    import numpy as np
    import torch

    import synth
    from oracle import results as R
    src = synth.uniform((rows, COPY_N), torch.float16, seed=42).numpy()
    reps, dt = 0, 0.0
    while dt < min_seconds:
        t0 = time.perf_counter()
        out = R.tile_copy(src)
        dt += time.perf_counter() - t0
        reps += 1
    assert np.array_equal(out.view(np.uint16), src.view(np.uint16))
    nbytes = 2 * rows * COPY_N * 2 * reps
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"tile copy of the first {rows} of {COPY_M} rows (x {COPY_N} fp16), "
                      f"{reps} passes, {nbytes} bytes read+write in {dt:.2f} s"}


def _threads():
    return max(1, min(os.cpu_count() or 1, 16))


def _parallel_rows(fn, rows, nthreads):
    """Run fn(r0, r1) over row blocks on nthreads threads (numpy releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    step = (rows + nthreads - 1) // nthreads
    with ThreadPoolExecutor(max_workers=nthreads) as ex:
        list(ex.map(lambda r0: fn(r0, min(rows, r0 + step)), range(0, rows, step)))


def cpu_oracle_extras(copy_rows, rowsum_rows, gemm_rows):
    """The CPU oracle on bounded samples, on one thread and on all host threads.

    copy: oracle.results.tile_copy on copy_rows x 16384; rowsum:
    oracle.results.rowsum_exact on rowsum_rows x 65536; GEMM: oracle.results.gemm_f64
    on gemm_rows rows of A (4096^2 bf16 inputs) against all of B. The copy oracle
    is a per-tile Python loop that holds the interpreter lock, so more threads
    cannot speed it up: it is timed on one thread only. The row sum and the GEMM
    spend their time in numpy and BLAS, which release the lock."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import results as R
    nt = _threads()
    res = {"threads_all": nt}
    src = synth.uniform((copy_rows, COPY_N), torch.float16, seed=42).numpy()
    A = synth.normal((rowsum_rows, ROWSUM_N), torch.float16, seed=42).numpy()
    Ga = synth.uniform((gemm_rows, GEMM_N), torch.bfloat16, seed=42, stream=0).float().numpy()
    Gb = synth.uniform((GEMM_N, GEMM_N), torch.bfloat16, seed=42, stream=1).float().numpy()
    for label, threads in (("1_thread", 1), ("all_threads", nt)):
        with threadpool_limits(limits=threads):
            tc = None
            if threads == 1:
                t0 = time.perf_counter()
                R.tile_copy(src)
                tc = time.perf_counter() - t0
            t0 = time.perf_counter()
            _parallel_rows(lambda a, b: R.rowsum_exact(A[a:b]), rowsum_rows, threads)
            tr = time.perf_counter() - t0
            t0 = time.perf_counter()
            R.gemm_f64(Ga, Gb)
            tg = time.perf_counter() - t0
        res[label] = {"copy_gbs": 4 * copy_rows * COPY_N / tc / 1e9 if tc else None,
                      "rowsum_gbs": 2 * rowsum_rows * ROWSUM_N / tr / 1e9,
                      "gemm_gflops": 2.0 * gemm_rows * GEMM_N * GEMM_N / tg / 1e9}
    res["sample"] = (f"copy {copy_rows}x{COPY_N} fp16, rowsum {rowsum_rows}x{ROWSUM_N} fp16, "
                     f"gemm {gemm_rows}x{GEMM_N} @ {GEMM_N}x{GEMM_N} bf16 in fp64")
    return res


def correctness_flags(obj):
    """Every "ok", "bit_exact" and "checksums_exact" value in a record tree."""
    if isinstance(obj, dict):
        for k, v in obj.items():
            if k in ("ok", "bit_exact", "checksums_exact"):
                yield bool(v)
            else:
                yield from correctness_flags(v)
    elif isinstance(obj, list):
        for v in obj:
            yield from correctness_flags(v)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed headline copies before any measurement, so that "
                         "the device reaches steady clocks (0 = none)")
    ap.add_argument("--stages", type=int, default=None,
                    help="ring depth (default: the library default of the workload, 2 for "
                         "the copy -- the best of the S sweeps measured on MI355X); 0 = the "
                         "best of this run's 1..4 copy sweep")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline sample")
    ap.add_argument("--only", choices=["copy", "copy_32x256", "copy_64x128", "copy_grouped",
                                       "copy_group_loads",
                                       "copy_regs", "copy_pitch", "rowsum", "rowsum_regs",
                                       "rowsum_32x256", "rowsum_64x128", "gemm", "gemm_bf16",
                                       "gemm_bcol", "gemm_tile256", "gemm_unified", "gemm_wide", "gemm_deep",
                                       "ceiling", "calib"],
                    default=None,
                    help="time one workload only (for profiling); prints no JSON line")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the tile stream has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm device", file=sys.stderr)
        sys.exit(1)

    if args.only == "calib":
        # Known-size reference for the traffic counters: torch's device copy of
        # 512 MiB (512 MiB read + 512 MiB written per launch).
        x = torch.empty(256 << 20, dtype=torch.float16, device="cuda")
        y = torch.empty_like(x)
        x.fill_(1.0)
        wall, kern = timed_launches(lambda: y.copy_(x), args.steps, args.warmup)
        log(f"[bench] calib copy of {x.numel() * 2} bytes: {kern:.4f} ms")
        return
    if args.only == "copy":
        r = bench_copy(args.stages or 2, args.steps, args.warmup)
        log(f"[bench] copy: {r}")
        return
    if args.only in ("copy_32x256", "copy_64x128"):
        cfg = dict(WIDE_COPY[args.only.split("_")[1]])
        r = bench_copy(cfg.pop("stages"), args.steps, args.warmup, **cfg)
        log(f"[bench] {args.only}: {r}")
        return
    if args.only == "copy_grouped":
        cfg = dict(GROUPED_COPY)
        r = bench_copy(cfg.pop("stages"), args.steps, args.warmup, **cfg)
        log(f"[bench] copy_grouped: {r}")
        return
    if args.only == "copy_group_loads":
        cfg = dict(GROUP_LOAD_COPY)
        r = bench_copy(cfg.pop("stages"), args.steps, args.warmup, **cfg)
        log(f"[bench] copy_group_loads: {r}")
        return
    if args.only == "copy_pitch":
        r = bench_copy_pitch(args.steps, args.warmup)
        log(f"[bench] copy_pitch: {r}")
        return
    if args.only == "copy_regs":
        cfg = dict(REGS_COPY)
        r = bench_copy(cfg.pop("stages"), args.steps, args.warmup, **cfg)
        log(f"[bench] copy_regs: {r}")
        return
    if args.only == "rowsum_regs":
        r = bench_rowsum(args.steps, args.warmup, **REGS_ROWSUM)
        log(f"[bench] rowsum_regs: {r}")
        return
    if args.only in ("rowsum_32x256", "rowsum_64x128"):
        r = bench_rowsum(args.steps, args.warmup, **WIDE_ROWSUM[args.only.split("_")[1]])
        log(f"[bench] {args.only}: {r}")
        return
    if args.only == "rowsum":
        r = bench_rowsum(args.steps, args.warmup, args.stages)
        log(f"[bench] rowsum: {r}")
        return
    if args.only == "gemm":
        r = bench_gemm(args.steps, args.warmup, args.stages)
        log(f"[bench] gemm: {r}")
        return
    if args.only == "gemm_tile256":
        r = bench_gemm(args.steps, args.warmup, args.stages or 3, tile_m=256, consumer_waves=8,
                       producer_waves=4)
        log(f"[bench] gemm, 256 x 128 tiles: {r}")
        return
    if args.only == "gemm_unified":
        r = bench_gemm(args.steps, args.warmup, 2, **UNIFIED_GEMM)
        log(f"[bench] gemm, unified 256 x 256 tiles: {r}")
        return
    if args.only == "gemm_wide":
        r = bench_gemm(args.steps, args.warmup, 2, **WIDE_GEMM)
        log(f"[bench] gemm, unified 256 x 256 tiles, 4 waves: {r}")
        return
    if args.only == "gemm_deep":
        r = bench_gemm(args.steps, args.warmup, args.stages or 4, **DEEP_GEMM)
        log(f"[bench] gemm, unified 256 x 256 x 32 tiles, 4 waves: {r}")
        return
    if args.only == "gemm_bcol":
        r = bench_gemm(args.steps, args.warmup, args.stages, b_colmajor=True)
        log(f"[bench] gemm, B column-major: {r}")
        return
    if args.only == "gemm_bf16":
        r = bench_gemm(args.steps, args.warmup, args.stages, out_dtype=torch.bfloat16)
        log(f"[bench] gemm, bf16 C: {r}")
        return
    if args.only == "ceiling":
        r = bench_ceilings(args.steps, args.warmup)
        log(f"[bench] ceilings: {r}")
        return

    if args.settle > 0:
        settle(args.settle)
    extras = {}
    stages = 2 if args.stages is None else args.stages
    if not args.no_extras or stages == 0:
        # Two passes in opposite orders, so that no depth gains from running
        # later in the process (clocks still settling); each point is the mean.
        depths = (1, 2, 3, 4, 6, 8)
        runs = {s: [] for s in depths}
        for order in (depths, depths[::-1]):
            for s in order:
                runs[s].append(bench_copy(s, max(3, args.steps // 2), args.warmup))
        sweep = []
        for s in depths:
            a, b = runs[s]
            sweep.append({"stages": s, "lds_bytes": a["lds_bytes"],
                          "kernel_ms": (a["kernel_ms"] + b["kernel_ms"]) / 2,
                          "gbs": (a["gbs"] + b["gbs"]) / 2,
                          "gbs_passes": [a["gbs"], b["gbs"]],
                          "bit_exact": a["bit_exact"] and b["bit_exact"]})
            log(f"[bench] sweep S={s}: {sweep[-1]['gbs']:.1f} GB/s "
                f"(passes {a['gbs']:.1f}, {b['gbs']:.1f})")
        extras["copy_stage_sweep"] = sweep
        if stages == 0:
            stages = max(sweep, key=lambda r: r["gbs"])["stages"]
    log(f"[bench] headline copy S={stages} ...")
    head = bench_copy(stages, args.steps, args.warmup)
    log(f"[bench] copy S={stages}: {head['gbs']:.1f} GB/s (kernel {head['kernel_gbs']:.1f})")
    if not args.no_extras:
        import async_stage_tile_amd as pt
        t = bench_copy(stages, args.steps, args.warmup, stats=True)["per_launch"]
        extras["copy_per_launch"] = t
        log(f"[bench] copy per launch: hot {t['hot']['median_gbs']:.1f}, "
            f"cold {t['cold']['median_gbs']:.1f} GB/s (median)")
        wide = {}
        for name, cfg in WIDE_COPY.items():
            cfg = dict(cfg)
            w = bench_copy(cfg.pop("stages"), args.steps, args.warmup, **cfg)
            wide[name] = {k: w[k] for k in ("tile", "stages", "producer_waves", "consumer_waves",
                                            "flags", "split", "grid", "kernel_ms", "gbs",
                                            "kernel_gbs", "bit_exact")}
            wide[name]["kernel_pct_of_peak"] = round(100.0 * w["kernel_gbs"] / PEAK_HBM_GBS, 2)
            log(f"[bench] copy, {name} tiles: {w['gbs']:.1f} GB/s (kernel {w['kernel_gbs']:.1f})")
        extras["copy_wide_tiles"] = wide
        cfg = dict(GROUPED_COPY)
        w = bench_copy(cfg.pop("stages"), args.steps, args.warmup, **cfg)
        extras["copy_grouped_strips"] = {
            **{k: w[k] for k in ("tile", "stages", "producer_waves", "consumer_waves", "flags",
                                 "split", "grid", "kernel_ms", "gbs", "kernel_gbs", "bit_exact")},
            "strip_tiles": 4,
            "kernel_pct_of_peak": round(100.0 * w["kernel_gbs"] / PEAK_HBM_GBS, 2)}
        log(f"[bench] copy, grouped strips: {w['gbs']:.1f} GB/s (kernel {w['kernel_gbs']:.1f})")
        cfg = dict(GROUP_LOAD_COPY)
        w = bench_copy(cfg.pop("stages"), args.steps, args.warmup, **cfg)
        extras["copy_group_loads"] = {
            **{k: w[k] for k in ("tile", "stages", "producer_waves", "consumer_waves", "flags",
                                 "split", "grid", "kernel_ms", "gbs", "kernel_gbs", "bit_exact")},
            "strip_tiles": 4, "load_shape": "2 rows x 512 B",
            "kernel_pct_of_peak": round(100.0 * w["kernel_gbs"] / PEAK_HBM_GBS, 2)}
        log(f"[bench] copy, grouped loads: {w['gbs']:.1f} GB/s (kernel {w['kernel_gbs']:.1f})")
        w = bench_copy_pitch(args.steps, args.warmup)
        extras["copy_pitch_32640"] = w
        log(f"[bench] copy, 16384 x 16320 (32 640-byte pitch): {w['gbs']:.1f} GB/s")
        cfg = dict(REGS_COPY)
        w = bench_copy(cfg.pop("stages"), args.steps, args.warmup, **cfg)
        extras["copy_register_engine"] = {
            k: w[k] for k in ("tile", "stages", "producer_waves", "consumer_waves", "flags",
                              "split", "grid", "kernel_ms", "gbs", "kernel_gbs", "bit_exact")}
        log(f"[bench] copy, register engine: {w['gbs']:.1f} GB/s")
        # Specialised ring against the unified (non-specialised) pipeline over the
        # same ring depths S = 1..4.
        uflags = pt.PIPE_FLAG_UNIFIED | pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_XCD_REMAP
        keys = ("stages", "consumer_waves", "flags", "lds_bytes", "kernel_ms", "gbs",
                "kernel_gbs", "bit_exact")
        n1 = {"specialised": [{k: r[k] for k in ("stages", "lds_bytes", "kernel_ms", "gbs",
                                                  "bit_exact")}
                              for r in extras.get("copy_stage_sweep", []) if r["stages"] <= 4],
              "unified": []}
        urun = {s_: [] for s_ in (1, 2, 3, 4)}
        for order in ((1, 2, 3, 4), (4, 3, 2, 1)):  # two passes, as for the stage sweep
            for s_ in order:
                urun[s_].append(bench_copy(s_, max(3, args.steps // 2), args.warmup,
                                           consumer_waves=2, flags=uflags))
        for s_, (a, b) in urun.items():
            u = {k: a[k] for k in keys}
            for k in ("kernel_ms", "gbs", "kernel_gbs"):
                u[k] = (a[k] + b[k]) / 2
            u["bit_exact"] = a["bit_exact"] and b["bit_exact"]
            n1["unified"].append(u)
            log(f"[bench] unified copy S={s_}: {u['gbs']:.1f} GB/s (kernel {u['kernel_gbs']:.1f})")
        extras["copy_specialised_vs_unified"] = n1
        _COPY_BUF.clear()
        torch.cuda.empty_cache()
        r = bench_rowsum(max(3, args.steps // 2), args.warmup, stats=True)
        log(f"[bench] rowsum: {r['gbs']:.1f} GB/s")
        extras["rowsum_8192x65536_fp16"] = r
        keys = ("stages", "consumer_waves", "split", "flags", "kernel_ms", "gbs", "kernel_gbs",
                "ok")
        n1 = {"specialised": [], "unified": []}
        for s_ in (1, 2, 3, 4):
            r = bench_rowsum(max(3, args.steps // 2), args.warmup, stages=s_)
            n1["specialised"].append({k: r[k] for k in keys})
            r = bench_rowsum(max(3, args.steps // 2), args.warmup, stages=s_, consumer_waves=2,
                             split=16, flags=uflags)
            n1["unified"].append({k: r[k] for k in keys})
            log(f"[bench] rowsum S={s_}: specialised {n1['specialised'][-1]['kernel_gbs']:.1f}, "
                f"unified {r['kernel_gbs']:.1f} GB/s (kernel)")
        for side in n1.values():
            for r in side:
                r["lds_bytes"] = r["stages"] * 16384 + (0 if r["flags"] & pt.PIPE_FLAG_UNIFIED
                                                        else r["stages"] * 4 * 7)
        extras["rowsum_specialised_vs_unified"] = n1
        r = bench_rowsum(max(3, args.steps // 2), args.warmup, **REGS_ROWSUM)
        log(f"[bench] rowsum, register engine: {r['gbs']:.1f} GB/s")
        extras["rowsum_register_engine"] = r
        wide = {}
        for name, cfg in WIDE_ROWSUM.items():
            w = bench_rowsum(max(3, args.steps // 2), args.warmup, **cfg)
            w["kernel_pct_of_peak"] = round(100.0 * w["kernel_gbs"] / PEAK_HBM_GBS, 2)
            wide[name] = w
            log(f"[bench] rowsum, {name}: {w['gbs']:.1f} GB/s (kernel {w['kernel_gbs']:.1f})")
        extras["rowsum_wide_tiles"] = wide
        _ROWSUM_BUF.clear()
        torch.cuda.empty_cache()
        # The GEMM workload as stated: 128 x 128 x 64 tiles through a three-stage
        # ring; the library default (two stages, two workgroups per CU) beside it.
        g = bench_gemm(max(3, args.steps // 2), args.warmup, stages=3)
        log(f"[bench] gemm, three-stage ring: {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, stages=2)
        log(f"[bench] gemm, two-stage ring (library default): {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_two_stage"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, stages=3, tile_m=256,
                       consumer_waves=8, producer_waves=4)
        log(f"[bench] gemm, 256 x 128 tiles, three-stage ring: {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_tile_256x128"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, stages=2, **UNIFIED_GEMM)
        log(f"[bench] gemm, unified 256 x 256 tiles (16 waves load and compute): "
            f"{g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_unified_256x256"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, stages=2, **WIDE_GEMM)
        log(f"[bench] gemm, unified 256 x 256 tiles, 4 waves: {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_unified_256x256_4_waves"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, stages=4, **DEEP_GEMM)
        log(f"[bench] gemm, unified 256 x 256 x 32 tiles, 4 waves, S = 4: {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_unified_256x256x32_4_waves_s4"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, stages=4, out_dtype=torch.bfloat16,
                       **DEEP_GEMM)
        log(f"[bench] gemm, unified 256 x 256 x 32 tiles, 4 waves, S = 4, bf16 C: "
            f"{g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_unified_256x256x32_4_waves_s4_c_bf16"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, out_dtype=torch.bfloat16)
        log(f"[bench] gemm, bf16 C: {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_c_bf16"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, out_dtype=torch.bfloat16,
                       flags=pt.PIPE_FLAG_EAGER_NEWEST | pt.PIPE_FLAG_GEMM_STORE_WAVE)
        log(f"[bench] gemm, bf16 C via a store wave: {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_c_bf16_store_wave"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, b_colmajor=True)
        log(f"[bench] gemm, B column-major: {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_b_colmajor"] = g
        g = bench_gemm(max(3, args.steps // 2), args.warmup, b_colmajor=True,
                       out_dtype=torch.bfloat16)
        log(f"[bench] gemm, B column-major, bf16 C: {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16_b_colmajor_c_bf16"] = g
        torch.cuda.empty_cache()
        sm = bench_small(max(20, args.steps), args.warmup)
        log(f"[bench] small configs: {sm}")
        extras["small_configs"] = sm
        c = bench_ceilings(max(3, args.steps // 2), args.warmup)
        log(f"[bench] ceilings: copy {c['best_copy_gbs']:.1f}, read {c['best_read_gbs']:.1f} GB/s")
        c["copy_frac_of_best_copy_ceiling"] = head["kernel_gbs"] / c["best_copy_gbs"]
        s128 = c["column_strips"]["128B"]
        log(f"[bench] 128-byte column strips, plain: read {s128['read_gbs']}, write "
            f"{s128['write_gbs']}, copy {s128['copy_gbs']}, serial read+write "
            f"{s128['serial_rw_gbs']} GB/s")
        c["copy_frac_of_strip128_copy"] = head["kernel_gbs"] / s128["copy_gbs"]
        c["copy_frac_of_strip128_serial_rw"] = head["kernel_gbs"] / s128["serial_rw_gbs"]
        extras["context_ceilings"] = c
        extras["device_memory"] = device_memory_peak()
        log(f"[bench] device memory: {extras['device_memory']}")
    cpu = None
    if not args.no_cpu:
        log("[bench] cpu baseline ...")
        cpu = cpu_baseline(args.cpu_rows, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']:.2f} GB/s")
        if not args.no_extras:
            extras["cpu_oracle"] = cpu_oracle_extras(2048, 256, 64)
            log(f"[bench] cpu oracle extras: {extras['cpu_oracle']}")

    # Every timed record that carries a correctness check passed it.
    checks = [head["bit_exact"]] + list(correctness_flags(extras))
    achieved = head["bytes"] / (head["kernel_ms"] * 1e-3) / 1e9
    kname = (f"void pipe::stream_kernel<{head['stages']}, {head['consumer_waves']}, "
             f"{head['producer_waves']}, 0, false, 64>(pipe::StreamParams)")
    traffic = recorded_traffic(kname)
    line = {
        "metric": METRIC,
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "tile copy fp16 16384x16384 uniform[-1,1) seed 42, 128x64 tiles, "
                               "persistent column strips",
                   "stages": head["stages"], "producer_waves": head["producer_waves"],
                   "consumer_waves": head["consumer_waves"], "flags": head["flags"],
                   "split": head["split"], "grid": head["grid"], "parallelism": "1 GPU"},
        "pct_of_peak": round(100.0 * head["gbs"] / PEAK_HBM_GBS, 2),
        "bit_exact": head["bit_exact"],
        "ok": all(bool(c) for c in checks),
        "resources": head["resources"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": kname},
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)
    if not head["bit_exact"]:
        sys.exit("the headline copy was not bit-exact (or its status word was set)")


if __name__ == "__main__":
    main()
