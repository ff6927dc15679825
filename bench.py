"""Benchmark of the pipelined tile stream on one MI355X.

Headline (the JSON line's `value`): achieved HBM bandwidth (read + write) of
the streaming tile copy, fp16 16384 x 16384 (1 GiB moved per step), 128 x 64
tiles through an S-slot LDS ring, persistent workgroups each streaming one
column strip. One step = one launch of the whole hot path over the matrix
(tile walk, cursor/barrier handshakes, direct-to-LDS producer, consumer
copy-out, release, tail).

Also reported (in "extras", each timed the same way): the S = 1..4 sweep of
the copy, the row sum of fp16 8192 x 65536 (GB/s) and the GEMM mainloop
4096^3 bf16 (TFLOP/s), each at the library's default configuration.

roofline.traffic: HBM bytes per launch of the headline kernel from rocprofv3
FETCH_SIZE / WRITE_SIZE counters (scaled by the counts the same counters give
for a known-size device copy), read from the committed counter summary under
profiles/ -- reported only while the kernel sources are unchanged since.

Timing: `warmup` untimed steps, then exactly `steps` steps between
synchronisations; per-launch kernel time from HIP events recorded on the
launch stream. Inputs are generated on the device before the timed region.

cpu_baseline: the CPU oracle (oracle.results.tile_copy) timed on a bounded
sample of the same matrix on the host, single-threaded numpy.
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
KERNEL_SOURCES = ("pipe_device.hpp", "pipe_kernels.hpp", "pipe_stream.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    """sha256 (first 16 hex digits) of the device sources of the stream kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "async_stage_tile_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
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


_COPY_BUF = {}


def copy_buffers():
    import torch

    import synth
    if not _COPY_BUF:
        src = synth.uniform((COPY_M, COPY_N), torch.float16, seed=42, device="cuda")
        _COPY_BUF["src"] = src
        _COPY_BUF["dst"] = torch.empty_like(src)
    return _COPY_BUF["src"], _COPY_BUF["dst"]


def bench_copy(stages, steps, warmup, **cfg):
    """The library's default copy configuration, with `stages` and any overrides."""
    import torch

    import async_stage_tile_amd as pt
    src, dst = copy_buffers()
    dst.zero_()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kw = dict(cfg, stages=stages)
    fn = pt.copy_launcher(src, dst, status=st, **kw)
    wall, kern = timed_launches(fn, steps, warmup)
    ok = int(st.item()) == 0 and torch.equal(dst.view(torch.int16), src.view(torch.int16))
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, COPY_M, COPY_N, **kw)
    c = pt.make_config(pt.PIPE_OP_COPY, **kw)
    nbytes = 2 * COPY_M * COPY_N * 2
    return {"stages": stages, "producer_waves": c.producer_waves,
            "consumer_waves": c.consumer_waves, "flags": c.flags, "split": q["split"],
            "grid": q["grid"], "lds_bytes": q["lds_bytes"], "wall_ms": wall, "kernel_ms": kern,
            "bytes": nbytes, "gbs": nbytes / (wall * 1e-3) / 1e9,
            "kernel_gbs": nbytes / (kern * 1e-3) / 1e9, "bit_exact": ok}


def bench_rowsum(steps, warmup, stages=3):
    """The library's default row-sum configuration at `stages`."""
    import torch

    import async_stage_tile_amd as pt
    import synth
    A = synth.normal((ROWSUM_M, ROWSUM_N), torch.float16, seed=42, device="cuda")
    out = torch.empty(ROWSUM_M, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, pt.pipe_rowsum_workspace_bytes(ROWSUM_M, ROWSUM_N, stages=stages)),
                     dtype=torch.uint8, device="cuda")
    fn = pt.rowsum_launcher(A, out, ws, stages=stages)
    wall, kern = timed_launches(fn, steps, warmup)
    nbytes = ROWSUM_M * ROWSUM_N * 2 + ROWSUM_M * 4
    q = pt.pipe_query_kernel(pt.PIPE_OP_ROWSUM, ROWSUM_M, ROWSUM_N, stages=stages)
    del A
    return {"stages": stages, "split": q["split"], "grid": q["grid"], "wall_ms": wall,
            "kernel_ms": kern, "bytes": nbytes, "gbs": nbytes / (wall * 1e-3) / 1e9}


def bench_gemm(steps, warmup, stages=3):
    """The library's default GEMM configuration at `stages`."""
    import torch

    import async_stage_tile_amd as pt
    import synth
    n = GEMM_N
    A = synth.uniform((n, n), torch.bfloat16, seed=42, stream=0, device="cuda")
    B = synth.uniform((n, n), torch.bfloat16, seed=42, stream=1, device="cuda")
    C = torch.empty((n, n), dtype=torch.float32, device="cuda")
    fn = pt.gemm_launcher(A, B, C, stages=stages)
    wall, kern = timed_launches(fn, steps, warmup)
    flops = 2.0 * n * n * n
    return {"stages": stages, "wall_ms": wall, "kernel_ms": kern, "flops": flops,
            "tflops": flops / (wall * 1e-3) / 1e12,
            "mfma_frac": flops / (wall * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def cpu_baseline(rows):
    """The oracle's tile copy on `rows` x 16384 of the same matrix, on the host."""
    import numpy as np
    import torch

    import synth
    from oracle import results as R
    src = synth.uniform((rows, COPY_N), torch.float16, seed=42).numpy()
    t0 = time.perf_counter()
    out = R.tile_copy(src)
    dt = time.perf_counter() - t0
    assert np.array_equal(out.view(np.uint16), src.view(np.uint16))
    nbytes = 2 * rows * COPY_N * 2
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"tile copy of the first {rows} of {COPY_M} rows (x {COPY_N} fp16), "
                      f"{nbytes} bytes read+write, {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--stages", type=int, default=None,
                    help="ring depth (default: the library default of the workload, 2 for "
                         "the copy -- the best of the S sweeps measured on MI355X); 0 = the "
                         "best of this run's 1..4 copy sweep")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--only", choices=["copy", "rowsum", "gemm", "calib"], default=None,
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
    if args.only == "rowsum":
        r = bench_rowsum(args.steps, args.warmup, args.stages or 4)
        log(f"[bench] rowsum: {r}")
        return
    if args.only == "gemm":
        r = bench_gemm(args.steps, args.warmup, args.stages or 4)
        log(f"[bench] gemm: {r}")
        return

    extras = {}
    stages = 2 if args.stages is None else args.stages
    if not args.no_extras or stages == 0:
        sweep = []
        for s in (1, 2, 3, 4):
            r = bench_copy(s, max(3, args.steps // 2), 2)
            log(f"[bench] sweep S={s}: {r['gbs']:.1f} GB/s")
            sweep.append({k: r[k] for k in ("stages", "kernel_ms", "gbs", "bit_exact",
                                            "lds_bytes")})
        extras["copy_stage_sweep"] = sweep
        if stages == 0:
            stages = max(sweep, key=lambda r: r["gbs"])["stages"]
    log(f"[bench] headline copy S={stages} ...")
    head = bench_copy(stages, args.steps, args.warmup)
    log(f"[bench] copy S={stages}: {head['gbs']:.1f} GB/s (kernel {head['kernel_gbs']:.1f})")
    if not args.no_extras:
        _COPY_BUF.clear()
        torch.cuda.empty_cache()
        r = bench_rowsum(max(3, args.steps // 2), 2, 4)
        log(f"[bench] rowsum: {r['gbs']:.1f} GB/s")
        extras["rowsum_8192x65536_fp16"] = r
        g = bench_gemm(max(3, args.steps // 2), 2, 4)
        log(f"[bench] gemm: {g['tflops']:.1f} TFLOP/s")
        extras["gemm_4096_bf16"] = g
    cpu = None
    if not args.no_cpu:
        log("[bench] cpu baseline ...")
        cpu = cpu_baseline(args.cpu_rows)
        log(f"[bench] cpu oracle: {cpu['value']:.2f} GB/s")

    achieved = head["bytes"] / (head["kernel_ms"] * 1e-3) / 1e9
    kname = (f"void pipe::stream_kernel<{head['stages']}, {head['consumer_waves']}, "
             f"{head['producer_waves']}, 0, false>(pipe::StreamParams)")
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
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": kname},
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
