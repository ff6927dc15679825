"""The library's launches inside a captured HIP graph.

A caller that wants to amortise launch cost can capture the entry points on
a stream and replay the graph: each entry point only enqueues kernels on the
stream it is given (no allocation, memset or synchronisation). The graph
below is captured once and replayed several times. Between replays the inputs
are rewritten eagerly and the outputs cleared, and every replay is checked
against the CPU oracle on that replay's inputs.
"""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_copy_rowsum_gemm_replayed_from_one_graph():
    src = torch.empty(1024, 1280, dtype=torch.float16, device=DEV)
    dst = torch.empty_like(src)
    chk = torch.empty((1024 // 128) * (1280 // 64), dtype=torch.int32, device=DEV)
    A = torch.empty(1000, 3000, dtype=torch.float16, device=DEV)       # ragged edges
    sums = torch.empty(1000, dtype=torch.float32, device=DEV)
    ws = torch.empty(pt.pipe_rowsum_workspace_bytes(1000, 3000), dtype=torch.uint8, device=DEV)
    Ga = torch.empty(256, 512, dtype=torch.bfloat16, device=DEV)
    Gb = torch.empty(512, 384, dtype=torch.bfloat16, device=DEV)
    Gc = torch.empty(256, 384, dtype=torch.float32, device=DEV)
    Gc2 = torch.empty(256, 384, dtype=torch.bfloat16, device=DEV)   # 256 x 128 tiles, bf16 C
    Gc3 = torch.empty(256, 384, dtype=torch.float32, device=DEV)    # unified 4-wave, 32-K stages
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def fill(seed):
        src.copy_(synth.uniform((1024, 1280), torch.float16, seed=seed).to(DEV))
        A.copy_(synth.small_int((1000, 3000), -8, 8, torch.float16, seed=seed + 1).to(DEV))
        Ga.copy_(synth.small_int((256, 512), -2, 2, torch.bfloat16, seed=seed + 2).to(DEV))
        Gb.copy_(synth.small_int((512, 384), -2, 2, torch.bfloat16, seed=seed + 3).to(DEV))
        for t in (dst, chk, sums, Gc, Gc2, Gc3):
            t.zero_()

    def body():
        pt.pipe_tile_copy(src, dst, checksums=False, stages=3, status=status)
        pt.copy_launcher(src, dst, checksums=chk, stages=2, status=status)()
        pt.pipe_rowsum(A, sums, ws, status=status)
        pt.pipe_gemm_mainloop(Ga, Gb, Gc, status=status)
        pt.pipe_gemm_mainloop(Ga, Gb, Gc2, status=status, tile_m=256, consumer_waves=8)
        pt.pipe_gemm_mainloop(Ga, Gb, Gc3, status=status, **pt.GEMM_UNIFIED_DEEP)

    fill(10)
    body()                      # eager run first: the same calls, outside any graph
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep, seed in enumerate((20, 30, 40, 50)):
        fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, rep
        s_np = src.cpu().numpy()
        assert np.array_equal(_bits(dst), R.tile_copy(s_np).view(np.uint16)), rep
        assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(s_np)), rep
        assert np.array_equal(sums.cpu().numpy(), R.rowsum_exact(A.cpu().numpy())), rep
        ref = R.gemm_f64(Ga.float().cpu().numpy(), Gb.float().cpu().numpy())
        assert np.array_equal(Gc.cpu().numpy(), ref), rep
        assert np.array_equal(Gc3.cpu().numpy(), ref), rep
        assert np.array_equal(Gc2.float().cpu().numpy(),
                              R.gemm_bf16(Ga.float().cpu().numpy(), Gb.float().cpu().numpy())), rep
        # eager work between replays, on the same buffers
        pt.pipe_tile_copy(dst, src, stages=1)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(src), _bits(dst)), rep


def test_grouped_loads_copy_replayed_from_a_graph():
    """The grouped-load copy (strips of 4 tile columns, S = 8) captured and
    replayed on fresh inputs, bit for bit against the oracle's copy."""
    M, N = 1024, 2048
    src = torch.empty(M, N, dtype=torch.float16, device=DEV)
    dst = torch.empty_like(src)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    cfg = dict(stages=8, producer_waves=4, consumer_waves=8, status=status,
               flags=pt.PIPE_FLAG_STRIP_GROUPS | pt.PIPE_FLAG_GROUP_LOADS |
               pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_LAZY_COMMIT)
    src.copy_(synth.uniform((M, N), torch.float16, seed=60).to(DEV))
    pt.pipe_tile_copy(src, dst, **cfg)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pt.pipe_tile_copy(src, dst, **cfg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep, seed in enumerate((61, 62, 63, 64)):
        src.copy_(synth.uniform((M, N), torch.float16, seed=seed).to(DEV))
        dst.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, rep
        assert np.array_equal(_bits(dst), R.tile_copy(src.cpu().numpy()).view(np.uint16)), rep
