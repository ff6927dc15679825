"""GPU parity of the tile stream (copy and row sum) against the CPU oracle.

Every input comes from ``synth`` (seeded); the expected values come from
``oracle`` on the same bits. Copies and integer-data row sums must match bit
for bit; fp row sums within |err| <= 1e-3 * max(|ref|, rms(ref)).
"""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import protocol as P
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


# ---------------------------------------------------------------- copy
def test_copy_single_tile_per_workgroup_index_codes():
    """128x64 tiles of a 256x128 matrix, one tile per workgroup (2x2), S=1."""
    src = synth.index_coded(256, 128).to(DEV)
    st = _status()
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 256, 128, stages=1, split=2)
    assert (q["items"], q["grid"], q["tiles_per_item"]) == (4, 4, 1)
    dst = pt.pipe_tile_copy(src, stages=1, split=2, producer_waves=1, flags=0, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), R.tile_copy(src.cpu().numpy()).view(np.uint16))
    # unique codes: a misplaced element names its source
    u = synth.unique_codes(256, 128).to(DEV)
    du = pt.pipe_tile_copy(u, stages=1, split=2)
    torch.cuda.synchronize()
    got, exp = _bits(du), _bits(u)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, f"first mismatches (r,c): {bad[:5].tolist()} got {got[tuple(bad[0])]}"


def test_copy_three_stage_ring_checksums_and_trace():
    """One workgroup (1 producer + 3 consumer waves), 8 tiles along the columns."""
    src = synth.uniform((128, 512), torch.float16, seed=42).to(DEV)
    trace = torch.zeros(16 * pt.PIPE_TRACE_WORDS, dtype=torch.int32, device=DEV)
    st = _status()
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=3, producer_waves=1,
                                 consumer_waves=3, grid=1, flags=pt.PIPE_FLAG_TRACE, trace=trace,
                                 trace_capacity=16, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    s_np = src.cpu().numpy()
    assert np.array_equal(_bits(dst), R.tile_copy(s_np).view(np.uint16))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(s_np))
    tr = trace.cpu().numpy().view(np.uint32).reshape(16, pt.PIPE_TRACE_WORDS)
    prod = tr[0::2]
    cons = tr[1::2]
    for t in range(8):
        assert prod[t][0] == 0 and prod[t][1] == t and cons[t][0] == 1 and cons[t][1] == t
        assert tuple(prod[t][2:4]) == P.cursor_after(3, t, 1)   # producer starts at phase 1
        assert tuple(cons[t][2:4]) == P.cursor_after(3, t, 0)
        assert prod[t][4] == t and cons[t][4] == t
    clock = lambda rec: (int(rec[7]) << 32) | int(rec[6])
    for t in range(8):
        # a consumer passes its wait only after the producer acquired that slot
        assert clock(cons[t]) >= clock(prod[t])
        # back-pressure: slot reuse for tile t+3 only after consumers passed tile t
        if t + 3 < 8:
            assert clock(prod[t + 3]) >= clock(cons[t])


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("C", [1, 2, 3, 4, 8])
def test_copy_stage_and_wave_sweep(S, C):
    M, N = 1024, 640  # 8 x 10 tiles
    src = synth.unique_codes(M, N).to(DEV)
    st = _status()
    # persistent grid smaller than the item count; strips cut in 3 segments
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=S, consumer_waves=C, split=3,
                                 grid=7, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("C", [2, 3, 8])
@pytest.mark.parametrize("remap", [False, True])
def test_copy_two_producer_waves(S, C, remap):
    M, N = 1024, 1024  # 8 x 16 tiles, 16 column strips x 2 segments = 32 items
    src = synth.unique_codes(M, N).to(DEV)
    st = _status()
    flags = pt.PIPE_FLAG_XCD_REMAP if remap else 0
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=S, consumer_waves=C,
                                 producer_waves=2, split=2, grid=9, flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


@pytest.mark.parametrize("split", [2, 3, 5])
@pytest.mark.parametrize("row_strips", [False, True])
def test_copy_interleaved_segments(split, row_strips):
    src = synth.unique_codes(1280, 640).to(DEV)   # 10 x 10 tiles
    flags = pt.PIPE_FLAG_SPLIT_INTERLEAVE | (pt.PIPE_FLAG_ROW_STRIPS if row_strips else 0)
    st = _status()
    dst, chk = pt.pipe_tile_copy(src, checksums=True, split=split, grid=7, flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


@pytest.mark.parametrize("shift", [0, 1, 2, 3])
@pytest.mark.parametrize("row_strips", [False, True])
def test_copy_swizzle_and_walk_order(shift, row_strips):
    src = synth.unique_codes(512, 1024).to(DEV)
    flags = pt.PIPE_FLAG_ROW_STRIPS if row_strips else 0
    dst = pt.pipe_tile_copy(src, stages=3, swizzle_shift=shift, flags=flags, grid=5)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst), _bits(src))


def test_copy_strided_views():
    big = synth.unique_codes(640, 1024).to(DEV)
    src = big[:512, 128:640]          # ld_src = 1024
    out = torch.zeros(512, 768, dtype=torch.float16, device=DEV)
    dst = out[:, 64:576]              # ld_dst = 768
    pt.pipe_tile_copy(src, dst, stages=2)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst.contiguous()), _bits(src.contiguous()))
    assert int((out[:, :64] != 0).sum()) == 0 and int((out[:, 576:] != 0).sum()) == 0


@pytest.mark.parametrize("S", [1, 2, 3, 4, 6, 8])
def test_copy_full_size_bit_exact(S):
    """fp16 16384 x 16384 uniform[-1,1), persistent column strips."""
    src = synth.uniform((16384, 16384), torch.float16, seed=42, device=DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=S, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))
    # and a sample of rows against the oracle on the host
    rows = torch.tensor([0, 1, 127, 128, 8191, 16383], device=DEV)
    s_np = src[rows].cpu().numpy()
    assert np.array_equal(_bits(dst[rows]), R.tile_copy(s_np).view(np.uint16))


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("shape", [(300, 200), (1000, 1000), (129, 8), (1, 72), (640, 4104)])
@pytest.mark.parametrize("row_strips", [False, True])
def test_copy_ragged_edges(S, shape, row_strips):
    """Partial last tile row / column: in-range elements copied, checksums over them."""
    M, N = shape
    src = synth.unique_codes(M, N).to(DEV)
    pitch = N + 24
    out = torch.full((M, pitch), -7.0, dtype=torch.float16, device=DEV)
    dst = out[:, :N]
    st = _status()
    flags = pt.PIPE_FLAG_ROW_STRIPS if row_strips else 0
    _, chk = pt.pipe_tile_copy(src, dst, checksums=True, stages=S, grid=3, flags=flags,
                               status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst.contiguous()), _bits(src))
    assert bool((out[:, N:] == -7.0).all())       # pitch padding untouched
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


# ---------------------------------------------------------------- watchdog
def test_start_phase_zero_times_out_instead_of_hanging():
    src = synth.unique_codes(256, 256).to(DEV)
    st = _status()
    pt.pipe_tile_copy(src, stages=3, spin_limit=2000, status=st,
                      flags=pt.PIPE_FLAG_TEST_START_PHASE0)
    torch.cuda.synchronize()
    v = int(st.item())
    assert v & pt.PIPE_STATUS_TIMEOUT_PRODUCER and v & pt.PIPE_STATUS_TIMEOUT_CONSUMER
    assert pt.pipe_status_from_word(v) == pt.PIPE_ERR_TIMEOUT


def test_missing_release_times_out_instead_of_hanging():
    src = synth.unique_codes(128, 640).to(DEV)  # 10 tiles in one strip walk
    st = _status()
    pt.pipe_tile_copy(src, stages=3, grid=1, spin_limit=2000, status=st,
                      flags=pt.PIPE_FLAG_TEST_NO_RELEASE | pt.PIPE_FLAG_ROW_STRIPS)
    torch.cuda.synchronize()
    assert int(st.item()) & pt.PIPE_STATUS_TIMEOUT_PRODUCER


def test_library_status_word_when_no_status_given():
    pt.pipe_device_status(clear=True)
    src = synth.unique_codes(256, 256).to(DEV)
    pt.pipe_tile_copy(src, stages=2, spin_limit=1000, flags=pt.PIPE_FLAG_TEST_START_PHASE0)
    torch.cuda.synchronize()
    assert pt.pipe_device_status(clear=True) != 0
    pt.pipe_tile_copy(src, stages=2)
    torch.cuda.synchronize()
    assert pt.pipe_device_status() == 0


# ---------------------------------------------------------------- row sum
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("C", [1, 3, 4, 8])
@pytest.mark.parametrize("split", [1, 3, 8])
def test_rowsum_small_integers_bit_exact(S, C, split):
    """Integer data keeps every partial sum exact in fp32: any order is exact."""
    A = synth.small_int((512, 2048), -8, 8, torch.float16, seed=5).to(DEV)
    st = _status()
    out = pt.pipe_rowsum(A, stages=S, consumer_waves=C, split=split, grid=11, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


@pytest.mark.parametrize("S", [2, 4])
@pytest.mark.parametrize("remap", [False, True])
def test_rowsum_two_producer_waves_bit_exact(S, remap):
    A = synth.small_int((1024, 4096), -8, 8, torch.float16, seed=6).to(DEV)
    flags = pt.PIPE_FLAG_XCD_REMAP | pt.PIPE_FLAG_NONTEMPORAL if remap else 0
    out = pt.pipe_rowsum(A, stages=S, consumer_waves=8, producer_waves=2, split=4, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


@pytest.mark.parametrize("split", [2, 4, 7])
@pytest.mark.parametrize("shape", [(1024, 4096), (300, 1000)])
def test_rowsum_interleaved_segments_bit_exact(split, shape):
    A = synth.small_int(shape, -8, 8, torch.float16, seed=8).to(DEV)
    out = pt.pipe_rowsum(A, split=split, flags=pt.PIPE_FLAG_SPLIT_INTERLEAVE, grid=9)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


def test_rowsum_normal_within_tolerance_and_deterministic():
    A = synth.normal((1024, 8192), torch.float16, seed=42).to(DEV)
    out1 = pt.pipe_rowsum(A)
    out2 = pt.pipe_rowsum(A)
    torch.cuda.synchronize()
    ref = R.rowsum_exact(A.cpu().numpy())
    res = R.within_tol(out1.cpu().numpy(), ref, 1e-3)
    assert res["ok"], res
    assert torch.equal(out1, out2)


@pytest.fixture(scope="module")
def rowsum_full():
    """The full 1 GiB row-sum input, fp16 8192 x 65536 normal(0,1), and its exact
    row sums (computed once for the tests below)."""
    A = synth.normal((8192, 65536), torch.float16, seed=42, device=DEV)
    return A, R.rowsum_exact(A.cpu().numpy())


@pytest.mark.parametrize("cfg", [
    {},                                                        # the default 3-stage ring
    dict(tile_m=64, tile_n=128, stages=3, producer_waves=4, consumer_waves=4, split=2,
         flags=pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_XCD_REMAP),
    dict(tile_m=32, tile_n=256, stages=3, producer_waves=4, consumer_waves=4, split=1,
         flags=pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_XCD_REMAP),
], ids=["default", "64x128", "32x256"])
def test_rowsum_full_size_within_tolerance(rowsum_full, cfg):
    """The full input in the configurations bench.py times."""
    A, ref = rowsum_full
    st = _status()
    out = pt.pipe_rowsum(A, status=st, **cfg)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    res = R.within_tol(out.cpu().numpy(), ref, 1e-3)
    assert res["ok"], res


@pytest.mark.parametrize("shape", [(1000, 3000), (129, 72), (5, 8), (2050, 640)])
@pytest.mark.parametrize("split", [1, 4])
def test_rowsum_ragged_bit_exact(shape, split):
    M, N = shape
    A = synth.small_int((M, N), -8, 8, torch.float16, seed=11).to(DEV)
    st = _status()
    out = pt.pipe_rowsum(A, split=split, grid=13, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


def test_rowsum_ragged_normal_within_tolerance():
    A = synth.normal((777, 10000), torch.float16, seed=42).to(DEV)
    out = pt.pipe_rowsum(A)
    torch.cuda.synchronize()
    res = R.within_tol(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()), 1e-3)
    assert res["ok"], res


def test_rowsum_degenerate_shapes():
    A = torch.empty((256, 0), dtype=torch.float16, device=DEV)
    out = torch.full((256,), 7.0, device=DEV)
    pt.pipe_rowsum(A, out)
    torch.cuda.synchronize()
    assert int((out != 0).sum()) == 0
    E = torch.empty((0, 128), dtype=torch.float16, device=DEV)
    assert pt.pipe_rowsum(E).numel() == 0
    ones = torch.ones((128, 65536), dtype=torch.float16, device=DEV)
    o = pt.pipe_rowsum(ones, split=5)
    torch.cuda.synchronize()
    assert torch.equal(o, torch.full((128,), 65536.0, device=DEV))


def test_premarshalled_launchers_match():
    src = synth.unique_codes(512, 512).to(DEV)
    dst = torch.zeros_like(src)
    launch = pt.copy_launcher(src, dst, stages=3)
    launch()
    launch()
    A = synth.small_int((512, 1024), -8, 8, torch.float16, seed=2).to(DEV)
    out = torch.empty(512, device=DEV)
    ws = torch.empty(pt.pipe_rowsum_workspace_bytes(512, 1024) + 4, dtype=torch.uint8, device=DEV)
    pt.rowsum_launcher(A, out, ws)()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


def test_copy_offsets_beyond_4gib():
    """fp16 (32768 + 72) x 65536 (4.3 GB per matrix): byte offsets pass 2**32, a
    ragged last tile row included."""
    M, N = 32768 + 72, 65536
    src = synth.uniform((M, N), torch.float16, seed=7, device=DEV)
    dst = torch.empty_like(src)
    st = _status()
    pt.pipe_tile_copy(src, dst, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))
    rows = torch.tensor([0, 32767, 32768, M - 1], device=DEV)
    assert np.array_equal(_bits(dst[rows]), R.tile_copy(src[rows].cpu().numpy()).view(np.uint16))
    del src, dst
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- deep rings, 4 producer waves
@pytest.mark.parametrize("S", [3, 5, 6, 7, 8])
@pytest.mark.parametrize("PW", [1, 2, 4])
@pytest.mark.parametrize("C", [4, 8])
def test_copy_deep_rings(S, PW, C):
    """S up to 8 slots (128 KiB of LDS) and 1, 2 or 4 producer waves; every
    workgroup walks several items, so the ring wraps many times."""
    M, N = 2048, 1280  # 16 x 20 tiles; 20 strips x 3 segments = 60 items on 7 workgroups
    src = synth.unique_codes(M, N).to(DEV)
    st = _status()
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=S, producer_waves=PW,
                                 consumer_waves=C, split=3, grid=7, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


@pytest.mark.parametrize("S", [5, 8])
@pytest.mark.parametrize("PW", [1, 2, 4])
@pytest.mark.parametrize("shape", [(1024, 4096), (1000, 3000)])
def test_rowsum_deep_rings_bit_exact(S, PW, shape):
    A = synth.small_int(shape, -8, 8, torch.float16, seed=13).to(DEV)
    st = _status()
    out = pt.pipe_rowsum(A, stages=S, producer_waves=PW, consumer_waves=8, split=3, grid=5,
                         status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


@pytest.mark.parametrize("row_strips", [False, True])
def test_copy_deep_ring_ragged(row_strips):
    src = synth.unique_codes(1000, 1000).to(DEV)
    flags = pt.PIPE_FLAG_ROW_STRIPS if row_strips else 0
    dst = pt.pipe_tile_copy(src, stages=8, producer_waves=4, consumer_waves=8, split=2, grid=3,
                            flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst), _bits(src))


# ---------------------------------------------------------------- commit policies
POLICY = {"eager": 0, "lazy": pt.PIPE_FLAG_LAZY_COMMIT, "newest": pt.PIPE_FLAG_EAGER_NEWEST}


@pytest.mark.parametrize("policy", ["eager", "lazy", "newest"])
@pytest.mark.parametrize("S,PW,C", [(1, 1, 3), (2, 1, 4), (3, 1, 8), (4, 2, 4), (6, 4, 8),
                                    (8, 2, 4)])
def test_copy_commit_policies_bit_exact(policy, S, PW, C):
    """Eager commits (two thresholds) and lag-only commits give the same bits,
    with the lag at its bound S - 1 or below it."""
    src = synth.unique_codes(1024, 1280).to(DEV)
    st = _status()
    flags = POLICY[policy]
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=S, producer_waves=PW,
                                 consumer_waves=C, split=2, grid=6, flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


@pytest.mark.parametrize("policy", ["eager", "lazy", "newest"])
@pytest.mark.parametrize("S,PW", [(2, 1), (3, 1), (4, 2), (6, 4)])
def test_rowsum_commit_policies_bit_exact(policy, S, PW):
    A = synth.small_int((1024, 4096), -8, 8, torch.float16, seed=14).to(DEV)
    st = _status()
    flags = POLICY[policy]
    out = pt.pipe_rowsum(A, stages=S, producer_waves=PW, consumer_waves=8, split=4, grid=9,
                         flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


# ---------------------------------------------------------------- wider tiles
SHAPES = [(64, 128), (32, 256)]


@pytest.mark.parametrize("tm,tn", SHAPES)
@pytest.mark.parametrize("S,PW,C", [(2, 4, 4), (3, 2, 8), (4, 4, 8)])
@pytest.mark.parametrize("split,flags", [(1, 0), (3, pt.PIPE_FLAG_SPLIT_INTERLEAVE),
                                         (2, pt.PIPE_FLAG_ROW_STRIPS)])
def test_copy_wide_tiles_bit_exact(tm, tn, S, PW, C, split, flags):
    src = synth.unique_codes(1024, 1536).to(DEV)
    st = _status()
    dst, chk = pt.pipe_tile_copy(src, checksums=True, tile_m=tm, tile_n=tn, stages=S,
                                 producer_waves=PW, consumer_waves=C, split=split, grid=5,
                                 flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32),
                          R.tile_checksums(src.cpu().numpy(), tm, tn))


@pytest.mark.parametrize("tm,tn", SHAPES)
@pytest.mark.parametrize("shape", [(1000, 1000), (33, 264), (300, 8)])
def test_copy_wide_tiles_ragged(tm, tn, shape):
    src = synth.unique_codes(*shape).to(DEV)
    dst, chk = pt.pipe_tile_copy(src, checksums=True, tile_m=tm, tile_n=tn, stages=2,
                                 producer_waves=4, consumer_waves=4, grid=3)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32),
                          R.tile_checksums(src.cpu().numpy(), tm, tn))


@pytest.mark.parametrize("tm,tn", SHAPES)
@pytest.mark.parametrize("shape", [(1024, 4096), (1000, 3000)])
@pytest.mark.parametrize("S,PW,C", [(2, 4, 4), (4, 2, 8)])
def test_rowsum_wide_tiles_bit_exact(tm, tn, shape, S, PW, C):
    A = synth.small_int(shape, -8, 8, torch.float16, seed=15).to(DEV)
    st = _status()
    out = pt.pipe_rowsum(A, tile_m=tm, tile_n=tn, stages=S, producer_waves=PW,
                         consumer_waves=C, split=3, grid=7, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


@pytest.mark.parametrize("tm,tn", SHAPES)
@pytest.mark.parametrize("S,W", [(2, 2), (4, 4)])
def test_unified_wide_tiles_bit_exact(tm, tn, S, W):
    src = synth.unique_codes(1024, 1536).to(DEV)
    dst = pt.pipe_tile_copy(src, tile_m=tm, tile_n=tn, stages=S, consumer_waves=W, split=2,
                            grid=5, flags=pt.PIPE_FLAG_UNIFIED)
    A = synth.small_int((512, 4096), -8, 8, torch.float16, seed=16).to(DEV)
    out = pt.pipe_rowsum(A, tile_m=tm, tile_n=tn, stages=S, consumer_waves=W, split=4, grid=5,
                         flags=pt.PIPE_FLAG_UNIFIED)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


@pytest.mark.parametrize("tm,tn", SHAPES)
def test_copy_wide_tiles_full_size_bit_exact(tm, tn):
    src = synth.uniform((16384, 16384), torch.float16, seed=42, device=DEV)
    dst = pt.pipe_tile_copy(src, tile_m=tm, tile_n=tn, stages=2, producer_waves=4,
                            consumer_waves=8, split=8, flags=pt.PIPE_FLAG_SPLIT_INTERLEAVE |
                            pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_XCD_REMAP |
                            pt.PIPE_FLAG_LAZY_COMMIT)
    torch.cuda.synchronize()
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))


# ---------------------------------------------------------------- unified variant
@pytest.mark.parametrize("S", [1, 2, 3, 4, 6, 8])
@pytest.mark.parametrize("W", [2, 4, 8])
def test_unified_copy_bit_exact(S, W):
    src = synth.unique_codes(1024, 640).to(DEV)
    dst = pt.pipe_tile_copy(src, stages=S, consumer_waves=W, split=3, grid=7,
                            flags=pt.PIPE_FLAG_UNIFIED | pt.PIPE_FLAG_NONTEMPORAL)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst), _bits(src))


@pytest.mark.parametrize("S", [1, 3, 4, 7])
@pytest.mark.parametrize("W", [2, 8])
@pytest.mark.parametrize("interleave", [False, True])
def test_unified_rowsum_bit_exact(S, W, interleave):
    A = synth.small_int((512, 4096), -8, 8, torch.float16, seed=12).to(DEV)
    flags = pt.PIPE_FLAG_UNIFIED | (pt.PIPE_FLAG_SPLIT_INTERLEAVE if interleave else 0)
    out = pt.pipe_rowsum(A, stages=S, consumer_waves=W, split=4, grid=5, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


def test_unified_copy_full_size_bit_exact():
    src = synth.uniform((16384, 16384), torch.float16, seed=42, device=DEV)
    dst = pt.pipe_tile_copy(src, stages=3, consumer_waves=4, flags=pt.PIPE_FLAG_UNIFIED)
    torch.cuda.synchronize()
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))


@pytest.mark.parametrize("op,M,N,K,cfg", [
    (pt.PIPE_OP_COPY, 16384, 16384, 0, {}),
    (pt.PIPE_OP_COPY, 1000, 1000, 0, {}),                      # ragged: the masked kernel
    (pt.PIPE_OP_COPY, 16384, 16384, 0, dict(tile_m=32, tile_n=256, consumer_waves=8)),
    (pt.PIPE_OP_COPY, 16384, 16384, 0, dict(stages=3, consumer_waves=4,
                                            flags=pt.PIPE_FLAG_UNIFIED)),
    (pt.PIPE_OP_COPY, 16384, 16384, 0, dict(stages=5, producer_waves=2,
                                            flags=pt.PIPE_FLAG_STRIP_GROUPS)),
    (pt.PIPE_OP_COPY, 16384, 16384, 0, dict(flags=pt.PIPE_FLAG_PRODUCER_VGPR)),
    (pt.PIPE_OP_COPY, 1000, 1000, 0, dict(stages=3, producer_waves=1, consumer_waves=3,
                                          flags=pt.PIPE_FLAG_PRODUCER_VGPR)),
    (pt.PIPE_OP_COPY, 16384, 16384, 0, dict(flags=pt.PIPE_FLAG_DEBUG_CHECKS)),
    (pt.PIPE_OP_ROWSUM, 8192, 65536, 0, {}),
    (pt.PIPE_OP_ROWSUM, 8192, 65536, 0, dict(stages=8, consumer_waves=8)),
    (pt.PIPE_OP_ROWSUM, 8192, 65536, 0, dict(stages=4, flags=pt.PIPE_FLAG_PRODUCER_VGPR)),
    (pt.PIPE_OP_ROWSUM, 1000, 3000, 0, dict(stages=2, producer_waves=1, consumer_waves=3,
                                            flags=pt.PIPE_FLAG_DEBUG_CHECKS)),
    (pt.PIPE_OP_GEMM, 4096, 4096, 4096, {}),
    (pt.PIPE_OP_GEMM, 4096, 4096, 4096, dict(flags=pt.PIPE_FLAG_GEMM_C_BF16 |
                                             pt.PIPE_FLAG_EAGER_NEWEST)),
    (pt.PIPE_OP_GEMM, 4096, 4096, 4096, dict(flags=pt.PIPE_FLAG_GEMM_B_COLMAJOR |
                                             pt.PIPE_FLAG_EAGER_NEWEST)),
    (pt.PIPE_OP_GEMM, 1024, 1024, 1024, dict(stages=4, producer_waves=2)),
    (pt.PIPE_OP_GEMM, 4096, 4096, 4096, dict(stages=3, flags=pt.PIPE_FLAG_GEMM_C_BF16 |
                                             pt.PIPE_FLAG_EAGER_NEWEST)),   # ring + staging
    (pt.PIPE_OP_GEMM, 4096, 4096, 4096, dict(stages=3, flags=pt.PIPE_FLAG_GEMM_C_BF16 |
                                             pt.PIPE_FLAG_GEMM_STORE_WAVE)),
    (pt.PIPE_OP_GEMM, 1000, 1000, 1000, dict(stages=3)),             # ragged: the masked kernel
    (pt.PIPE_OP_COPY, 16384, 16384, 0, dict(stages=8, consumer_waves=8,
                                            flags=pt.PIPE_FLAG_STRIP_GROUPS |
                                            pt.PIPE_FLAG_GROUP_LOADS)),
])
def test_kernel_resources_agree_with_the_launch_geometry(op, M, N, K, cfg):
    """The runtime's static LDS for the kernel an op launches equals the LDS
    that pipe_query_kernel computes for it; the kernel fits the workgroup, and
    the default configurations spill nothing."""
    res = pt.pipe_kernel_resources(op, M, N, K, **cfg)
    q = pt.pipe_query_kernel(op, M, N, K, **cfg)
    assert res["lds_bytes"] == q["lds_bytes"], (res, q)
    assert 0 < res["vgprs"] <= 512
    assert res["max_threads"] >= q["threads"]
    if not cfg or cfg.get("flags", 0) & (pt.PIPE_FLAG_STRIP_GROUPS | pt.PIPE_FLAG_PRODUCER_VGPR):
        assert res["scratch_bytes"] == 0   # defaults and the grouped / register kernels: no spills


def test_kernel_lookup_on_one_thread_never_swallows_a_launch_on_another():
    """pipe_kernel_resources finds its kernel by running the launch path with a
    record slot set; the slot is per thread, so copies launched meanwhile from
    another thread must all run (ctypes releases the GIL during each call)."""
    import threading
    src = synth.uniform((1024, 4096), torch.float16, seed=21, device=DEV)
    stop = threading.Event()
    seen = []

    def lookups():
        while not stop.is_set():
            seen.append(pt.pipe_kernel_resources(pt.PIPE_OP_COPY, 1024, 4096)["vgprs"])

    t = threading.Thread(target=lookups)
    t.start()
    try:
        for i in range(200):
            dst = torch.zeros_like(src)
            pt.pipe_tile_copy(src, dst)
            torch.cuda.synchronize()
            assert torch.equal(dst.view(torch.int16), src.view(torch.int16)), f"copy {i} did not run"
    finally:
        stop.set()
        t.join()
    assert len(seen) > 0 and all(v > 0 for v in seen)


def test_binding_checks_buffer_sizes():
    """Undersized trace, status, out and checksum buffers are refused by the
    binding before any launch (the kernels would write past them)."""
    src = synth.unique_codes(256, 256).to(DEV)
    small_trace = torch.zeros(8 * pt.PIPE_TRACE_WORDS - 1, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        pt.pipe_tile_copy(src, flags=pt.PIPE_FLAG_TRACE, trace=small_trace, trace_capacity=8)
    with pytest.raises(ValueError):
        pt.pipe_tile_copy(src, status=torch.zeros(0, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        pt.pipe_tile_copy(src, status=torch.zeros(4, dtype=torch.int32, device=DEV)[::2])
    A = synth.small_int((256, 1024), -8, 8, torch.float16, seed=3).to(DEV)
    with pytest.raises(ValueError):
        pt.pipe_rowsum(A, out=torch.empty(255, device=DEV))
    with pytest.raises(ValueError):
        pt.pipe_rowsum(A, out=torch.empty(256, dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):
        pt.rowsum_launcher(A, torch.empty(256, device=DEV),
                           workspace=torch.empty(2 * 65536, dtype=torch.uint8, device=DEV)[::2],
                           split=4)
    dst = torch.empty_like(src)
    with pytest.raises(ValueError):   # 2 x 4 tiles of 128 x 64 need 8 words
        pt.copy_launcher(src, dst, checksums=torch.zeros(7, dtype=torch.int32, device=DEV))
    # the exact sizes are accepted
    trace = torch.zeros(8 * pt.PIPE_TRACE_WORDS, dtype=torch.int32, device=DEV)
    pt.pipe_tile_copy(src, dst, flags=pt.PIPE_FLAG_TRACE, trace=trace, trace_capacity=8)
    chk = torch.zeros(8, dtype=torch.int32, device=DEV)
    pt.copy_launcher(src, dst, checksums=chk)()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


