"""GPU parity of grouped loads (PIPE_FLAG_GROUP_LOADS with strips of 4 tile
columns): producers that fill the 4 slots of a tile row with 2-row x 512-byte
loads into interleaved slots, and consumers that store the 4 tiles together,
must give the copy's bits; shapes the grouped kernels do not take run the
plain or pairwise path."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import protocol as P
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GL = pt.PIPE_FLAG_STRIP_GROUPS | pt.PIPE_FLAG_GROUP_LOADS


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("S", [4, 8])
@pytest.mark.parametrize("C,PW", [(4, 4), (4, 2), (8, 4), (8, 2)])
@pytest.mark.parametrize("extra", [0, pt.PIPE_FLAG_SPLIT_INTERLEAVE | pt.PIPE_FLAG_XCD_REMAP])
def test_group_loads_bit_exact(S, C, PW, extra):
    """1280 x 1024: 10 tile rows, 4 strips of 4 tile columns, each in 3 segments
    on 5 persistent workgroups, so rings wrap across items; unique 16-bit codes."""
    print(f"[group_loads] S={S} C={C} PW={PW} extra={extra}", flush=True)
    M, N = 1280, 1024
    src = synth.unique_codes(M, N).to(DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=S, consumer_waves=C, producer_waves=PW, split=3, grid=5,
                            flags=GL | extra | pt.PIPE_FLAG_NONTEMPORAL, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), R.tile_copy(src.cpu().numpy()).view(np.uint16))


@pytest.mark.parametrize("shift", [0, 1, 3])
def test_group_loads_swizzle_shifts_and_temporal_stores(shift):
    src = synth.unique_codes(512, 2048).to(DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=8, swizzle_shift=shift, flags=GL, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))


@pytest.mark.parametrize("shape", [(512, 384), (1000, 1024), (1024, 1000), (129, 8)])
def test_group_loads_flag_elsewhere_runs_other_paths(shape):
    """6 tile columns group in pairs; ragged shapes run the plain ring."""
    M, N = shape
    src = synth.unique_codes(M, N).to(DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=8, flags=GL, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))


def test_group_loads_strided_views():
    big = synth.unique_codes(640, 1024).to(DEV)
    src = big[:512, 128:640]          # ld_src = 1024, 8 tile columns
    out = torch.zeros(512, 768, dtype=torch.float16, device=DEV)
    dst = out[:, 64:576]              # ld_dst = 768
    pt.pipe_tile_copy(src, dst, stages=8, flags=GL)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst.contiguous()), _bits(src.contiguous()))
    assert int((out[:, :64] != 0).sum()) == 0 and int((out[:, 576:] != 0).sum()) == 0


def test_group_loads_trace_cursors():
    """One workgroup, 3 tile rows of one 4-wide strip through an 8-slot ring:
    the producer acquires and the consumers pass their waits at the cursor
    values of tiles 0..11, and a group's slots are refilled only after all
    four tiles of the group before last were released."""
    src = synth.uniform((384, 256), torch.float16, seed=42).to(DEV)
    trace = torch.zeros(24 * pt.PIPE_TRACE_WORDS, dtype=torch.int32, device=DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=8, grid=1, split=1, trace=trace, trace_capacity=24,
                            flags=GL | pt.PIPE_FLAG_TRACE, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    tr = trace.cpu().numpy().view(np.uint32).reshape(24, pt.PIPE_TRACE_WORDS)
    prod, cons = tr[0::2], tr[1::2]
    clock = lambda rec: (int(rec[7]) << 32) | int(rec[6])
    for t in range(12):
        assert prod[t][0] == 0 and prod[t][1] == t and cons[t][0] == 1 and cons[t][1] == t
        assert tuple(prod[t][2:4]) == P.cursor_after(8, t, 1)
        assert tuple(cons[t][2:4]) == P.cursor_after(8, t, 0)
        assert clock(cons[t]) >= clock(prod[t])
    # tiles 8..11 reuse the slots of tiles 0..3, released only with their group
    assert clock(prod[8]) >= clock(cons[3])


def test_group_loads_missing_release_times_out():
    src = synth.unique_codes(1024, 512).to(DEV)
    st = _status()
    pt.pipe_tile_copy(src, stages=4, grid=1, flags=GL | pt.PIPE_FLAG_TEST_NO_RELEASE,
                      spin_limit=20000, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & pt.PIPE_STATUS_TIMEOUT_PRODUCER


@pytest.mark.parametrize("S,C,PW,split,remap", [(8, 4, 4, 4, True), (8, 8, 4, 4, True),
                                                 (4, 4, 4, 4, True), (8, 4, 4, 16, False)])
def test_group_loads_full_size_bit_exact(S, C, PW, split, remap):
    """fp16 16384 x 16384 uniform[-1,1): 64 strips of 4 tile columns, in 4
    interleaved segments each, or in 16 without the XCD remap (the launch the
    benchmark times: 1024 workgroups of 32 tiles)."""
    print(f"[group_loads] full size S={S} C={C} PW={PW} split={split} remap={remap}", flush=True)
    src = synth.uniform((16384, 16384), torch.float16, seed=42, device=DEV)
    flags = GL | pt.PIPE_FLAG_SPLIT_INTERLEAVE | pt.PIPE_FLAG_NONTEMPORAL | \
        pt.PIPE_FLAG_LAZY_COMMIT | (pt.PIPE_FLAG_XCD_REMAP if remap else 0)
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 16384, 16384, stages=S, consumer_waves=C,
                             producer_waves=PW, split=split, flags=flags)
    items = 64 * split
    assert (q["items"], q["grid"], q["tiles_per_item"], q["split"]) == \
        (items, items, 128 * 4 // split, split)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=S, consumer_waves=C, producer_waves=PW, split=split,
                            flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))
    rows = torch.tensor([0, 1, 127, 128, 8191, 16383], device=DEV)
    assert np.array_equal(_bits(dst[rows]), R.tile_copy(src[rows].cpu().numpy()).view(np.uint16))
