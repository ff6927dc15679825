"""GPU parity of grouped column strips (PIPE_FLAG_STRIP_GROUPS) against the
CPU oracle: consumers that wait on the G slots of a tile row and store G
neighbouring 128 x 64 tiles at once must give the plain copy's bits, and
shapes or requests the grouped kernels do not take must run the plain path."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import protocol as P
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GROUPS = pt.PIPE_FLAG_STRIP_GROUPS
POLICY = {"eager": 0, "lazy": pt.PIPE_FLAG_LAZY_COMMIT, "newest": pt.PIPE_FLAG_EAGER_NEWEST}


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def _group(M, N, S, C, PW):
    """Group size the library chooses, read back from the launch geometry: with
    one segment per strip there is one work item per strip of G tile columns."""
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, M, N, stages=S, consumer_waves=C,
                             producer_waves=PW, split=1, flags=GROUPS)
    return (N // 64) // q["items"]


@pytest.mark.parametrize("S", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("C,PW", [(4, 4), (8, 2)])
@pytest.mark.parametrize("policy", ["eager", "lazy", "newest"])
def test_grouped_copy_bit_exact(S, C, PW, policy):
    """1280 x 1024: 10 x 16 tiles, strips of G = 4 (2 when S < 4) tile columns,
    each strip in 3 segments on 5 persistent workgroups, so rings wrap across items."""
    M, N = 1280, 1024
    src = synth.unique_codes(M, N).to(DEV)
    st = _status()
    assert _group(M, N, S, C, PW) == (4 if S >= 4 else 2)
    dst = pt.pipe_tile_copy(src, stages=S, consumer_waves=C, producer_waves=PW, split=3, grid=5,
                            flags=GROUPS | POLICY[policy] | pt.PIPE_FLAG_NONTEMPORAL, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))


@pytest.mark.parametrize("split", [1, 2, 3, 4, 7])
@pytest.mark.parametrize("extra", [0, pt.PIPE_FLAG_SPLIT_INTERLEAVE, pt.PIPE_FLAG_XCD_REMAP,
                                   pt.PIPE_FLAG_SPLIT_INTERLEAVE | pt.PIPE_FLAG_XCD_REMAP])
def test_grouped_copy_segments_and_item_order(split, extra):
    M, N = 1792, 2048   # 14 x 32 tiles: 8 strips of 4 tile columns
    src = synth.unique_codes(M, N).to(DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=8, split=split, grid=11, flags=GROUPS | extra, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))


def test_grouped_copy_pairs_when_four_do_not_divide():
    """384 tile columns would take G = 4; 6 tile columns take G = 2."""
    M, N = 512, 384
    assert _group(M, N, 8, 4, 4) == 2
    src = synth.unique_codes(M, N).to(DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=8, flags=GROUPS, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))


@pytest.mark.parametrize("shape", [(1000, 1024), (1024, 1000), (300, 200), (129, 8)])
def test_grouped_flag_on_ragged_shapes_runs_the_plain_path(shape):
    M, N = shape
    src = synth.unique_codes(M, N).to(DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=8, flags=GROUPS, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))


def test_grouped_flag_with_checksums_runs_the_plain_path():
    src = synth.uniform((1024, 1024), torch.float16, seed=42).to(DEV)
    st = _status()
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=8, flags=GROUPS, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    s_np = src.cpu().numpy()
    assert np.array_equal(_bits(dst), R.tile_copy(s_np).view(np.uint16))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(s_np))


def test_grouped_copy_strided_views():
    big = synth.unique_codes(640, 1024).to(DEV)
    src = big[:512, 128:640]          # ld_src = 1024, 8 tile columns
    out = torch.zeros(512, 768, dtype=torch.float16, device=DEV)
    dst = out[:, 64:576]              # ld_dst = 768
    pt.pipe_tile_copy(src, dst, stages=4, flags=GROUPS)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst.contiguous()), _bits(src.contiguous()))
    assert int((out[:, :64] != 0).sum()) == 0 and int((out[:, 576:] != 0).sum()) == 0


def test_grouped_copy_trace_cursors():
    """One workgroup, 2 tile rows of a 4-wide strip: the producer acquires and the
    consumers pass their waits at the cursor values of tiles 0..7, and a
    consumer passes tile t's wait only after the producer acquired its slot."""
    src = synth.uniform((256, 256), torch.float16, seed=42).to(DEV)
    trace = torch.zeros(16 * pt.PIPE_TRACE_WORDS, dtype=torch.int32, device=DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=6, grid=1, split=1, trace=trace, trace_capacity=16,
                            flags=GROUPS | pt.PIPE_FLAG_TRACE, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    tr = trace.cpu().numpy().view(np.uint32).reshape(16, pt.PIPE_TRACE_WORDS)
    prod, cons = tr[0::2], tr[1::2]
    clock = lambda rec: (int(rec[7]) << 32) | int(rec[6])
    for t in range(8):
        assert prod[t][0] == 0 and prod[t][1] == t and cons[t][0] == 1 and cons[t][1] == t
        assert tuple(prod[t][2:4]) == P.cursor_after(6, t, 1)
        assert tuple(cons[t][2:4]) == P.cursor_after(6, t, 0)
        assert clock(cons[t]) >= clock(prod[t])
    # slot reuse: tile 6 goes into tile 0's slot, released only with its whole group
    assert clock(prod[6]) >= clock(cons[3])


def test_grouped_copy_missing_release_times_out():
    src = synth.unique_codes(512, 512).to(DEV)
    st = _status()
    pt.pipe_tile_copy(src, stages=4, grid=1, flags=GROUPS | pt.PIPE_FLAG_TEST_NO_RELEASE,
                      spin_limit=20000, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & pt.PIPE_STATUS_TIMEOUT_PRODUCER


@pytest.mark.parametrize("S,extra", [(4, 0), (8, 0), (8, pt.PIPE_FLAG_SPLIT_INTERLEAVE)])
def test_grouped_copy_full_size_bit_exact(S, extra):
    """fp16 16384 x 16384 uniform[-1,1): 64 strips of 4 tile columns, 4 segments each."""
    src = synth.uniform((16384, 16384), torch.float16, seed=42, device=DEV)
    st = _status()
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 16384, 16384, stages=S, flags=GROUPS | extra)
    assert (q["items"], q["grid"], q["tiles_per_item"], q["split"]) == (256, 256, 128, 4)
    dst = pt.pipe_tile_copy(src, stages=S, flags=GROUPS | extra | pt.PIPE_FLAG_NONTEMPORAL |
                            pt.PIPE_FLAG_XCD_REMAP | pt.PIPE_FLAG_LAZY_COMMIT, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))
    rows = torch.tensor([0, 1, 127, 128, 8191, 16383], device=DEV)
    assert np.array_equal(_bits(dst[rows]), R.tile_copy(src[rows].cpu().numpy()).view(np.uint16))
