"""GPU parity of the register producer engine (PIPE_FLAG_PRODUCER_VGPR):
producers load tiles into registers and write the swizzled slot with
ds_write_b128; every result must equal the oracle's, as with the
direct-to-LDS engine."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import protocol as P
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
V = pt.PIPE_FLAG_PRODUCER_VGPR
SHAPES = [(S, C, PW) for S in (1, 2, 3, 4) for C in (3, 4) for PW in (1, 4)]


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("S,C,PW", SHAPES)
def test_copy_register_engine_bit_exact(S, C, PW):
    src = synth.unique_codes(1280, 1024).to(DEV)   # 10 x 16 tiles, 3 segments, 7 workgroups
    st = _status()
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=S, consumer_waves=C,
                                 producer_waves=PW, split=3, grid=7,
                                 flags=V | pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_XCD_REMAP,
                                 status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


@pytest.mark.parametrize("shape", [(300, 200), (1000, 1000), (129, 8), (1, 72)])
@pytest.mark.parametrize("row_strips", [False, True])
def test_copy_register_engine_ragged(shape, row_strips):
    src = synth.unique_codes(*shape).to(DEV)
    st = _status()
    flags = V | (pt.PIPE_FLAG_ROW_STRIPS if row_strips else 0)
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=3, split=2, grid=3, flags=flags,
                                 status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


def test_copy_register_engine_trace_cursors():
    """One workgroup, 1 producer + 3 consumer waves, 8 tiles through 3 slots."""
    src = synth.uniform((128, 512), torch.float16, seed=42).to(DEV)
    trace = torch.zeros(16 * pt.PIPE_TRACE_WORDS, dtype=torch.int32, device=DEV)
    st = _status()
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=3, producer_waves=1,
                                 consumer_waves=3, grid=1, flags=V | pt.PIPE_FLAG_TRACE,
                                 trace=trace, trace_capacity=16, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    s_np = src.cpu().numpy()
    assert np.array_equal(_bits(dst), R.tile_copy(s_np).view(np.uint16))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(s_np))
    tr = trace.cpu().numpy().view(np.uint32).reshape(16, pt.PIPE_TRACE_WORDS)
    prod, cons = tr[0::2], tr[1::2]
    clock = lambda rec: (int(rec[7]) << 32) | int(rec[6])
    for t in range(8):
        assert tuple(prod[t][:2]) == (0, t) and tuple(cons[t][:2]) == (1, t)
        assert tuple(prod[t][2:4]) == P.cursor_after(3, t, 1)
        assert tuple(cons[t][2:4]) == P.cursor_after(3, t, 0)
        assert clock(cons[t]) >= clock(prod[t])
        if t + 3 < 8:
            assert clock(prod[t + 3]) >= clock(cons[t])


@pytest.mark.parametrize("S,C,PW", SHAPES)
def test_rowsum_register_engine_bit_exact(S, C, PW):
    A = synth.small_int((1024, 4096), -8, 8, torch.float16, seed=21).to(DEV)
    st = _status()
    out = pt.pipe_rowsum(A, stages=S, consumer_waves=C, producer_waves=PW, split=3, grid=5,
                         flags=V | pt.PIPE_FLAG_NONTEMPORAL, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


@pytest.mark.parametrize("shape", [(1000, 3000), (129, 72), (5, 8)])
def test_rowsum_register_engine_ragged(shape):
    A = synth.small_int(shape, -8, 8, torch.float16, seed=22).to(DEV)
    st = _status()
    out = pt.pipe_rowsum(A, stages=2, split=4, flags=V, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


def test_register_engine_missing_release_times_out():
    src = synth.unique_codes(512, 512).to(DEV)
    st = _status()
    pt.pipe_tile_copy(src, stages=2, grid=1, flags=V | pt.PIPE_FLAG_TEST_NO_RELEASE,
                      spin_limit=20000, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & pt.PIPE_STATUS_TIMEOUT_PRODUCER


def test_register_engine_full_size():
    """fp16 16384 x 16384 copy (bit-exact) and 8192 x 65536 N(0,1) row sum
    (within 1e-3 of the exact sums) on the default rings."""
    src = synth.uniform((16384, 16384), torch.float16, seed=42, device=DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, flags=V | pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_XCD_REMAP,
                            status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))
    del src, dst
    A = synth.normal((8192, 65536), torch.float16, seed=42, device=DEV)
    out = pt.pipe_rowsum(A, flags=V | pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_XCD_REMAP,
                         status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rows = np.array([0, 1, 127, 128, 4095, 8191])
    ref = R.rowsum_exact(A[torch.from_numpy(rows).to(DEV)].cpu().numpy())
    got = out.cpu().numpy()[rows]
    full_ref_rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    assert np.all(np.abs(got - ref) <= 1e-3 * np.maximum(np.abs(ref), full_ref_rms))
    del A
    torch.cuda.empty_cache()
