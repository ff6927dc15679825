"""Run-time protocol checks (PIPE_FLAG_DEBUG_CHECKS) and jittered stress runs.

The debug kernels check, at every wait, that the barrier word holds exactly the
completed phases the full/empty protocol allows and that the cursor has its
closed form, and that nothing is committed into a slot while a consumer reads
it. A clean protocol must never trip them, also when every wave pauses a
pseudo-random time before each wait (PIPE_FLAG_TEST_JITTER); the early release
that "cuda-features-10-pipelines" 4.10.3 warns against must trip them.
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
D = pt.PIPE_FLAG_DEBUG_CHECKS
J = pt.PIPE_FLAG_TEST_JITTER
POLICY = {"eager": 0, "lazy": pt.PIPE_FLAG_LAZY_COMMIT, "newest": pt.PIPE_FLAG_EAGER_NEWEST}
RINGS = [(S, C, PW) for S in (1, 2, 3, 4) for (C, PW) in ((3, 1), (4, 4))]


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("S,C,PW", RINGS)
@pytest.mark.parametrize("policy", ["eager", "lazy", "newest"])
@pytest.mark.parametrize("jitter", [False, True])
def test_copy_checks_hold(S, C, PW, policy, jitter):
    src = synth.unique_codes(1024, 1280).to(DEV)   # 8 x 20 tiles, 3 segments, 7 workgroups
    st = _status()
    flags = D | POLICY[policy] | (J if jitter else 0)
    dst, chk = pt.pipe_tile_copy(src, checksums=True, stages=S, consumer_waves=C,
                                 producer_waves=PW, split=3, grid=7, flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))
    assert np.array_equal(chk.cpu().numpy().view(np.uint32), R.tile_checksums(src.cpu().numpy()))


@pytest.mark.parametrize("S,C,PW", RINGS)
@pytest.mark.parametrize("jitter", [False, True])
def test_rowsum_checks_hold(S, C, PW, jitter):
    A = synth.small_int((1000, 3000), -8, 8, torch.float16, seed=31).to(DEV)  # ragged edges
    st = _status()
    out = pt.pipe_rowsum(A, stages=S, consumer_waves=C, producer_waves=PW, split=3, grid=5,
                         flags=D | (J if jitter else 0), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))


@pytest.mark.parametrize("shape", [(300, 200), (129, 8), (640, 4104)])
@pytest.mark.parametrize("row_strips", [False, True])
def test_ragged_copy_checks_hold_under_jitter(shape, row_strips):
    src = synth.unique_codes(*shape).to(DEV)
    st = _status()
    flags = D | J | (pt.PIPE_FLAG_ROW_STRIPS if row_strips else 0)
    dst = pt.pipe_tile_copy(src, stages=2, split=2, grid=3, flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), _bits(src))


def test_three_stage_ring_trace_under_checks():
    """The pages' one-workgroup ring (1 producer + 3 consumer waves, 8 tiles,
    S = 3) under the checks and jitter: the cursors still follow the closed form."""
    src = synth.uniform((128, 512), torch.float16, seed=42).to(DEV)
    trace = torch.zeros(16 * pt.PIPE_TRACE_WORDS, dtype=torch.int32, device=DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=3, producer_waves=1, consumer_waves=3, grid=1,
                            flags=D | J | pt.PIPE_FLAG_TRACE, trace=trace, trace_capacity=16,
                            status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(_bits(dst), R.tile_copy(src.cpu().numpy()).view(np.uint16))
    tr = trace.cpu().numpy().view(np.uint32).reshape(16, pt.PIPE_TRACE_WORDS)
    for t in range(8):
        assert tuple(tr[2 * t][2:4]) == P.cursor_after(3, t, 1)
        assert tuple(tr[2 * t + 1][2:4]) == P.cursor_after(3, t, 0)


@pytest.mark.parametrize("S,C,PW", [(1, 3, 1), (2, 4, 4)])
def test_early_release_is_reported(S, C, PW):
    """Consumers that release a slot before reading it let the producer refill
    it under them: the read-window check reports it (and the kernel ends)."""
    src = synth.unique_codes(1024, 256).to(DEV)
    st = _status()
    pt.pipe_tile_copy(src, stages=S, consumer_waves=C, producer_waves=PW, grid=2,
                      flags=D | pt.PIPE_FLAG_TEST_EARLY_RELEASE, status=st)
    torch.cuda.synchronize()
    status = int(st.item())
    assert status & pt.PIPE_STATUS_INVARIANT
    assert not status & (pt.PIPE_STATUS_TIMEOUT_PRODUCER | pt.PIPE_STATUS_TIMEOUT_CONSUMER)
    assert pt.pipe_status_from_word(status) == pt.PIPE_ERR_INVARIANT


def test_full_size_copy_under_checks():
    src = synth.uniform((16384, 16384), torch.float16, seed=42, device=DEV)
    st = _status()
    dst = pt.pipe_tile_copy(src, stages=2, flags=D | pt.PIPE_FLAG_NONTEMPORAL |
                            pt.PIPE_FLAG_XCD_REMAP | pt.PIPE_FLAG_LAZY_COMMIT, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))
    del src, dst
    torch.cuda.empty_cache()
