"""pipe_rowsum_noalloc (the row sum with the library's own workspace buffer)
against pipe_rowsum on the same inputs: the same kernels, so bit-identical
outputs; on small-integer data both equal the exact row sums of the oracle.
Two calls in a row, the second on a smaller matrix, so the second finds the
first's contents in the shared buffer."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import results as R

DEV = "cuda:0"


def _both(A, **cfg):
    M = A.shape[0]
    ref = torch.full((M,), float("nan"), device=DEV)
    got = torch.full((M,), float("nan"), device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    pt.pipe_rowsum(A, out=ref, status=st, **cfg)
    pt.pipe_rowsum_noalloc(A, got, status=st, **cfg)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", [{}, {"split": 8}, {"stages": 4, "split": 2},
                                 {"flags": pt.PIPE_FLAG_UNIFIED | pt.PIPE_FLAG_NONTEMPORAL,
                                  "stages": 2, "consumer_waves": 2}])
def test_noalloc_rowsum_equals_rowsum_two_calls(cfg):
    print(f"[no_alloc] cfg={cfg}", flush=True)
    # first call: 8192 x 16384 normal data (workspace of split x 8192 partials)
    A1 = synth.normal((8192, 16384), torch.float16, seed=11).to(DEV)
    ref1, got1 = _both(A1, **cfg)
    assert np.array_equal(ref1.view(np.uint32), got1.view(np.uint32))
    # second call, smaller: small integers, so both must equal the exact sums
    M2, N2 = (1024, 4096) if cfg.get("flags", 0) & pt.PIPE_FLAG_UNIFIED else (1000, 3000)
    A2 = synth.small_int((M2, N2), -8, 8, torch.float16, seed=12).to(DEV)
    ref2, got2 = _both(A2, **cfg)
    assert np.array_equal(ref2.view(np.uint32), got2.view(np.uint32))
    assert np.array_equal(got2, R.rowsum_exact(A2.cpu().numpy()))


@pytest.mark.gpu
def test_noalloc_rowsum_full_size_and_rejects_oversized():
    print("[no_alloc] 8192 x 65536 default config", flush=True)
    A = synth.small_int((8192, 65536), -8, 8, torch.float16, seed=13).to(DEV)
    ref, got = _both(A)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    assert np.array_equal(got, R.rowsum_exact(A.cpu().numpy()))
    # split 8 over 65536 rows needs 2 MiB of partials: more than the buffer
    big = torch.empty((65536, 4096), dtype=torch.float16, device=DEV)
    out = torch.empty(65536, device=DEV)
    with pytest.raises(pt.PipeError) as e:
        pt.pipe_rowsum_noalloc(big, out, split=8)
    assert e.value.status == pt.PIPE_ERR_WORKSPACE


@pytest.mark.gpu
def test_noalloc_rowsum_captured_and_replayed():
    """The allocation-free row sum inside a captured HIP graph: the first call
    on the device runs eagerly (it looks up the buffer's address), then the
    capture, then four replays on fresh inputs with eager row sums between
    them, every replay checked against the oracle."""
    print("[no_alloc] graph capture and replay", flush=True)
    M, N = 1000, 3000                       # ragged edges, split 4 tickets
    A = torch.empty((M, N), dtype=torch.float16, device=DEV)
    out = torch.empty(M, dtype=torch.float32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    A.copy_(synth.small_int((M, N), -8, 8, torch.float16, seed=30).to(DEV))
    pt.pipe_rowsum_noalloc(A, out, status=st)   # eager first call on this device
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pt.pipe_rowsum_noalloc(A, out, status=st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    other = synth.small_int((512, 8192), -8, 8, torch.float16, seed=31).to(DEV)
    other_out = torch.empty(512, device=DEV)
    for rep, seed in enumerate((32, 33, 34, 35)):
        A.copy_(synth.small_int((M, N), -8, 8, torch.float16, seed=seed).to(DEV))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0, rep
        assert np.array_equal(out.cpu().numpy(), R.rowsum_exact(A.cpu().numpy())), rep
        # an eager call between replays leaves its own contents in the buffer
        pt.pipe_rowsum_noalloc(other, other_out, status=st, split=8)
        torch.cuda.synchronize()
        assert np.array_equal(other_out.cpu().numpy(), R.rowsum_exact(other.cpu().numpy())), rep
